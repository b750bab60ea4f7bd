// Launchers of the gfx950 kernels of libgqa (host side). Each returns the HIP error of its
// launch; none synchronises.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace gqa {

// QK prologue: RMSNorm + RoPE of Q and K (and the decode append of the new K/V row).
hipError_t launch_prologue(const PrologueArgs& a, int grid, int d, bool bf16, hipStream_t s);
// bf16 prefill on matrix cores; grid = B * G * n_blk column blocks.
hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, hipStream_t s);
int prefill_bf16_cols_per_block();
// fp32 prefill; grid = (ceil(T/64), H, B).
hipError_t launch_prefill_f32(const PrefillArgs& a, int d, hipStream_t s);
// decode split-KV pass, then the cross-split combine pass.
hipError_t launch_decode_split(const DecodeArgs& a, int d, bool bf16, hipStream_t s);
hipError_t launch_decode_combine(const DecodeArgs& a, int d, bool bf16, hipStream_t s);
// decode graph of several steps: step n's combine and step n + 1's prologue (with its K/V
// append) in one launch; the prologue's slots are the B sequences (pa.decode == 1)
hipError_t launch_decode_combine_prologue(const DecodeArgs& ca, const PrologueArgs& pa, int d,
                                          bool bf16, hipStream_t s);

}  // namespace gqa
