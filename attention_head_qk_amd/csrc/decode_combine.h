// The cross-split combine of one (sequence b, query head) by D threads (one per output
// element), shared by the combine pass and the fused combine + prologue pass of a multi-step
// decode graph. For each (sequence, head): M = max_s m_s, L = sum_s l_s 2^(m_s - M),
// out = sum_s O_s 2^(m_s - M) / L -- the exact regrouping of the max-subtracted softmax
// (zhanghao0806.com "Qwen3系列1-理论基础&真实结构", D1-2) over a partition of the keys, so the
// result does not depend on the split size. A sequence of length 0 gets a zero output.
// sw (kMaxCombineSplits floats) and s_inv are the block's LDS; the block has D threads.
#pragma once

#include "device_common.h"

namespace gqa {

template <typename T, int D>
__device__ __forceinline__ void combine_one(const DecodeArgs& a, int head, int b, int d,
                                            float* sw, float& s_inv) {
  const int L = a.seq_lens[b];
  const int ns = (L + a.split - 1) / a.split;
  // generation-loop step: the step's lengths become the caller's (nothing else reads the
  // caller's array during the step, so the copy can be made at any point of this pass)
  if (a.lens_commit && head == 0 && d == 0) a.lens_commit[b] = L;
  const long base = ((long)b * a.H + head) * a.nsplit;
  T* out = reinterpret_cast<T*>(a.out) + ((long)b * a.H + head) * D + d;
  if (ns == 0) {
    if constexpr (sizeof(T) == 2) *out = (bf16_t)0;
    else *out = 0.f;
    return;
  }
  // the first wave turns the split maxima into weights 2^(m_s - M) and the total 1 / L
  if (d < 64) {
    float M = -INFINITY;
    for (int s = d; s < ns; s += 64) M = fmaxf(M, a.part_ml[2 * (base + s)]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, xor_shfl(M, m));
    float Ls = 0.f;
    for (int s = d; s < ns; s += 64) {
      const float w = __builtin_amdgcn_exp2f(a.part_ml[2 * (base + s)] - M);
      sw[s] = w;
      Ls = fmaf(a.part_ml[2 * (base + s) + 1], w, Ls);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) Ls += xor_shfl(Ls, m);
    if (d == 0) s_inv = 1.0f / Ls;
  }
  __syncthreads();
  const float* po = a.part_o + base * D + d;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  int s = 0;
  for (; s + 4 <= ns; s += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = fmaf(po[(long)(s + u) * D], sw[s + u], acc[u]);
  }
  for (; s < ns; ++s) acc[0] = fmaf(po[(long)s * D], sw[s], acc[0]);
  const float r = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * s_inv;
  if constexpr (sizeof(T) == 2) {
    *out = (bf16_t)(pack_bf16x2(r, 0.f) & 0xffffu);
  } else {
    *out = r;
  }
}

}  // namespace gqa
