// Device-side helpers shared by the gfx950 kernels of libgqa: vector types, bf16 packing,
// wave-level shuffles and the kernel argument blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// bf16 is carried as raw 16-bit patterns in memory.
typedef uint16_t bf16_t;

constexpr int kMaxHalfD = 64;  // d <= 128

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two fp32 values to one packed bf16 pair (low half = a), round to nearest even
// (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  bf16x2_t r = __builtin_convertvector(v, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Unpack 8 bf16 (one 16-byte chunk) to fp32.
__device__ __forceinline__ void unpack8(const u32x4_t w, float x[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = lo_bf16(w[i]);
    x[2 * i + 1] = hi_bf16(w[i]);
  }
}

__device__ __forceinline__ u32x4_t pack8(const float x[8]) {
  u32x4_t w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
  return w;
}

// Element loads/stores of 8 consecutive values in either storage type.
__device__ __forceinline__ void load8(const float* p, float x[8]) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
__device__ __forceinline__ void load8(const bf16_t* p, float x[8]) {
  unpack8(*reinterpret_cast<const u32x4_t*>(p), x);
}
__device__ __forceinline__ void store8(float* p, const float x[8]) {
  f32x4_t a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = x[i];
    b[i] = x[4 + i];
  }
  *reinterpret_cast<f32x4_t*>(p) = a;
  *reinterpret_cast<f32x4_t*>(p + 4) = b;
}
__device__ __forceinline__ void store8(bf16_t* p, const float x[8]) {
  *reinterpret_cast<u32x4_t*>(p) = pack8(x);
}

__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }

constexpr int BUF_RSRC_DW3 = 0x00020000;  // buffer descriptor word 3 for gfx9-class parts

// Buffer descriptor over [base, base + nbytes): loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes, BUF_RSRC_DW3);
}

// Wait for every outstanding vector-memory load of this wave, including LDS DMA
// (s_waitcnt vmcnt(0); gfx9 encoding: expcnt and lgkmcnt fields left at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// 16 bytes per lane from a buffer straight into LDS: lane i lands at lds + 16 i (the LDS
// address is taken from the first lane, so it must be the same for the whole wave).
// (A plain address-space cast keeps the pointer's provenance, so alias analysis can tell
// which LDS array a DMA writes.)
// POL is the instruction's cache-policy operand (0, or kNonTemporal).
constexpr int kNonTemporal = 2;  // the "nt" bit: streamed data, not kept in the caches
template <int POL = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, const char* lds, int voff, int soff) {
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)const_cast<char*>(lds), 16, voff, soff, 0, POL);
}

// cos and sin of the RoPE angle phi = pos * omega_j: the angle is reduced to revolutions in
// fp64 (exact to ~1e-12 rad at pos 32767). bf16 outputs then take the hardware sin/cos of the
// fp32 revolution count (abs error ~1e-6, far below bf16 rounding), fp32 outputs an fp64
// sincos.
template <bool BF16>
__device__ __forceinline__ void rope_cos_sin(double phi, float& c, float& s) {
  const double rev = phi * 0.15915494309189533577;  // 1 / (2 pi)
  if constexpr (BF16) {
    const float r = (float)(rev - floor(rev));
    s = __builtin_amdgcn_sinf(r);  // sin(2 pi r)
    c = __builtin_amdgcn_cosf(r);
  } else {
    double sd, cd;
    sincos(phi - floor(rev) * 6.283185307179586476925286766559, &sd, &cd);
    s = (float)sd;
    c = (float)cd;
  }
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = 1; m < W; m <<= 1) v += xor_shfl(v, m);
  return v;
}

// ---------------------------------------------------------------------------- kernel args
struct PrologueArgs {
  const void* q;      // rows to normalise and rotate with gamma_q   [rows, H, D]
  const void* k;      // rows to normalise and rotate with gamma_k   [rows, G, D] or null
  const void* v;      // decode only: V rows copied into the cache    [B, G, D] or null
  void* q_out;        // [rows, H, D]
  void* k_out;        // prefill: [N, G, D]; decode: K cache [B, max_seq, G, D]
  void* v_out;        // decode: V cache
  const int32_t* positions;
  const int32_t* cu_seqlens;  // prefill, packed
  const int32_t* seq_lens;    // decode: tokens per sequence; cached prefill: cached rows
  const void* gq;
  const void* gk;
  float eps;
  int decode;         // 0: token rows (prefill / stand-alone), 1: one row per sequence,
                      // 2: token rows appended to a cache after seq_lens[b] earlier rows
  int B, T, H, G;
  int max_seq;
  int use_rope;
  int slot0;          // first token slot of this launch (set by the launcher)
  int32_t* lens_out;  // decode, generation-loop step: non-null = the sequence gains its new
                      // token here (length min(seq_lens[b] + 1, max_seq)), and that length is
                      // written to lens_out[b] for the rest of the step
  int32_t* zero;      // prefill: zero_n counters the attention kernel that follows claims
  int zero_n;         // its blocks from (zeroed by the first workgroup), or null
  double omega[kMaxHalfD];  // theta^(-2j/d), computed on the host in fp64
};

struct PrefillArgs {
  const void* qt;     // fp32 kernel: [N, H, D] normalised, rotated Q
  const void* q;      // bf16 kernel: [N, H, D] raw Q, normalised and rotated in the kernel
  const int32_t* positions;  // bf16 kernel: RoPE positions [N] or null (index in sequence)
  const void* gq;     // bf16 kernel: gamma_q [D] or null (no norm)
  float eps;
  int use_rope;
  const void* kt;     // [N, G, D] normalised, rotated K
  const void* v;      // [N, G, D]
  void* out;          // [N, H, D]
  const int32_t* cu_seqlens;  // null: dense, sequence b = tokens [b*T, (b+1)*T)
  int B, T, H, G, h;
  int causal;
  int n_blk;          // column blocks of the longest sequence
  int zigzag;         // 1: pair heavy and light blocks (see the prefill kernel)
  int rank_chunk;     // bf16 kernel: consecutive ranks of one sequence before the next one
  int32_t* claim;     // bf16 kernel: [G] zeroed counters; non-null = a workgroup takes its
                      // rank inside its group from claim[g] instead of from its block id
  float* pair_part;   // bf16 kernel, paired schedule of a one-round grid (non-null): per pair
                      // two partial softmax states of COLS columns (O [COLS][D], then (m, l)
                      // per column), and a zeroed arrival counter per pair
  int32_t* pair_arrive;
  const int32_t* cache_lens;  // bf16 kernel, cached prefill: earlier tokens per sequence in
                              // the cache; kt / v are then caches [B, max_seq, G, D]
  int max_seq;
  int window;         // bf16 kernel: > 0 keeps only keys with index > query index - window
  const uint32_t* block_mask;  // bf16 kernel: [query block][bm_words] bit rows over 64-key
                               // blocks (bit j of word w = key block 32 w + j), or null
  int bm_words;
  float scale;        // score scale (1/sqrt(d) by default)
  float scale_log2e;  // scale * log2(e)
  double omega[kMaxHalfD];  // bf16 kernel: theta^(-2j/d), computed on the host in fp64
};

struct DecodeArgs {
  const void* qt;     // [B, H, D] normalised, rotated query
  const void* k_cache;
  const void* v_cache;  // [B, max_seq, G, D]
  const int32_t* seq_lens;
  float* part_o;      // [B, H, nsplit, D]
  float* part_ml;     // [B, H, nsplit, 2]  (running max in log2 units, sum)
  void* out;          // [B, H, D]
  int B, H, G, h, max_seq, nsplit;
  int split;          // keys per split, a multiple of 128 (4 waves x 32 keys)
  int stream_v;       // 1: V rows are read non-temporally (caches larger than the chip's caches)
  float scale_log2e;
  int32_t* lens_commit;  // generation-loop step: the combine pass copies seq_lens[b] (the
                         // step's own lengths) here at the end; null otherwise
};

constexpr int kDecodeSplit = 1024;       // longest split of the decode pass (keys)
constexpr int kDecodeSplitMin = 256;     // shortest split the host picks
constexpr int kMaxCombineSplits = 4096;  // splits per sequence the combine pass can merge

}  // namespace gqa
