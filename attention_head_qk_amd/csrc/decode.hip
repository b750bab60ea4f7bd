// Single-token GQA decode on gfx950: split-KV pass + cross-split combine.
//
// The new token's query (already normalised and rotated, its own K/V already in the cache:
// zhanghao0806.com "Qwen3系列1-理论基础&真实结构", D2-3, the layer writes K/V into the cache
// before attention) attends to every cached row of its sequence. Decode reads the whole
// cache once and does ~4 FLOP per byte, so it is bound by HBM bandwidth (same section: decode
// is memory-bound, prefill compute-bound).
//
// Split pass. A workgroup takes one split of kDecodeSplit keys of one sequence and one KV
// group (and a chunk of HC of the group's h query heads). The K/V cache is token-major
// [B, max_seq, G, d], so a key row of one group is d contiguous elements: d/8 lanes read it
// with 16-byte loads, a wave covers 64/(d/8) rows at once and each row-slot of lanes keeps
// its own online-softmax state over a batch of 8 keys at a time (8 K and 8 V loads in flight
// per lane before any arithmetic). Scores are reduced across the row's lanes with DPP row
// permutes (no LDS). At the end the row-slots' states (m, l, O) are merged through LDS and the
// split writes one (m, l, O) partial per head, with O unnormalised and m in log2 units.
//
// Combine pass. For each (sequence, head): M = max_s m_s, L = sum_s l_s 2^(m_s - M),
// out = sum_s O_s 2^(m_s - M) / L. This is the exact regrouping of the max-subtracted
// softmax (D1-2) over a partition of the keys, so the result does not depend on the split
// size. A sequence of length 0 gets a zero output.
#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int x = __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true);
  return v + __int_as_float(x);
}

// Sum over aligned 16-lane (or 8-lane) rows with DPP: xor 1, xor 2 (quad_perm), then the
// half-row mirror (lane i <-> 7-i) and the row mirror (lane i <-> 15-i).
template <int W>
__device__ __forceinline__ float row_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);  // row_half_mirror
  if (W == 16) v = dpp_add<0x140>(v);  // row_mirror
  return v;
}

template <typename T>
struct Row8;

template <>
struct Row8<bf16_t> {
  u32x4_t w;
  __device__ __forceinline__ void load(const bf16_t* p) { w = *reinterpret_cast<const u32x4_t*>(p); }
  __device__ __forceinline__ void zero() { w = u32x4_t{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ void to_f32(float x[8]) const { unpack8(w, x); }
};

template <>
struct Row8<float> {
  f32x4_t a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const f32x4_t*>(p);
    b = *reinterpret_cast<const f32x4_t*>(p + 4);
  }
  __device__ __forceinline__ void zero() { a = b = f32x4_t{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ void to_f32(float x[8]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
};

}  // namespace

template <typename T, int D, int HC>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int LPR = D / 8;         // lanes per key row
  constexpr int RPW = 64 / LPR;      // row-slots per wave
  constexpr int NR = 4 * RPW;        // row-slots per workgroup
  constexpr int NB = 8;              // keys per row-slot batch
  constexpr int KPI = NR * NB;       // keys per workgroup iteration
  __shared__ float sm_m[NR][HC];
  __shared__ float sm_l[NR][HC];
  __shared__ __attribute__((aligned(16))) float sm_o[NR][HC][D];

  const int s = blockIdx.x;
  const int b = blockIdx.z;
  const int nhc = a.h / HC;
  const int g = blockIdx.y / nhc;
  const int head0 = g * a.h + (blockIdx.y % nhc) * HC;
  const int L = a.seq_lens[b];
  const int k0 = s * kDecodeSplit;
  if (k0 >= L) return;
  const int k1 = (k0 + kDecodeSplit < L) ? k0 + kDecodeSplit : L;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int R = wave * RPW + lane / LPR;
  const int e0 = (lane % LPR) * 8;

  // the group's HC query rows, pre-scaled so that scores come out in log2 units
  const T* qt = reinterpret_cast<const T*>(a.qt);
  const float sl2e = a.scale_log2e;
  float q[HC][8];
#pragma unroll
  for (int i = 0; i < HC; ++i) {
    load8(qt + ((long)b * a.H + head0 + i) * D + e0, q[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) q[i][e] *= sl2e;
  }

  const long row_stride = (long)a.G * D;
  const T* kc = reinterpret_cast<const T*>(a.k_cache) + (long)b * a.max_seq * row_stride + (long)g * D + e0;
  const T* vc = reinterpret_cast<const T*>(a.v_cache) + (long)b * a.max_seq * row_stride + (long)g * D + e0;

  float m[HC], l[HC], o[HC][8];
#pragma unroll
  for (int i = 0; i < HC; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[i][e] = 0.f;
  }

  for (int it = k0; it < k1; it += KPI) {
    const int kb = it + R * NB;
    Row8<T> kr[NB], vr[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (kb + j < k1) {
        kr[j].load(kc + (long)(kb + j) * row_stride);
        vr[j].load(vc + (long)(kb + j) * row_stride);
      } else {
        kr[j].zero();
        vr[j].zero();
      }
    }
    float sc[HC][NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      float kf[8];
      kr[j].to_f32(kf);
#pragma unroll
      for (int i = 0; i < HC; ++i) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(q[i][e], kf[e], acc);
        const float x = row_sum<LPR>(acc);
        sc[i][j] = (kb + j < k1) ? x : -INFINITY;
      }
    }
    float vf[NB][8];
#pragma unroll
    for (int j = 0; j < NB; ++j) vr[j].to_f32(vf[j]);
#pragma unroll
    for (int i = 0; i < HC; ++i) {
      float bm = sc[i][0];
#pragma unroll
      for (int j = 1; j < NB; ++j) bm = fmaxf(bm, sc[i][j]);
      const float m_new = fmaxf(m[i], bm);
      if (m_new == -INFINITY) continue;  // nothing visible in this slot yet
      const float alpha = __builtin_amdgcn_exp2f(m[i] - m_new);
      l[i] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[i][e] *= alpha;
      m[i] = m_new;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float p = __builtin_amdgcn_exp2f(sc[i][j] - m_new);
        l[i] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[i][e] = fmaf(p, vf[j][e], o[i][e]);
      }
    }
  }

  // merge the NR row-slot states of this split
#pragma unroll
  for (int i = 0; i < HC; ++i) {
    if ((lane % LPR) == 0) {
      sm_m[R][i] = m[i];
      sm_l[R][i] = l[i];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) sm_o[R][i][e0 + e] = o[i][e];
  }
  __syncthreads();
  for (int idx = tid; idx < HC * D; idx += 256) {
    const int i = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < NR; ++r) M = fmaxf(M, sm_m[r][i]);
    float Ls = 0.f, Os = 0.f;
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const float w = __builtin_amdgcn_exp2f(sm_m[r][i] - M);  // empty slots: 2^-inf = 0
      Ls = fmaf(sm_l[r][i], w, Ls);
      Os = fmaf(sm_o[r][i][d], w, Os);
    }
    const long pidx = ((long)b * a.H + head0 + i) * a.nsplit + s;
    a.part_o[pidx * D + d] = Os;
    if (d == 0) {
      a.part_ml[2 * pidx] = M;
      a.part_ml[2 * pidx + 1] = Ls;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int L = a.seq_lens[b];
  const int ns = (L + kDecodeSplit - 1) / kDecodeSplit;
  const long base = ((long)b * a.H + head) * a.nsplit;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_ml[2 * (base + s)]);
  float Ls = 0.f, Os = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float w = __builtin_amdgcn_exp2f(a.part_ml[2 * (base + s)] - M);
    Ls = fmaf(a.part_ml[2 * (base + s) + 1], w, Ls);
    Os = fmaf(a.part_o[(base + s) * D + d], w, Os);
  }
  const float r = (ns > 0) ? Os / Ls : 0.f;
  T* out = reinterpret_cast<T*>(a.out) + ((long)b * a.H + head) * D + d;
  if constexpr (sizeof(T) == 2) {
    *out = (bf16_t)(pack_bf16x2(r, 0.f) & 0xffffu);
  } else {
    *out = r;
  }
}

template <typename T, int D, int HC>
static hipError_t launch_split(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.nsplit, a.G * (a.h / HC), a.B);
  hipLaunchKernelGGL((decode_split_kernel<T, D, HC>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t split_td(const DecodeArgs& a, hipStream_t s) {
  if (a.h % 4 == 0) return launch_split<T, D, 4>(a, s);
  if (a.h % 2 == 0) return launch_split<T, D, 2>(a, s);
  return launch_split<T, D, 1>(a, s);
}

template <typename T, int D>
static hipError_t combine_td(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.H, a.B), dim3(D), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeArgs& a, int d, bool bf16, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (bf16) return d == 128 ? split_td<bf16_t, 128>(a, s) : split_td<bf16_t, 64>(a, s);
  return d == 128 ? split_td<float, 128>(a, s) : split_td<float, 64>(a, s);
}

hipError_t launch_decode_combine(const DecodeArgs& a, int d, bool bf16, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (bf16) return d == 128 ? combine_td<bf16_t, 128>(a, s) : combine_td<bf16_t, 64>(a, s);
  return d == 128 ? combine_td<float, 128>(a, s) : combine_td<float, 64>(a, s);
}

}  // namespace gqa
