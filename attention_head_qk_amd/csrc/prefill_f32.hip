// fp32 causal GQA prefill (true fp32 products and sums; no matrix-core rounding).
//
// Same operation as the bf16 kernel -- zhanghao0806.com "Qwen3系列1-理论基础&真实结构",
// D1-4 softmax(QK^T/sqrt(d_k) + M)V, D1-5 causal mask, D1-2 max-subtracted softmax, D2-3
// shared K/V per group; ewbang.com "深入剖析Qwen3模型架构" 3.1.2 head i -> K/V head
// floor(i/h) -- for the fp32 dtype, which exists for small, exact checks.
//
// One wave per (sequence, head, 8 query rows). The 8 lanes of a row split its keys: lane r
// takes keys r, r + 8, r + 16, ... of every 64-key tile and keeps its own online-softmax state
// (max, sum, unnormalised output row in registers) over them; at the end the 8 states of a
// row merge by the exact regrouping of the max-subtracted softmax (M = max m_r,
// O = sum_r e^(m_r - M) O_r / sum_r e^(m_r - M) l_r), in butterfly shuffles. K and V tiles sit
// in LDS with rows padded by 4 floats, so the 8 key rows a wave reads at once fall in
// different banks. A key a row does not see adds nothing (not even 0 * v).
#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {
constexpr int KT = 64;   // keys per tile
constexpr int RPW = 8;   // query rows per wave
constexpr int LPR = 8;   // lanes per row (key interleave)
}  // namespace

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int DP = D + 4;  // padded LDS row
  __shared__ __attribute__((aligned(16))) float ks[KT][DP];
  __shared__ __attribute__((aligned(16))) float vs[KT][DP];

  const int lane = threadIdx.x;
  const int rb = blockIdx.x;
  const int head = blockIdx.y;
  const int b = blockIdx.z;
  int seq0, Tb;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    Tb = a.cu_seqlens[b + 1] - seq0;
  } else {
    seq0 = b * a.T;
    Tb = a.T;
  }
  const int r0 = rb * RPW;
  if (r0 >= Tb) return;
  const int g = head / a.h;
  const int rl = lane / LPR;   // row inside the wave
  const int kr = lane % LPR;   // this lane's key residue
  const int row = r0 + rl;
  const bool rvalid = row < Tb;
  const int last_row = (r0 + RPW < Tb ? r0 + RPW : Tb) - 1;
  const int kv_end = a.causal ? last_row + 1 : Tb;
  const int lim = a.causal ? row : 0x7fffffff;  // highest key this row sees

  const float* qt = reinterpret_cast<const float*>(a.qt);
  const float* kt = reinterpret_cast<const float*>(a.kt);
  const float* vv = reinterpret_cast<const float*>(a.v);
  float q[D], o[D];
  {
    const float* qp = qt + ((long)(seq0 + (rvalid ? row : r0)) * a.H + head) * D;
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      const f32x4_t w = *reinterpret_cast<const f32x4_t*>(qp + e);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        q[e + i] = w[i];
        o[e + i] = 0.f;
      }
    }
  }
  float m = -INFINITY, l = 0.f;

  for (int t0 = 0; t0 < kv_end; t0 += KT) {
    // lane j stages key t0 + j (zeros past the end; never used)
    {
      const int key = t0 + lane;
      const long src = ((long)(seq0 + key) * a.G + g) * D;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        f32x4_t kw = {0.f, 0.f, 0.f, 0.f}, vw = {0.f, 0.f, 0.f, 0.f};
        if (key < kv_end) {
          kw = *reinterpret_cast<const f32x4_t*>(kt + src + e);
          vw = *reinterpret_cast<const f32x4_t*>(vv + src + e);
        }
        *reinterpret_cast<f32x4_t*>(&ks[lane][e]) = kw;
        *reinterpret_cast<f32x4_t*>(&vs[lane][e]) = vw;
      }
    }
    __syncthreads();

    // this lane's KT / LPR keys of the tile: scores, their max, one rescale, then the sums
    constexpr int NK = KT / LPR;
    float s[NK];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int kk = j * LPR + kr;
      const int key = t0 + kk;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        const f32x4_t kw = *reinterpret_cast<const f32x4_t*>(&ks[kk][e]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(q[e + i], kw[i], acc);
      }
      s[j] = (key < kv_end && key <= lim) ? acc * a.scale : -INFINITY;
      tmax = fmaxf(tmax, s[j]);
    }
    const float m_new = fmaxf(m, tmax);
    if (m_new > m) {
      const float alpha = expf(m - m_new);
      l *= alpha;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] *= alpha;
      m = m_new;
    }
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      // a key this row does not see adds nothing, not even 0 * v (a non-finite v would
      // turn that into NaN)
      if (s[j] == -INFINITY) continue;
      const float p = expf(s[j] - m);
      l += p;
      const int kk = j * LPR + kr;
#pragma unroll
      for (int e = 0; e < D; e += 4) {
        const f32x4_t vw = *reinterpret_cast<const f32x4_t*>(&vs[kk][e]);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[e + i] = fmaf(p, vw[i], o[e + i]);
      }
    }
    __syncthreads();
  }

  // merge the LPR states of each row (lanes rl * LPR + 0 .. LPR - 1)
  float M = m;
#pragma unroll
  for (int x = 1; x < LPR; x <<= 1) M = fmaxf(M, xor_shfl(M, x));
  const float w = (m == -INFINITY) ? 0.f : expf(m - M);  // a lane that saw no key adds 0
  float L = l * w;
#pragma unroll
  for (int x = 1; x < LPR; x <<= 1) L += xor_shfl(L, x);
#pragma unroll
  for (int e = 0; e < D; ++e) {
    float v = o[e] * w;
#pragma unroll
    for (int x = 1; x < LPR; x <<= 1) v += xor_shfl(v, x);
    o[e] = v;
  }
  if (rvalid) {
    // lane kr of the row stores elements [kr * D / LPR, (kr + 1) * D / LPR)
    float* op = reinterpret_cast<float*>(a.out) + ((long)(seq0 + row) * a.H + head) * D;
    const float inv = 1.0f / L;
    constexpr int PER = D / LPR;
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      if (e / PER == kr) {
        f32x4_t wv = {o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
        *reinterpret_cast<f32x4_t*>(op + e) = wv;
      }
    }
  }
}

template <int D>
static hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  const dim3 grid((a.T + RPW - 1) / RPW, a.H, a.B);
  hipLaunchKernelGGL((prefill_f32_kernel<D>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& a, int d, hipStream_t s) {
  if (a.B <= 0 || a.T <= 0) return hipSuccess;
  return d == 128 ? launch_t<128>(a, s) : launch_t<64>(a, s);
}

}  // namespace gqa
