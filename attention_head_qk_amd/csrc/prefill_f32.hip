// fp32 causal GQA prefill (true fp32 products and sums; no matrix-core rounding).
//
// Same operation as the bf16 kernel -- zhanghao0806.com "Qwen3系列1-理论基础&真实结构",
// D1-4 softmax(QK^T/sqrt(d_k) + M)V, D1-5 causal mask, D1-2 max-subtracted softmax, D2-3
// shared K/V per group; ewbang.com "深入剖析Qwen3模型架构" 3.1.2 head i -> K/V head
// floor(i/h) -- for the fp32 dtype, which exists for small, exact checks. One wave per
// (sequence, head, 64 query rows): a lane owns one query row (q and its output accumulator
// in registers) and walks 64-key tiles of its group's K/V staged in LDS; every lane reads the
// same K/V row at a time, which LDS broadcasts. Per chunk of keys: the scores, their max, one
// rescale, then the weighted sum of V rows.
#include "device_common.h"
#include "kernels.h"

namespace gqa {

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int KT = 64;
  __shared__ __attribute__((aligned(16))) float ks[KT][D];
  __shared__ __attribute__((aligned(16))) float vs[KT][D];

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
  const int r0 = rb * KT;
  if (r0 >= Tb) return;
  const int g = head / a.h;
  const int row = r0 + lane;
  const bool rvalid = row < Tb;
  const int kv_end = a.causal ? (r0 + KT < Tb ? r0 + KT : Tb) : Tb;

  const float* qt = reinterpret_cast<const float*>(a.qt);
  const float* kt = reinterpret_cast<const float*>(a.kt);
  const float* vv = reinterpret_cast<const float*>(a.v);
  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = rvalid ? qt[((long)(seq0 + row) * a.H + head) * D + e] : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int lim = a.causal ? row : 0x7fffffff;

  for (int t0 = 0; t0 < kv_end; t0 += KT) {
    // lane j stages key t0 + j
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
    __syncthreads();

    // scores in sub-chunks of SUB keys keep the register footprint within budget at d=128
    constexpr int SUB = D == 128 ? 16 : 64;
#pragma unroll 1
    for (int j0 = 0; j0 < KT; j0 += SUB) {
      float s[SUB];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) acc = fmaf(q[e], ks[j0 + j][e], acc);
        const int kj = t0 + j0 + j;
        s[j] = (kj < kv_end && kj <= lim) ? acc * a.scale : -INFINITY;
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
      for (int j = 0; j < SUB; ++j) {
        // a key this row does not see adds nothing, not even 0 * v (a non-finite v would
        // turn that into NaN)
        if (s[j] == -INFINITY) continue;
        const float p = expf(s[j] - m);
        l += p;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] = fmaf(p, vs[j0 + j][e], o[e]);
      }
    }
    __syncthreads();
  }

  if (rvalid) {
    float* op = reinterpret_cast<float*>(a.out) + ((long)(seq0 + row) * a.H + head) * D;
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < D; e += 4) {
      f32x4_t w = {o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv};
      *reinterpret_cast<f32x4_t*>(op + e) = w;
    }
  }
}

template <int D>
static hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  const dim3 grid((a.T + 63) / 64, a.H, a.B);
  hipLaunchKernelGGL((prefill_f32_kernel<D>), grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& a, int d, hipStream_t s) {
  if (a.B <= 0 || a.T <= 0) return hipSuccess;
  return d == 128 ? launch_t<128>(a, s) : launch_t<64>(a, s);
}

}  // namespace gqa
