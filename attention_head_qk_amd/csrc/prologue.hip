// QK prologue for gfx950: per-head RMSNorm then RoPE, fused in one pass over Q and K.
//
// RMSNorm: zhanghao0806.com "Qwen3系列1-理论基础&真实结构", D2-1 (gamma * x / sqrt(mean x^2
// + eps)); applied per head to Q (gamma_q) and K (gamma_k), then RoPE, V untouched: same page
// D2-2 and the nano-vllm "Qwen3" page, attention forward steps (4) and (5). RoPE turns each
// adjacent pair (2j, 2j+1) counter-clockwise by pos * omega_j (D2-2 matrix R(pos); ewbang.com
// "深入剖析Qwen3模型架构" 3.1.2 and 3.4.1 for the pairing and omega_j = theta^(-2j/d)).
//
// One workgroup per token (prefill) or per sequence (decode). The angles of a token are the
// same for all its H + G heads, so one wave evaluates cos/sin of the d/2 angles once, in
// fp64 after an exact-ish fp64 range reduction, and parks them in LDS; then every wave
// streams head rows: 8 elements per lane (one 16-byte load for bf16), d/8 lanes per row,
// the sum of squares reduced across those lanes with shuffles. The kernel is HBM-bound
// (reads and writes (H+G)*d elements per token).
#include "device_common.h"
#include "kernels.h"

namespace gqa {

template <typename T, int D>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(PrologueArgs a) {
  constexpr int LPR = D / 8;        // lanes per head row
  constexpr int RPW = 64 / LPR;     // rows per wave pass
  constexpr int RPB = 4 * RPW;      // rows per workgroup pass
  __shared__ float cs[D / 2];
  __shared__ float sn[D / 2];

  const int tid = threadIdx.x;
  long row_in;    // index of the q row block [H, D] of this token / sequence
  long k_row_out; // destination row block of K (and V) in k_out / v_out; -1 = no K output
  int pos;
  if (!a.decode) {
    int b, t, Tb;
    if (a.cu_seqlens) {
      b = blockIdx.x / a.T;
      t = blockIdx.x % a.T;
      const int s0 = a.cu_seqlens[b];
      Tb = a.cu_seqlens[b + 1] - s0;
      if (t >= Tb) return;
      row_in = s0 + t;
    } else {
      b = blockIdx.x / a.T;
      t = blockIdx.x % a.T;
      row_in = blockIdx.x;
    }
    pos = a.positions ? a.positions[row_in] : t;
    k_row_out = a.k ? row_in : -1;
  } else {
    const int b = blockIdx.x;
    const int L = a.seq_lens[b];
    pos = a.positions ? a.positions[b] : (L > 0 ? L - 1 : 0);
    row_in = b;
    k_row_out = (a.k && L > 0) ? ((long)b * a.max_seq + (L - 1)) : -1;
  }

  if (a.use_rope) {
    if (tid < D / 2) {
      // fp64 angle, reduced to [-pi, pi] before the fp64 sincos.
      const double phi = (double)pos * a.omega[tid];
      const double two_pi = 6.283185307179586476925286766559;
      const double r = phi - rint(phi / two_pi) * two_pi;
      double s, c;
      sincos(r, &s, &c);
      cs[tid] = (float)c;
      sn[tid] = (float)s;
    }
    __syncthreads();
  }

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int sub = lane / LPR;       // row slot within the wave pass
  const int ch = lane % LPR;        // 8-element chunk of the row
  const int e0 = ch * 8;

  float gq[8], gk[8];
  const bool norm_q = a.gq != nullptr, norm_k = a.gk != nullptr;
  if (norm_q) load8(reinterpret_cast<const T*>(a.gq) + e0, gq);
  if (norm_k) load8(reinterpret_cast<const T*>(a.gk) + e0, gk);
  float c4[4], s4[4];
  if (a.use_rope) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      c4[m] = cs[ch * 4 + m];
      s4[m] = sn[ch * 4 + m];
    }
  }

  const int nq = a.H;
  const int nk = (k_row_out >= 0) ? a.G : 0;
  const int nv = (a.decode && a.v && k_row_out >= 0) ? a.G : 0;
  const int total = nq + nk + nv;
  const T* qin = reinterpret_cast<const T*>(a.q) + row_in * (long)a.H * D;
  T* qout = reinterpret_cast<T*>(a.q_out) + row_in * (long)a.H * D;

  for (int r0 = 0; r0 < total; r0 += RPB) {
    const int r = r0 + wave * RPW + sub;
    const bool active = r < total;
    float x[8];
    const T* src;
    T* dst;
    bool norm, rope_it;
    const float* gam;
    if (r < nq) {
      src = qin + (long)r * D;
      dst = qout + (long)r * D;
      norm = norm_q;
      gam = gq;
      rope_it = true;
    } else if (r < nq + nk) {
      const int g = r - nq;
      src = reinterpret_cast<const T*>(a.k) + (row_in * (long)a.G + g) * D;
      dst = reinterpret_cast<T*>(a.k_out) + (k_row_out * a.G + g) * D;
      norm = norm_k;
      gam = gk;
      rope_it = true;
    } else {
      const int g = r - nq - nk;
      src = reinterpret_cast<const T*>(a.v) + (row_in * (long)a.G + g) * D;
      dst = reinterpret_cast<T*>(a.v_out) + (k_row_out * a.G + g) * D;
      norm = false;
      gam = gq;
      rope_it = false;
    }
    if (active) {
      load8(src + e0, x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
    // Row type is uniform across the LPR lanes of a row, so the reduction below only mixes
    // lanes that agree on `norm`.
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
    ss = group_sum<LPR>(ss);
    if (norm) {
      const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (x[i] * rinv) * gam[i];
    }
    if (rope_it && a.use_rope) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float x0 = x[2 * m], x1 = x[2 * m + 1];
        x[2 * m] = x0 * c4[m] - x1 * s4[m];
        x[2 * m + 1] = x0 * s4[m] + x1 * c4[m];
      }
    }
    if (active) store8(dst + e0, x);
  }
}

template <typename T, int D>
static hipError_t launch_prologue_t(const PrologueArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((qk_norm_rope_kernel<T, D>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueArgs& a, int grid, int d, bool bf16, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (bf16) return d == 128 ? launch_prologue_t<bf16_t, 128>(a, grid, s)
                            : launch_prologue_t<bf16_t, 64>(a, grid, s);
  return d == 128 ? launch_prologue_t<float, 128>(a, grid, s)
                  : launch_prologue_t<float, 64>(a, grid, s);
}

}  // namespace gqa
