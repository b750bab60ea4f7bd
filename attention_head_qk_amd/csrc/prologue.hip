// QK prologue for gfx950: per-head RMSNorm then RoPE, fused in one pass over Q and K.
//
// RMSNorm: zhanghao0806.com "Qwen3系列1-理论基础&真实结构", D2-1 (gamma * x / sqrt(mean x^2
// + eps)); applied per head to Q (gamma_q) and K (gamma_k), then RoPE, V untouched: same page
// D2-2 and the nano-vllm "Qwen3" page, attention forward steps (4) and (5). RoPE turns each
// adjacent pair (2j, 2j+1) counter-clockwise by pos * omega_j (D2-2 matrix R(pos); ewbang.com
// "深入剖析Qwen3模型架构" 3.1.2 and 3.4.1 for the pairing and omega_j = theta^(-2j/d)).
//
// HBM-bound: it reads and writes (H + G) * d elements per token. Every lane owns one 16-byte
// chunk (4 rotation pairs) of one head row of one token, so the whole tensor is in flight at
// once; d/8 lanes cover a row with one coalesced read, the sum of squares is reduced across
// them with DPP row permutes, and each lane evaluates its own four angles (cheap next to the
// row's HBM traffic; rope_cos_sin gives the precision). With q null (the bf16 prefill, whose
// attention kernel prepares Q itself) only K rows are processed.
#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {

template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  const int x = __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true);
  return v + __int_as_float(x);
}

// Sum over aligned groups of W lanes (W = 8 or 16) inside a DPP row.
template <int W>
__device__ __forceinline__ float lane_group_sum(float v) {
  v = dpp_add<0xB1>(v);   // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v);   // quad_perm [2,3,0,1]
  v = dpp_add<0x141>(v);  // row_half_mirror
  if (W == 16) v = dpp_add<0x140>(v);  // row_mirror
  return v;
}

}  // namespace

template <typename T, int D>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(PrologueArgs a) {
  constexpr int LPR = D / 8;  // lanes per head row (8 elements = one 16-byte bf16 chunk each)
  const int nq = a.q ? a.H : 0, nk = a.k ? a.G : 0;
  const int rows_per_token = nq + nk + ((a.decode && a.v) ? a.G : 0);
  const long item = (long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;  // (token slot, row)
  const int ch = threadIdx.x % LPR;
  const int e0 = ch * 8;
  const int slot = (int)(item / rows_per_token);
  const int r = (int)(item % rows_per_token);

  // ---- the token this row belongs to, its RoPE position, and the row's source/destination
  bool active;
  long tok = 0;        // token index of the source rows
  long k_tok_out = 0;  // destination token row for K / V
  int pos = 0;
  if (a.decode != 1) {
    const int b = slot / a.T, t = slot % a.T;
    active = b < a.B;
    if (active && a.cu_seqlens) {
      const int s0 = a.cu_seqlens[b];
      active = t < a.cu_seqlens[b + 1] - s0;
      tok = s0 + t;
    } else {
      tok = slot;
    }
    if (active) pos = a.positions ? a.positions[tok] : t;
    k_tok_out = tok;
    if (a.decode == 2 && active) {
      // cached prefill: the token follows the sequence's cached rows; its K/V go to slot
      // past + t of the cache (rows that would not fit are not written)
      const int past = max(0, min(a.seq_lens[b], a.max_seq));
      if (!a.positions) pos = past + t;
      k_tok_out = (long)b * a.max_seq + past + t;
      if (r >= nq && past + t >= a.max_seq) active = false;
    }
  } else {
    active = slot < a.B;
    const int L = active ? a.seq_lens[slot] : 0;
    if (active) pos = a.positions ? a.positions[slot] : (L > 0 ? L - 1 : 0);
    tok = slot;
    k_tok_out = (long)slot * a.max_seq + (L > 0 ? L - 1 : 0);
    if (r >= a.H && L == 0) active = false;  // nothing to append to an empty sequence
  }
  const bool is_q = r < nq, is_k = !is_q && r < nq + nk;
  const T* src;
  T* dst;
  if (is_q) {
    src = reinterpret_cast<const T*>(a.q) + (tok * a.H + r) * (long)D;
    dst = reinterpret_cast<T*>(a.q_out) + (tok * a.H + r) * (long)D;
  } else if (is_k) {
    src = reinterpret_cast<const T*>(a.k) + (tok * a.G + (r - nq)) * (long)D;
    dst = reinterpret_cast<T*>(a.k_out) + (k_tok_out * a.G + (r - nq)) * (long)D;
  } else {
    src = reinterpret_cast<const T*>(a.v) + (tok * a.G + (r - nq - nk)) * (long)D;
    dst = reinterpret_cast<T*>(a.v_out) + (k_tok_out * a.G + (r - nq - nk)) * (long)D;
  }

  float x[8];
  if (active) {
    load8(src + e0, x);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.f;
  }
  // all LPR lanes of a row share `active`, `is_q` and `is_k`, so the reduction below only
  // mixes lanes of one row
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
  ss = lane_group_sum<LPR>(ss);
  const void* gam = is_q ? a.gq : (is_k ? a.gk : nullptr);
  if (gam) {
    float gw[8];
    load8(reinterpret_cast<const T*>(gam) + e0, gw);
    const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (x[i] * rinv) * gw[i];
  }
  if ((is_q || is_k) && a.use_rope) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float c, sn;
      rope_cos_sin<sizeof(T) == 2>((double)pos * a.omega[4 * ch + m], c, sn);
      const float x0 = x[2 * m], x1 = x[2 * m + 1];
      x[2 * m] = x0 * c - x1 * sn;
      x[2 * m + 1] = x0 * sn + x1 * c;
    }
  }
  if (active) store8(dst + e0, x);
}

template <typename T, int D>
static hipError_t launch_prologue_t(const PrologueArgs& a, int slots, hipStream_t s) {
  constexpr int ROWS_PER_BLOCK = 256 / (D / 8);
  const long rows = (long)slots * ((a.q ? a.H : 0) + (a.k ? a.G : 0) + ((a.decode && a.v) ? a.G : 0));
  const long grid = (rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((qk_norm_rope_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prologue(const PrologueArgs& a, int slots, int d, bool bf16, hipStream_t s) {
  if (slots <= 0) return hipSuccess;
  if (bf16) return d == 128 ? launch_prologue_t<bf16_t, 128>(a, slots, s)
                            : launch_prologue_t<bf16_t, 64>(a, slots, s);
  return d == 128 ? launch_prologue_t<float, 128>(a, slots, s)
                  : launch_prologue_t<float, 64>(a, slots, s);
}

}  // namespace gqa
