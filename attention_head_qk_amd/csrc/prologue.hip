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
#include <algorithm>

#include "decode_combine.h"
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

// The rows of one 256-thread block `blk` of the prologue grid; thread `tid` of it. (The fused
// combine + prologue pass of a multi-step decode graph runs these blocks as D-thread pieces:
// nothing here synchronises beyond a wave.)
template <typename T, int D>
__device__ __forceinline__ void prologue_block(const PrologueArgs& a, unsigned blk, unsigned tid) {
  constexpr int LPR = D / 8;  // lanes per head row (8 elements = one 16-byte bf16 chunk each)
  const int nq = a.q ? a.H : 0, nk = a.k ? a.G : 0;
  const int rows_per_token = nq + nk + ((a.decode && a.v) ? a.G : 0);
  // (token slot, row) of this lane's row; the launcher keeps slots * rows below 2^31
  const unsigned item = blk * (256u / LPR) + tid / LPR;
  const int ch = tid % LPR;
  const int e0 = ch * 8;
  const int slot = a.slot0 + (int)(item / (unsigned)rows_per_token);
  const int r = (int)(item % (unsigned)rows_per_token);
  const bool is_q = r < nq, is_k = !is_q && r < nq + nk;

  // ---- the token this row belongs to. Every load of the row (data, gamma, position, the
  // sequence's length, the four frequencies) is issued before the first wait: addresses of
  // lanes past the end point at a valid row and their values are discarded. Only packed
  // sequences need one load (cu_seqlens) before the row's address is known.
  bool active;
  int tok;         // token index of the source rows
  int b = 0, t = 0;
  if (a.decode != 1) {
    b = slot / a.T;
    t = slot - b * a.T;
    active = b < a.B;
    tok = active ? slot : 0;
    if (a.cu_seqlens) {
      const int bb = active ? b : 0;
      const int s0 = a.cu_seqlens[bb];
      active = active && t < a.cu_seqlens[bb + 1] - s0;
      tok = active ? s0 + t : 0;
    }
  } else {
    b = slot;
    active = slot < a.B;
    tok = active ? slot : 0;
  }
  // a packed batch launches max-length slots for every sequence: a wave whose slots all lie
  // past their sequence's end (or past the last sequence) has nothing to do
  if (!__any(active)) return;
  const int bb = active ? b : 0;
  const T* src;
  if (is_q) src = reinterpret_cast<const T*>(a.q) + ((long)tok * a.H + r) * D;
  else if (is_k) src = reinterpret_cast<const T*>(a.k) + ((long)tok * a.G + (r - nq)) * D;
  else src = reinterpret_cast<const T*>(a.v) + ((long)tok * a.G + (r - nq - nk)) * D;
  const void* gam = is_q ? a.gq : (is_k ? a.gk : nullptr);
  const T* gsrc = gam ? reinterpret_cast<const T*>(gam) : src;
  const int32_t* pp = a.positions ? a.positions + tok : reinterpret_cast<const int32_t*>(src);
  const int32_t* lp = (a.decode && a.seq_lens) ? a.seq_lens + bb : reinterpret_cast<const int32_t*>(src);
  float x[8], gw[8];
  load8(src + e0, x);
  load8(gsrc + e0, gw);
  const int pos_in = *pp;
  const int len_in = *lp;
  double om[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) om[m] = a.omega[4 * ch + m];

  // ---- the RoPE position and the destination row (K / V rows of decode and cached prefill
  // go to the cache)
  int pos;
  long k_tok_out;  // destination token row for K / V
  if (a.decode == 0) {
    pos = a.positions ? pos_in : t;
    k_tok_out = tok;
  } else if (a.decode == 2) {
    // cached prefill: the token follows the sequence's cached rows; its K/V go to slot
    // past + t of the cache (rows that would not fit are not written)
    const int past = max(0, min(len_in, a.max_seq));
    pos = a.positions ? pos_in : past + t;
    k_tok_out = (long)bb * a.max_seq + past + t;
    if (r >= nq && past + t >= a.max_seq) active = false;
  } else {
    // a generation-loop step first gives the sequence its new token (capped at max_seq);
    // one lane per sequence hands that length to the rest of the step
    const int L = a.lens_out ? min(len_in + 1, a.max_seq) : len_in;
    if (a.lens_out && active && r == 0 && ch == 0) a.lens_out[b] = L;
    pos = a.positions ? pos_in : (L > 0 ? L - 1 : 0);
    k_tok_out = (long)bb * a.max_seq + (L > 0 ? L - 1 : 0);
    if (r >= a.H && L == 0) active = false;  // nothing to append to an empty sequence
  }
  T* dst;
  if (is_q) dst = reinterpret_cast<T*>(a.q_out) + ((long)tok * a.H + r) * D;
  else if (is_k) dst = reinterpret_cast<T*>(a.k_out) + (k_tok_out * a.G + (r - nq)) * D;
  else dst = reinterpret_cast<T*>(a.v_out) + (k_tok_out * a.G + (r - nq - nk)) * D;

  if (!active) {
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = 0.f;
  }
  // all LPR lanes of a row share `active`, `is_q` and `is_k`, so the reduction below only
  // mixes lanes of one row
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
  ss = lane_group_sum<LPR>(ss);
  if (gam) {
    const float rinv = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (x[i] * rinv) * gw[i];
  }
  if ((is_q || is_k) && a.use_rope) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float c, sn;
      rope_cos_sin<sizeof(T) == 2>((double)pos * om[m], c, sn);
      const float x0 = x[2 * m], x1 = x[2 * m + 1];
      x[2 * m] = x0 * c - x1 * sn;
      x[2 * m + 1] = x0 * sn + x1 * c;
    }
  }
  if (active) store8(dst + e0, x);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(PrologueArgs a) {
  if (a.zero && blockIdx.x == 0)
    for (int i = threadIdx.x; i < a.zero_n; i += 256) a.zero[i] = 0;
  prologue_block<T, D>(a, blockIdx.x, threadIdx.x);
}

// A multi-step decode graph's pass between two steps: blocks [0, n_comb) merge step n's splits
// (one (sequence, head) each, D threads), the rest run step n + 1's prologue (its norm, RoPE
// and K/V append), each 256-thread prologue block as 256 / D consecutive blocks. The two
// jobs touch disjoint data (the combine reads the split partials and step n's lengths and
// writes out; the prologue reads step n's lengths and writes q~, the cache rows and step
// n + 1's lengths), so one launch runs them side by side.
template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_prologue_kernel(DecodeArgs ca, PrologueArgs pa,
                                                                    int n_comb) {
  __shared__ float sw[kMaxCombineSplits];
  __shared__ float s_inv;
  const unsigned bx = blockIdx.x;
  if (bx < (unsigned)n_comb) {
    combine_one<T, D>(ca, (int)(bx % (unsigned)ca.H), (int)(bx / (unsigned)ca.H), threadIdx.x, sw,
                      s_inv);
    return;
  }
  constexpr unsigned PIECES = 256 / D;
  const unsigned v = bx - (unsigned)n_comb;
  prologue_block<T, D>(pa, v / PIECES, (v % PIECES) * D + threadIdx.x);
}

template <typename T, int D>
static hipError_t launch_prologue_t(const PrologueArgs& a, int slots, hipStream_t s) {
  constexpr int ROWS_PER_BLOCK = 256 / (D / 8);
  const long rpt = (a.q ? a.H : 0) + (a.k ? a.G : 0) + ((a.decode && a.v) ? a.G : 0);
  if (rpt == 0) return hipSuccess;
  // launches of at most 2^22 rows (2^18 workgroups), so the kernel's row index stays
  // 32-bit with room to spare; inputs that large amortise the extra launches
  const long per = std::max(1L, (1L << 22) / rpt);
  for (long s0 = 0; s0 < slots; s0 += per) {
    PrologueArgs c = a;
    c.slot0 = (int)s0;
    const long rows = std::min(per, (long)slots - s0) * rpt;
    const long grid = (rows + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    hipLaunchKernelGGL((qk_norm_rope_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, s, c);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <typename T, int D>
static hipError_t launch_combine_prologue_t(const DecodeArgs& ca, const PrologueArgs& pa,
                                            hipStream_t s) {
  constexpr int ROWS_PER_BLOCK = 256 / (D / 8);
  const long rpt = pa.H + 2L * pa.G;  // q, k_new and v_new rows of every sequence
  const long pblocks = (pa.B * rpt + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
  const long grid = (long)ca.H * ca.B + pblocks * (256 / D);
  hipLaunchKernelGGL((decode_combine_prologue_kernel<T, D>), dim3((unsigned)grid), dim3(D), 0, s,
                     ca, pa, ca.H * ca.B);
  return hipGetLastError();
}

hipError_t launch_decode_combine_prologue(const DecodeArgs& ca, const PrologueArgs& pa, int d,
                                          bool bf16, hipStream_t s) {
  if (ca.B <= 0) return hipSuccess;
  if (bf16) return d == 128 ? launch_combine_prologue_t<bf16_t, 128>(ca, pa, s)
                            : launch_combine_prologue_t<bf16_t, 64>(ca, pa, s);
  return d == 128 ? launch_combine_prologue_t<float, 128>(ca, pa, s)
                  : launch_combine_prologue_t<float, 64>(ca, pa, s);
}

hipError_t launch_prologue(const PrologueArgs& a, int slots, int d, bool bf16, hipStream_t s) {
  if (slots <= 0) return hipSuccess;
  if (bf16) return d == 128 ? launch_prologue_t<bf16_t, 128>(a, slots, s)
                            : launch_prologue_t<bf16_t, 64>(a, slots, s);
  return d == 128 ? launch_prologue_t<float, 128>(a, slots, s)
                  : launch_prologue_t<float, 64>(a, slots, s);
}

}  // namespace gqa
