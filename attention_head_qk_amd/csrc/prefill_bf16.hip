// Causal GQA prefill on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// What it computes (per sequence, per query head i with KV head g = floor(i/h)):
//   out = softmax(q k^T * scale + M) v, M = -inf above the diagonal, the row max subtracted
// -- zhanghao0806.com "Qwen3系列1-理论基础&真实结构", D1-4 (formula), D1-5 (mask), D1-2
// (stable softmax), D2-3 (h query heads of a group share one K/V head); ewbang.com
// "深入剖析Qwen3模型架构" 3.1.2 (head i reads K/V head floor(i/h)). Q and K arrive already
// normalised and rotated by the prologue kernel.
//
// Design for CDNA4 (not a port of any FlashAttention code):
// * Columns. A workgroup owns 128 "columns"; a column is one (query position, head) pair of
//   one KV group g, ordered position-major (c = pos*h + j). All h heads of a position share
//   K/V, so a K/V tile staged once in LDS is used by every head of the group, and the
//   causal limit of a column depends on its position only.
// * Transposed scores. Each wave computes S^T = K Q^T for its 32 columns with
//   v_mfma_f32_32x32x16_bf16 (A = K tile from LDS, B = Q^T held in registers for the whole
//   sweep). In the 32x32 accumulator layout lane l owns column l%32, so the online softmax
//   of a column lives in one lane (plus its partner lane l^32 for the other half of the
//   keys), and the bf16-packed probabilities already sit in the B-operand layout of the
//   second product O^T = V^T P^T: no LDS round trip for P.
// * V^T in LDS. The A operand of O^T needs 8 consecutive keys per lane, so V tiles are
//   transposed on their way into LDS (4 keys x 8 d per thread, v_perm_b32 regroups the
//   halves, 8-byte LDS stores), with the key order inside each 16-key step permuted so the
//   8 keys a lane needs are one 16-byte LDS read. K and V^T rows are XOR-swizzled in 16-byte
//   chunks to spread LDS banks.
// * Pipeline. LDS is double-buffered: the global loads of tile t+1 are issued before the
//   MFMAs of tile t and written to the other buffer after them; one barrier per tile.
// * Softmax in base 2 with scale*log2(e) folded into one FMA per score; the O rescale is
//   skipped when no column's max moved (a wave-uniform test).
// * Scheduling. Blocks are issued heaviest first (descending position) so the causal
//   triangle drains without a long tail, and the group index is the fastest-varying part of
//   the block id, which keeps the blocks of one KV group on the same XCD (blocks are dealt
//   round-robin over the 8 XCDs) when G is a multiple of 8, so its K/V stay in that L2.
#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {

constexpr int KT = 64;     // keys per tile
constexpr int COLS = 128;  // columns per workgroup (4 waves x 32)

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t w) { return __builtin_bit_cast(bf16x8_t, w); }

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Swizzle of the 16-byte chunk index of a V^T row (8 chunks of 8 keys).
__device__ __forceinline__ int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }

template <int D>
struct Tile {
  static constexpr int DCH = D / 8;                // 16-byte chunks per K row
  static constexpr int KROWS = 256 / DCH;          // K rows loaded per pass
  static constexpr int KPASS = KT / KROWS;         // passes per K tile
  static constexpr int VTHREADS = (KT / 4) * DCH;  // threads that load V (4 keys x 8 d each)
  static constexpr int ELEMS = KT * D;             // bf16 elements per K (or V^T) tile
};

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillArgs a) {
  using TL = Tile<D>;
  constexpr int DCH = TL::DCH;
  constexpr int NST = D / 16;  // k-steps of S^T = K Q^T
  constexpr int NMT = D / 32;  // 32-row tiles of O^T
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][2][TL::ELEMS];  // [buf][K | V^T]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int grp = lane >> 5;

  // ---- block -> (sequence, group, column block), heaviest first
  const int id = blockIdx.x;
  const int g = id % a.G;
  const int rest = id / a.G;
  const int b = rest % a.B;
  const int blk = a.n_blk - 1 - rest / a.B;
  int seq0, Tb;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    Tb = a.cu_seqlens[b + 1] - seq0;
  } else {
    seq0 = b * a.T;
    Tb = a.T;
  }
  const int h = a.h;
  const long ncol = (long)Tb * h;
  const long col0 = (long)blk * COLS;
  if (col0 >= ncol) return;
  const long colmax = (col0 + COLS - 1 < ncol) ? col0 + COLS - 1 : ncol - 1;
  const int p_hi = (int)(colmax / h);
  const int kv_end = a.causal ? p_hi + 1 : Tb;
  const int ntiles = (kv_end + KT - 1) / KT;

  // ---- this lane's column
  const long mycol = col0 + wave * 32 + l32;
  const bool cvalid = mycol < ncol;
  const int pcol = cvalid ? (int)(mycol / h) : Tb - 1;
  const int head = g * h + (cvalid ? (int)(mycol % h) : 0);
  const long wcol = col0 + wave * 32;
  const int p_wlo = (wcol < ncol) ? (int)(wcol / h) : Tb - 1;  // lowest position in the wave
  const int plim = a.causal ? pcol : 0x7fffffff;

  // ---- Q^T (B operand): step st holds d = 16 st + 8 grp + [0, 8) of this lane's column
  const bf16_t* qt = reinterpret_cast<const bf16_t*>(a.qt);
  const bf16_t* kt = reinterpret_cast<const bf16_t*>(a.kt);
  const bf16_t* vv = reinterpret_cast<const bf16_t*>(a.v);
  bf16x8_t qf[NST];
  {
    const bf16_t* qp = qt + ((long)(seq0 + pcol) * a.H + head) * D + 8 * grp;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (cvalid) w = *reinterpret_cast<const u32x4_t*>(qp + 16 * st);
      qf[st] = as_bf16x8(w);
    }
  }

  // ---- tile staging: global -> registers -> LDS
  const long kv_stride = (long)a.G * D;  // elements between consecutive tokens of K / V
  const bf16_t* kg = kt + (long)seq0 * kv_stride + (long)g * D;
  const bf16_t* vg = vv + (long)seq0 * kv_stride + (long)g * D;
  const int krow0 = tid / DCH, kch = tid % DCH;
  const bool vload = tid < TL::VTHREADS;
  const int vq = tid / DCH, vch = tid % DCH;

  u32x4_t kreg[TL::KPASS];
  u32x4_t vreg[4];

  auto load_tile = [&](int t) {
    const int t0 = t * KT;
#pragma unroll
    for (int i = 0; i < TL::KPASS; ++i) {
      const int key = t0 + krow0 + i * TL::KROWS;
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (key < Tb) w = *reinterpret_cast<const u32x4_t*>(kg + (long)key * kv_stride + kch * 8);
      kreg[i] = w;
    }
    if (vload) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = t0 + 4 * vq + kk;
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (key < Tb) w = *reinterpret_cast<const u32x4_t*>(vg + (long)key * kv_stride + vch * 8);
        vreg[kk] = w;
      }
    }
  };

  auto store_tile = [&](int buf) {
    bf16_t* ks = smem[buf][0];
    bf16_t* vs = smem[buf][1];
#pragma unroll
    for (int i = 0; i < TL::KPASS; ++i) {
      const int row = krow0 + i * TL::KROWS;
      *reinterpret_cast<u32x4_t*>(ks + row * D + ((kch ^ (row & (DCH - 1))) * 8)) = kreg[i];
    }
    if (vload) {
      // keys 4vq..4vq+3 -> physical slot 32kb + 16half + 8grp' + 4a' (see file comment)
      const int kb = vq >> 3, qi = vq & 7;
      const int half = qi >> 2, aa = (qi >> 1) & 1, gg = qi & 1;
      const int chunk = 4 * kb + 2 * half + gg;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // d = 8 vch + 2w (low halves) and 8 vch + 2w + 1 (high halves)
        const uint32_t lo01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x07060302u);
        const int d0 = 8 * vch + 2 * w;
        const int d1 = d0 + 1;
        u32x2_t e0 = {lo01, lo23};
        u32x2_t e1 = {hi01, hi23};
        *reinterpret_cast<u32x2_t*>(vs + d0 * KT + ((chunk ^ vt_swz(d0)) * 8) + 4 * aa) = e0;
        *reinterpret_cast<u32x2_t*>(vs + d1 * KT + ((chunk ^ vt_swz(d1)) * 8) + 4 * aa) = e1;
      }
    }
  };

  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = f32x16_t{};
  float m_run = -INFINITY;  // running max of this column, in log2 units
  float l_run = 0.f;        // this lane's share of the running sum
  const float sl2e = a.scale_log2e;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1);

    const bf16_t* ks = smem[cur][0];
    const bf16_t* vs = smem[cur][1];

    // ---- S^T = K Q^T: two 32-key blocks
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int st = 0; st < NST; ++st) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int row = 32 * mt + l32;
        const int ch = 2 * st + grp;
        const u32x4_t kw = *reinterpret_cast<const u32x4_t*>(ks + row * D + ((ch ^ (row & (DCH - 1))) * 8));
        s[mt] = mfma32(as_bf16x8(kw), qf[st], s[mt]);
      }
    }

    // ---- mask: only tiles that reach past the wave's lowest position, or past the end
    const int t0 = t * KT;
    if ((a.causal && t0 + KT - 1 > p_wlo) || t0 + KT > Tb) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = t0 + 32 * mt + 8 * (i >> 2) + 4 * grp + (i & 3);
          if (key > plim || key >= Tb) s[mt][i] = -INFINITY;
        }
      }
    }

    // ---- online softmax of this column (lanes l and l^32 share it)
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fmaxf(s[0][i], s[1][i]));
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const float m_new = fmaxf(m_run, mx * sl2e);
    if (__any(m_new > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) o[mt] *= alpha;
      m_run = m_new;
    }
    bf16x8_t pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * hf + j], sl2e, -m_run));
          l_run += p[j];
        }
        u32x4_t w = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                     pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
        pb[kb][hf] = as_bf16x8(w);
      }
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int d = 32 * mt + l32;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int ch = 4 * kb + 2 * hf + grp;
          const u32x4_t vw = *reinterpret_cast<const u32x4_t*>(vs + d * KT + ((ch ^ vt_swz(d)) * 8));
          o[mt] = mfma32(as_bf16x8(vw), pb[kb][hf], o[mt]);
        }
      }
    }

    if (more) store_tile(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O / l -> bf16
  const float l_tot = l_run + xor_shfl(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (cvalid) {
    bf16_t* op = reinterpret_cast<bf16_t*>(a.out) + ((long)(seq0 + pcol) * a.H + head) * D;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d0 = 32 * mt + 8 * r4 + 4 * grp;
        u32x2_t w = {pack_bf16x2(o[mt][4 * r4 + 0] * inv, o[mt][4 * r4 + 1] * inv),
                     pack_bf16x2(o[mt][4 * r4 + 2] * inv, o[mt][4 * r4 + 3] * inv)};
        *reinterpret_cast<u32x2_t*>(op + d0) = w;
      }
    }
  }
}

template <int D>
static hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  const long grid = (long)a.B * a.G * a.n_blk;
  hipLaunchKernelGGL((prefill_bf16_kernel<D>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, hipStream_t s) {
  if ((long)a.B * a.G * a.n_blk <= 0) return hipSuccess;
  return d == 128 ? launch_t<128>(a, s) : launch_t<64>(a, s);
}

int prefill_bf16_cols_per_block() { return COLS; }

}  // namespace gqa
