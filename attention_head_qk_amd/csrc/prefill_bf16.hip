// Causal GQA prefill on gfx950 matrix cores (bf16 in, fp32 accumulate).
//
// What it computes (per sequence, per query head i with KV head g = floor(i/h)):
//   out = softmax(q k^T * scale + M) v, M = -inf above the diagonal, the row max subtracted
// -- zhanghao0806.com "Qwen3系列1-理论基础&真实结构", D1-4 (formula), D1-5 (mask), D1-2
// (stable softmax), D2-3 (h query heads of a group share one K/V head); ewbang.com
// "深入剖析Qwen3模型架构" 3.1.2 (head i reads K/V head floor(i/h)). K arrives normalised and
// rotated by the prologue kernel; each workgroup applies the same per-head RMSNorm and RoPE
// (D2-1, D2-2) to its own Q columns as it loads them.
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
// * K tiles go global -> LDS by DMA (16-byte buffer loads into LDS), XOR-swizzled by 16-byte
//   chunk. The A operand of O^T needs 8 consecutive keys per lane, so V tiles are loaded
//   into registers and transposed on their way into LDS (4 keys x 8 d per thread, v_perm_b32
//   regroups the halves, 8-byte stores), with the key order inside each 16-key step permuted
//   so the 8 keys a lane needs are one 16-byte read. Both layouts are bank-conflict free for
//   the reads and writes they see. Buffer descriptors bound each sequence, so rows past its
//   end read as zero without per-load tests, and every LDS address is computed once.
// * Pipeline. LDS is double-buffered: the loads of tile t+1 are issued before the MFMAs of
//   tile t and the V^T store follows them; one barrier per tile.
// * Softmax in base 2 with scale*log2(e) folded into one FMA per score. The reference max
//   of a column only moves when the probabilities it gives would exceed 2^32 (a wave-uniform
//   test on the tile sums), so the common tile needs neither a max nor an O rescale; the
//   result is unchanged because softmax does not depend on the subtracted constant.
// * Scheduling. Blocks are issued heaviest first (descending position) so the causal
//   triangle drains without a long tail; when the whole grid fits on the chip in about two
//   rounds, heavy and light blocks are paired instead (zigzag). The group index is the
//   fastest-varying part of the block id, which keeps the blocks of one KV group on the same
//   XCD (blocks are dealt round-robin over the 8 XCDs) when G is a multiple of 8, so its K/V
//   stay in that XCD's L2.
#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {

constexpr int KT = 64;      // keys per tile
constexpr int COLS = 128;   // columns per workgroup (4 waves x 32)

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Swizzle of the 16-byte chunk index of a V^T row (8 chunks of 8 keys). It depends on d mod 32
// only, so the 32-row tiles of one lane differ by a constant offset, and it is conflict-free
// both for the MFMA reads (16 consecutive d) and for the transposing writes (one d per 16 lanes).
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 3) & 3) ^ (d & 7); }

}  // namespace

template <int D>
__global__ __launch_bounds__(256, 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int DCH = D / 8;               // 16-byte chunks per K row
  constexpr int NST = D / 16;              // k-steps of S^T = K Q^T
  constexpr int NMT = D / 32;              // 32-row tiles of O^T
  constexpr int KBYTES = KT * D * 2;       // one K tile
  constexpr int VBYTES = D * KT * 2;       // one V^T tile
  constexpr int BUFBYTES = KBYTES + VBYTES;
  constexpr int KDMA = KBYTES / 1024 / 4;  // 1 KB DMA instructions per wave per K tile
  constexpr int KROWS_DMA = 1024 / (D * 2);  // K rows per DMA instruction
  __shared__ __attribute__((aligned(16))) char smem[2 * BUFBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep it scalar
  const int l32 = lane & 31;
  const int grp = lane >> 5;

  // ---- block -> (sequence, group, column block). Heaviest first; with zigzag the second
  // half of the grid runs lightest first instead, so that block ids i and i + grid/2, which
  // the dispatcher places on the same CU when the whole grid is resident at once, carry
  // complementary causal work (n_blk - r and r + 1 tiles).
  const int id = blockIdx.x;
  const int g = id % a.G;
  const int rest = id / a.G;
  const int b = rest % a.B;
  const int r = rest / a.B;
  const int half_r = (a.n_blk + 1) / 2;
  const int blk = (a.zigzag && r >= half_r) ? r - half_r : a.n_blk - 1 - r;
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

  // ---- Q^T (B operand): step st holds d = 16 st + 8 grp + [0, 8) of this lane's column; the
  // rest of the row is in the partner lane l^32. The row is normalised (per-head RMSNorm with
  // gamma_q) and rotated (RoPE at the column's position) here in fp32, then rounded to bf16:
  // the same arithmetic as the prologue kernel, without a trip through HBM.
  bf16x8_t qf[NST];
  {
    const long qrow = ((long)(seq0 + pcol) * a.H + head) * D + 8 * grp;
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) + qrow;
    u32x4_t raw[NST];
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      raw[st] = u32x4_t{0u, 0u, 0u, 0u};
      if (cvalid) raw[st] = *reinterpret_cast<const u32x4_t*>(qp + 16 * st);
    }
    float rinv = 1.f;
    if (a.gq) {
      float ss = 0.f;
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        float x[8];
        unpack8(raw[st], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
      }
      ss += xor_shfl(ss, 32);
      rinv = 1.0f / sqrtf(ss * (1.0f / D) + a.eps);
    }
    const int pos = a.positions ? a.positions[seq0 + pcol] : pcol;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      float x[8];
      unpack8(raw[st], x);
      if (a.gq) {
        float gw[8];
        load8(reinterpret_cast<const bf16_t*>(a.gq) + 16 * st + 8 * grp, gw);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (x[e] * rinv) * gw[e];
      }
      if (a.use_rope) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float c, sn;
          rope_cos_sin<true>((double)pos * a.omega[8 * st + 4 * grp + m], c, sn);
          const float x0 = x[2 * m], x1 = x[2 * m + 1];
          x[2 * m] = x0 * c - x1 * sn;
          x[2 * m + 1] = x0 * sn + x1 * c;
        }
      }
      qf[st] = as_bf16x8(pack8(x));
    }
  }

  // ---- buffer descriptors over this (sequence, group)'s K and V rows; rows >= Tb read as 0
  const int row_bytes = a.G * D * 2;  // bytes between consecutive tokens
  const long base_el = ((long)seq0 * a.G + g) * D;
  const int nrec = (Tb - 1) * row_bytes + D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16_t*>(a.kt) + base_el, nrec);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16_t*>(a.v) + base_el, nrec);

  // K tile: DMA straight into LDS. DMA instruction n (= i*4 + wave) fills bytes
  // [n KB, (n+1) KB) of the tile; lane slot pos of row r receives logical chunk pos ^ (r % DCH),
  // i.e. the tile is stored XOR-swizzled by 16-byte chunk.
  int k_voff[KDMA];
#pragma unroll
  for (int i = 0; i < KDMA; ++i) {
    const int n = i * 4 + wave;
    const int r = n * KROWS_DMA + lane / DCH;
    const int c = (lane % DCH) ^ (r % DCH);
    k_voff[i] = r * row_bytes + c * 16;
  }
  // V tile: thread (vch = tid / 16, vq = tid % 16) loads keys 4vq..4vq+3 at d-chunk vch.
  const bool vload = tid < (KT / 4) * DCH;
  const int vch = tid >> 4, vq = tid & 15;
  int v_voff[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) v_voff[kk] = (4 * vq + kk) * row_bytes + vch * 16;
  // V^T destination of this thread: keys 4vq.. -> physical slot 32kb + 16half + 8gg + 4aa
  int vt_woff[8];
  {
    const int kb = vq >> 3, qi = vq & 7;
    const int half = qi >> 2, aa = (qi >> 1) & 1, gg = qi & 1;
    const int chunk = 4 * kb + 2 * half + gg;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * vch + e;
      vt_woff[e] = KBYTES + d * KT * 2 + ((chunk ^ vt_swz(d)) * 16) + 8 * aa;
    }
  }
  // LDS read offsets (the m-tile and buffer parts are compile-time offsets)
  int k_roff[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) k_roff[st] = l32 * D * 2 + ((((2 * st + grp) ^ (l32 % DCH))) * 16);
  int v_roff[2][2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
      v_roff[kb][hf] = KBYTES + l32 * KT * 2 + (((4 * kb + 2 * hf + grp) ^ vt_swz(l32)) * 16);

  u32x4_t vreg[4];

  // The buffer index is always a literal at the call sites, so after inlining every LDS
  // offset below folds into the instructions' immediate offset field.
  auto issue_tile = [&](int BUF, int t) {
    const int soff = t * KT * row_bytes;
#pragma unroll
    for (int i = 0; i < KDMA; ++i)
      dma16(krs, smem + BUF * BUFBYTES + (i * 4 + wave) * 1024, k_voff[i], soff);
    if (vload) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        vreg[kk] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, v_voff[kk], soff, 0));
    }
  };

  auto store_vt = [&](int BUF) {
    if (vload) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        // d = 8 vch + 2w (low halves of the four keys) and d + 1 (high halves)
        const uint32_t lo01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
        const uint32_t lo23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
        const uint32_t hi23 = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], 0x07060302u);
        *reinterpret_cast<u32x2_t*>(smem + BUF * BUFBYTES + vt_woff[2 * w]) = u32x2_t{lo01, lo23};
        *reinterpret_cast<u32x2_t*>(smem + BUF * BUFBYTES + vt_woff[2 * w + 1]) = u32x2_t{hi01, hi23};
      }
    }
  };

  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = f32x16_t{};
  float m_run = -INFINITY;  // reference max of this column, log2 units
  float l_run = 0.f;        // this lane's share of the running sum
  const float sl2e = a.scale_log2e;

  auto compute_tile = [&](int BUF, int t) {
    const char* sb = smem + BUF * BUFBYTES;
    // ---- S^T = K Q^T: two 32-key blocks
    f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
    for (int st = 0; st < NST; ++st) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const u32x4_t kw = *reinterpret_cast<const u32x4_t*>(sb + k_roff[st] + mt * 32 * D * 2);
        s[mt] = mfma32(as_bf16x8(kw), qf[st], s[mt]);
      }
    }
    // ---- mask: only tiles that reach past the wave's lowest position, or past the end.
    // key = t0 + 32 mt + 8 (i/4) + 4 grp + i%4 is visible iff key <= min(plim, Tb - 1).
    const int t0 = t * KT;
    if ((a.causal && t0 + KT - 1 > p_wlo) || t0 + KT > Tb) {
      const int lim = (plim < Tb - 1 ? plim : Tb - 1) - t0 - 4 * grp;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * mt + 8 * (i >> 2) + (i & 3) > lim) s[mt][i] = -INFINITY;
      }
    }
    // ---- probabilities against the column's reference max m_run (log2 units). The common
    // case needs no max at all: P = 2^(s*c - m_run) is accepted while every lane's tile sum
    // stays <= 2^32 (so every P does); otherwise (always on the first tile, where m_run is
    // -inf) the wave takes the exact path: tile max, new reference, rescale O and l, redo P.
    // The row sum is taken over the bf16-rounded P that also feeds the P.V product.
    const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
    uint32_t pk[2][8];
    float ls = 0.f;
    auto probs = [&]() {
      ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * j], sl2e, -m_run));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][2 * j + 1], sl2e, -m_run));
          f32x2_t pp = {p0, p1};
          const bf16x2_t pb2 = __builtin_convertvector(pp, bf16x2_t);
          pk[kb][j] = __builtin_bit_cast(uint32_t, pb2);
          ls = __builtin_amdgcn_fdot2_f32_bf16(pb2, one2, ls, false);
        }
      }
    };
    probs();
    if (__any(!(ls <= 0x1p32f))) {
      float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s[0][i], s[1][i]));
      mx = fmaxf(mx, xor_shfl(mx, 32)) * sl2e;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) o[mt] *= alpha;
      m_run = m_new;
      probs();
    }
    l_run += ls;
    bf16x8_t pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        pb[kb][hf] = as_bf16x8(u32x4_t{pk[kb][4 * hf], pk[kb][4 * hf + 1], pk[kb][4 * hf + 2], pk[kb][4 * hf + 3]});
    // ---- O^T += V^T P^T
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const u32x4_t vw = *reinterpret_cast<const u32x4_t*>(sb + v_roff[kb][hf] + mt * 32 * KT * 2);
          o[mt] = mfma32(as_bf16x8(vw), pb[kb][hf], o[mt]);
        }
      }
    }
  };

  // ---- pipeline: tile t+1 is in flight (K by DMA, V in registers) while tile t computes
  auto step = [&](int cur, int nxt, int t) {
    const bool more = t + 1 < ntiles;
    if (more) issue_tile(nxt, t + 1);
    compute_tile(cur, t);
    if (more) store_vt(nxt);
    wait_vmem();
    __syncthreads();
  };

  issue_tile(0, 0);
  store_vt(0);
  wait_vmem();
  __syncthreads();
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    step(0, 1, t);
    step(1, 0, t + 1);
  }
  if (t < ntiles) step(0, 1, t);

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
