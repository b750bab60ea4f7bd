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
// * K and V tiles go global -> LDS by DMA (16-byte buffer loads into LDS), each row's 16-byte
//   chunks XOR-swizzled. The A operand of O^T (V^T: 8 keys of one d per lane) comes out of
//   the natural [key][d] layout through transposing reads (ds_read_b64_tr_b16), so V needs
//   no registers or VALU on its way in. Every read pattern is bank-conflict free. Buffer
//   descriptors bound each sequence, so rows past its end read as zero without per-load
//   tests, and every LDS address is computed once.
// * MFMA chains. An MFMA that accumulates onto a result still in flight waits for it
//   (~100 cycles for this shape on gfx950, against ~32 between independent issues), so both
//   products keep four independent accumulators in flight: S^T splits each 32-key block's
//   d-sum in two halves, O^T updates its four 32-row tiles in turn. Fragments are read one
//   round ahead.
// * Pipeline. LDS is double-buffered: the DMA of tile t+1 is issued before the MFMAs of tile t;
//   one barrier per tile.
// * Softmax in base 2: Q is pre-scaled by scale*log2(e), so scores come out in log2 units. The
//   reference m of a column (P = 2^(s - m)) starts at 0 and only moves when a tile's
//   probabilities would leave [2^-100, 2^32], so the common tile needs neither a max, a
//   subtraction nor an O rescale; the result is unchanged because softmax does not depend on
//   the subtracted constant.
// * Scheduling. Blocks are issued heaviest first (descending position) so the causal
//   triangle drains without a long tail; when the whole grid fits on the chip in at most 2.5
//   rounds, heavy and light blocks are paired instead (zigzag), and when it fits at once
//   (and its heaviest blocks are long) the light block of a pair also takes a fixed share of
//   its heavy partner's key tiles, the two partial softmax states merged in a fixed order
//   (the paired schedule, template parameter PAIR). The group index is the
//   fastest-varying part of the block id, which keeps the blocks of one KV group on the same
//   XCD (blocks are dealt round-robin over the 8 XCDs) when G is a multiple of 8, so its K/V
//   stay in that XCD's L2; with several sequences the ranks go in runs of 32 per sequence, so
//   an XCD streams few sequences' K/V at a time. When a group spans several XCDs (G < 8) the
//   unmasked kernel's workgroups claim their ranks from a counter per group, so faster XCDs
//   take more of the work.
#include "device_common.h"
#include "kernels.h"

namespace gqa {

namespace {

constexpr int KT = 64;      // keys per tile
constexpr int COLS = 128;   // columns per workgroup (4 waves x 32)

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Swizzle of the 16-byte chunk index of a V row in LDS (row = key). A transposing read of the
// O^T product touches 8 rows (4 consecutive keys for each lane half) at 4 chunks of one 32-d
// tile; the XOR moves those rows to 4 different 64-byte bank windows, so every read is two
// bank cycles for its 512 bytes. It depends on the row's low bits only, which DMA instruction
// and read-row offsets (multiples of 4 or 8 rows) leave unchanged.
template <int D>
__device__ __forceinline__ int v_swz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }

// ds_read_b64_tr_b16: inside every 16-lane block, lane i receives element i%4 of the 8-byte
// values addressed by lanes 4j + i/4 of that block, j = 0..3.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2_t ds_read_tr16(const char* lds) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)const_cast<char*>(lds));
  return __builtin_bit_cast(u32x2_t, v);
}

}  // namespace

// MASK: bit 0 = sliding window (a.window), bit 1 = 64-key block layout (a.block_mask).
// CACHE: keys come from caches after a.cache_lens[b] earlier rows (cached prefill).
template <int D, int MASK, bool CACHE, bool PAIR>
__global__ __launch_bounds__(256, D == 64 && !PAIR ? 3 : 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int DCH = D / 8;               // 16-byte chunks per K row
  constexpr int NST = D / 16;              // k-steps of S^T = K Q^T
  constexpr int NMT = D / 32;              // 32-row tiles of O^T
  constexpr int KBYTES = KT * D * 2;       // one K tile
  constexpr int VBYTES = D * KT * 2;       // one V^T tile
  constexpr int KDMA = KBYTES / 1024 / 4;  // 1 KB DMA instructions per wave per K tile
  constexpr int KROWS_DMA = 1024 / (D * 2);  // K rows per DMA instruction
  // The four tile buffers (K and V, two of each) are separate LDS objects, so the compiler can
  // tell that the DMA into one never feeds reads of another and keeps its waits exact.
  __shared__ __attribute__((aligned(16))) char kbuf0[KBYTES];
  __shared__ __attribute__((aligned(16))) char kbuf1[KBYTES];
  __shared__ __attribute__((aligned(16))) char vbuf0[VBYTES];
  __shared__ __attribute__((aligned(16))) char vbuf1[VBYTES];
  auto k_lds = [&](int BUF) -> char* { return BUF ? kbuf1 : kbuf0; };
  auto v_lds = [&](int BUF) -> char* { return BUF ? vbuf1 : vbuf0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep it scalar
  const int l32 = lane & 31;
  const int grp = lane >> 5;

  // ---- RoPE frequencies: each wave keeps its own copy in LDS, written and read by that wave
  // only (so no barrier), filled just before the first Q row is rotated. Its global load is
  // the first of the kernel, so waiting for it never includes the Q rows or the K/V tiles
  // issued later (read lane by lane from the kernel argument inside the rotation, they cost
  // one memory round trip per 16-element step).
  __shared__ double s_omega[4][D / 2];
  const double om_in = lane < D / 2 ? a.omega[lane] : 0.0;
  auto fill_omega = [&]() {
    if (lane < D / 2) s_omega[wave][lane] = om_in;
    __builtin_amdgcn_wave_barrier();
  };
  const double* const om = s_omega[wave];

  // ---- block -> (sequence, group, column block). Heaviest first; with zigzag the second
  // half of the grid runs lightest first instead, so that block ids i and i + grid/2, which
  // the dispatcher places on the same CU when the whole grid is resident at once, carry
  // complementary causal work (n_blk - r and r + 1 tiles).
  // With rank_chunk > 1 the ranks go in chunks: the B sequences take turns with runs of
  // rank_chunk consecutive ranks each, so an XCD holds the K/V of fewer sequences at once.
  // With a.claim the rank inside the group is taken from a counter instead of the block id:
  // the dispatcher hands every XCD the same number of workgroups, and under load the XCDs
  // run at different clocks, so a fixed share of blocks per XCD ends with the slowest one;
  // claimed in time order, the heaviest-first ranks go to whichever workgroups start first.
  const int id = blockIdx.x;
  const int g = id % a.G;
  int rest = id / a.G;
  if constexpr (MASK == 0 && !CACHE) if (a.claim) {
    __shared__ int s_rank;
    if (tid == 0)
      s_rank = __hip_atomic_fetch_add(a.claim + g, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    rest = __builtin_amdgcn_readfirstlane(s_rank);
  }
  int b, r;
  if (a.rank_chunk > 1) {
    const int chunk = rest / (a.B * a.rank_chunk);
    const int w = rest - chunk * a.B * a.rank_chunk;
    const int rb = min(a.rank_chunk, a.n_blk - chunk * a.rank_chunk);
    b = w / rb;
    r = chunk * a.rank_chunk + (w - b * rb);
  } else {
    b = rest % a.B;
    r = rest / a.B;
  }
  const int half_r = (a.n_blk + 1) / 2;
  const int blk = (a.zigzag && r >= half_r) ? r - half_r : a.n_blk - 1 - r;

  // ---- one column block `blk` of sequence b, key tiles [t_lo, min(t_hi, its tiles)): with
  // slot < 0 the block's output; otherwise (paired schedule) this part's softmax state goes
  // to partial slot `slot` (0: the heavy block's own part, 1: the part its light partner
  // took), and the part that ends last merges the two and writes the output
  __shared__ int s_arrived;
  auto run = [&](const int blk, const int t_lo, const int t_hi, const int pair, const int slot) {
  int seq0, Tb;
  if (a.cu_seqlens) {
    seq0 = a.cu_seqlens[b];
    Tb = a.cu_seqlens[b + 1] - seq0;
  } else {
    seq0 = b * a.T;
    Tb = a.T;
  }
  const int h = a.h;
  // column indices fit in 32 bits (the host keeps T * h below 2^31), so the divisions by h
  // stay 32-bit
  const int ncol = Tb * h;
  const int col0 = blk * COLS;
  if (col0 >= ncol) return;
  // Keys: the sequence's own tokens, or with a cache its past cached rows followed by them
  // (the query at position p inside the chunk sits at key index past + p). kvrow0 is the
  // sequence's first K/V row, Tkv its number of keys.
  int past = 0, Tkv = Tb;
  long kvrow0 = seq0;
  if constexpr (CACHE) {
    past = max(0, min(a.cache_lens[b], a.max_seq));
    kvrow0 = (long)b * a.max_seq;
    Tkv = min(past + Tb, a.max_seq);
  }
  const int colmax = (col0 + COLS - 1 < ncol) ? col0 + COLS - 1 : ncol - 1;
  const int p_hi = (int)((unsigned)colmax / (unsigned)h);
  const int kv_end = a.causal ? min(past + p_hi + 1, Tkv) : Tkv;
  const int ntiles = (kv_end + KT - 1) / KT;

  // ---- this lane's column
  const int mycol = col0 + wave * 32 + l32;
  const bool cvalid = mycol < ncol;
  const int pcol = cvalid ? (int)((unsigned)mycol / (unsigned)h) : Tb - 1;
  const int head = g * h + (cvalid ? mycol - pcol * h : 0);
  const int wcol = col0 + wave * 32;
  const int p_wlo = (wcol < ncol) ? (int)((unsigned)wcol / (unsigned)h) : Tb - 1;  // lowest position in the wave
  const int plim = a.causal ? past + pcol : 0x7fffffff;

  // ---- the raw Q row, gamma_q and the RoPE position are loaded before anything else: the Q
  // row comes from HBM (it is read once), and its latency then overlaps the setup below and
  // the first K/V tile's loads. Lanes past the last column read row 0 (their results are
  // never stored); a null gamma or position array is replaced by a valid dummy address.
  u32x4_t qraw[NST], qgam[NST];
  int qpos_in;
  {
    const long qrow = cvalid ? ((long)(seq0 + pcol) * a.H + head) * D : 0;
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) + qrow + 8 * grp;
    const bf16_t* gp = reinterpret_cast<const bf16_t*>(a.gq ? a.gq : a.q) + 8 * grp;
    const int32_t* pp = a.positions ? a.positions + seq0 + pcol : reinterpret_cast<const int32_t*>(a.q);
    qpos_in = *pp;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      qraw[st] = *reinterpret_cast<const u32x4_t*>(qp + 16 * st);
      qgam[st] = *reinterpret_cast<const u32x4_t*>(gp + 16 * st);
    }
  }

  // ---- masks beyond causal (MASK bit 0: sliding window, bit 1: block layout). A key tile is
  // one 64-key block; tiles that no column of the workgroup sees are never visited.
  const int p_lo = (int)((unsigned)col0 / (unsigned)h);  // lowest position of the workgroup
  int t_first = 0;
  if constexpr ((MASK & 1) != 0) {
    const int klo = past + p_lo - a.window + 1;  // lowest key any column here sees
    t_first = klo > 0 ? klo / KT : 0;
  }
  // query blocks (64 key indices each) of the workgroup's columns: at most three
  const int qb_lo = (past + p_lo) / KT, qb_hi = (past + p_hi) / KT;
  const int nqb = ((CACHE ? a.max_seq : a.T) + KT - 1) / KT;  // rows of block_mask
  auto bm_word = [&](int qb, int w) -> uint32_t {  // word w of query block qb's row
    return (qb <= qb_hi && qb < nqb && w < a.bm_words) ? a.block_mask[(long)qb * a.bm_words + w]
                                                       : 0u;
  };
  // visible tiles among [32 w, 32 w + 32) for the workgroup: its rows' bits and diagonals
  auto tile_bits = [&](int w) -> uint32_t {
    uint32_t bits = bm_word(qb_lo, w) | bm_word(qb_lo + 1, w) | bm_word(qb_lo + 2, w);
    for (int qb = qb_lo; qb <= qb_hi; ++qb)
      if ((qb >> 5) == w) bits |= 1u << (qb & 31);
    return bits;
  };
  auto next_tile = [&](int t) -> int {  // first visible tile after t, or ntiles
    if constexpr ((MASK & 2) == 0) {
      return t + 1;
    } else {
      int c = t + 1;
      while (c < ntiles) {
        const int w = c >> 5;
        const uint32_t bits = tile_bits(w) & (~0u << (c & 31));
        if (bits) {
          c = (w << 5) + __builtin_ctz(bits);
          break;
        }
        c = (w + 1) << 5;
      }
      return c < ntiles ? c : ntiles;
    }
  };
  // this column: key index, first key of its window, query block; the wave's highest
  // window start (tiles below it need the lower-edge mask)
  const int kq = past + pcol;
  const int lane_lo = (MASK & 1) ? kq - a.window + 1 : 0;
  const int qb_c = kq / KT;
  int wlo_hi = 0;
  if constexpr ((MASK & 1) != 0) {
    const int wlast = (wcol + 31 < ncol) ? wcol + 31 : ncol - 1;
    wlo_hi = past + (int)((unsigned)wlast / (unsigned)h) - a.window + 1;
  }
  // does this column see any key of tile t? (same answer for both lanes of the column)
  auto col_sees = [&](int t) -> bool {
    const int t0 = t * KT;
    const int hi = min(min(plim, Tkv - 1), t0 + KT - 1);
    bool vis = max(t0, lane_lo) <= hi;
    if constexpr ((MASK & 2) != 0) {
      const int k = qb_c - qb_lo;  // 0..2
      const int w = t >> 5;
      const uint32_t row = k == 0 ? bm_word(qb_lo, w) : (k == 1 ? bm_word(qb_lo + 1, w)
                                                                : bm_word(qb_lo + 2, w));
      vis = vis && (((row >> (t & 31)) & 1u) != 0u || qb_c == t);
    }
    return vis;
  };

  // ---- Q^T (B operand): step st holds d = 16 st + 8 grp + [0, 8) of this lane's column; the
  // rest of the row is in the partner lane l^32. The row is normalised (per-head RMSNorm with
  // gamma_q) and rotated (RoPE at the column's position) here in fp32 -- the same arithmetic
  // as the prologue kernel, without a trip through HBM -- then multiplied by scale * log2(e),
  // so that the scores come out of the matrix cores in log2 units, and rounded to bf16.
  bf16x8_t qf[NST];
  // RoPE cos / sin: all h heads of a position share them, so with h >= 4 they are computed
  // once per (position, pair) into the second LDS buffer, which nothing uses before the
  // first tile's barrier. Only the masked variants do this: their workgroups visit few
  // tiles, so the start matters; elsewhere the extra barrier and code cost more than the
  // trigonometry saved.
  const int npos = p_hi - p_lo + 1;
  const bool rope_tab = MASK != 0 && a.use_rope && h >= 4 && npos * (D / 2) * 8 <= KBYTES;
  f32x2_t* const tab = reinterpret_cast<f32x2_t*>(kbuf1);
  auto build_rope_table = [&]() {
    for (int e = tid; e < npos * (D / 2); e += 256) {
      const int p = p_lo + e / (D / 2), j = e % (D / 2);
      const int pos = a.positions ? a.positions[seq0 + p] : past + p;
      float c, sn;
      rope_cos_sin<true>((double)pos * om[j], c, sn);
      tab[e] = f32x2_t{c, sn};
    }
  };
  auto make_q = [&]() {  // once the first K/V tile is in flight
    const u32x4_t (&raw)[NST] = qraw;
    const u32x4_t (&gr)[NST] = qgam;
    const int pos = a.positions ? qpos_in : past + pcol;
    // one factor for the norm and the score scale (RoPE is linear, so scaling before the
    // rotation is the same as after it)
    float f = a.scale_log2e;
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
      f = a.scale_log2e / sqrtf(ss * (1.0f / D) + a.eps);
    }
    const f32x2_t* trow = tab + (pcol - p_lo) * (D / 2) + 4 * grp;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      float x[8];
      unpack8(raw[st], x);
      if (a.gq) {
        float gw[8];
        unpack8(gr[st], gw);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = (x[e] * f) * gw[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] *= f;
      }
      if (a.use_rope) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          float c, sn;
          if (rope_tab) {
            const f32x2_t cs = trow[8 * st + m];
            c = cs[0];
            sn = cs[1];
          } else {
            rope_cos_sin<true>((double)pos * om[8 * st + 4 * grp + m], c, sn);
          }
          // explicit FMAs: every kernel variant rounds the rotation the same way
          const float x0 = x[2 * m], x1 = x[2 * m + 1];
          x[2 * m] = fmaf(x0, c, -(x1 * sn));
          x[2 * m + 1] = fmaf(x0, sn, x1 * c);
        }
      }
      qf[st] = as_bf16x8(pack8(x));
    }
  };

  // ---- buffer descriptors over this (sequence, group)'s K and V rows. They end at kv_end,
  // the last key any column of the workgroup sees: rows past it (in the last tile) read as 0,
  // so nothing past the workgroup's own causal limit is fetched, and a non-finite V value
  // there never meets the zero weight it would get (0 * inf and 0 * NaN are NaN)
  const int row_bytes = a.G * D * 2;  // bytes between consecutive tokens
  const long base_el = (kvrow0 * a.G + g) * D;
  const int nrec = (kv_end - 1) * row_bytes + D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16_t*>(a.kt) + base_el, nrec);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16_t*>(a.v) + base_el, nrec);

  // K tile: DMA straight into LDS. DMA instruction n (= i*4 + wave) fills bytes
  // [n KB, (n+1) KB) of the tile; lane slot pos of row r receives logical chunk pos ^ (r % DCH),
  // i.e. the tile is stored XOR-swizzled by 16-byte chunk. Row r = 4 KROWS_DMA i + r0 and
  // r % DCH does not depend on i, so the i part goes into the scalar offset. (Buffer range
  // checks include the scalar offset: rows past the sequence still read as zero.)
  int k_voff;
  {
    const int r0 = wave * KROWS_DMA + lane / DCH;
    static_assert((4 * KROWS_DMA) % DCH == 0, "the swizzle of a DMA row is the same for every i");
    k_voff = r0 * row_bytes + ((lane % DCH) ^ (r0 % DCH)) * 16;
  }
  // V tile: DMA into LDS in natural [key][d] order (after K in the same buffer), each row's
  // 16-byte chunks XOR-swizzled by v_swz; the row layout of the DMA is the same as K's.
  int vd_voff;
  {
    const int r0 = wave * KROWS_DMA + lane / DCH;
    vd_voff = r0 * row_bytes + ((lane % DCH) ^ v_swz<D>(r0)) * 16;
  }
  // LDS read offsets (the m-tile and buffer parts are compile-time offsets)
  int k_roff[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) k_roff[st] = l32 * D * 2 + ((((2 * st + grp) ^ (l32 % DCH))) * 16);
  // O^T A operand (V^T, rows d = 32 mt + l32): two transposing reads per fragment. Lane l
  // (s = l % 16, grp = l / 32) addresses key row 4 grp + s/4 (+ 32 kb + 16 hf + 8 rd, all
  // immediate offsets) at d = 32 mt + 16 ((l / 16) & 1) + 4 (s % 4): it then receives keys
  // 4 grp + 0..3 (rd = 0) and 8 + 4 grp + 0..3 (rd = 1) of its own d, the key order of the
  // P^T operand.
  int v_roff[NMT];
  {
    const int s16 = lane & 15;
    const int row = 4 * grp + (s16 >> 2);
    const int cl = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
      v_roff[mt] = row * D * 2 + (((4 * mt + cl) ^ v_swz<D>(row)) * 16) + 8 * (s16 & 1);
  }

  // The buffer index is always a literal at the call sites, so after inlining every LDS
  // offset below folds into the instructions' immediate offset field.
  auto issue_k = [&](int BUF, int t) {  // K tile t -> LDS buffer BUF (DMA)
    const int soff = t * KT * row_bytes;
#pragma unroll
    for (int i = 0; i < KDMA; ++i)
      dma16(krs, k_lds(BUF) + (i * 4 + wave) * 1024, k_voff,
            soff + i * 4 * KROWS_DMA * row_bytes);
  };
  auto issue_v = [&](int BUF, int t) {  // V tile t -> LDS buffer BUF (DMA)
    const int soff = t * KT * row_bytes;
#pragma unroll
    for (int i = 0; i < KDMA; ++i)
      dma16(vrs, v_lds(BUF) + (i * 4 + wave) * 1024, vd_voff,
            soff + i * 4 * KROWS_DMA * row_bytes);
  };

  f32x16_t o[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = f32x16_t{};
  float m_run = 0.f;     // reference of this column (log2 units): P = 2^(s - m_run)
  float l_run = 0.f;     // this lane's share of the running sum
  bool shifted = false;  // wave-uniform: some column's reference has left 0

  // ---- S^T = K Q^T for one tile (two 32-key blocks) from LDS buffer BUF. An MFMA that
  // accumulates onto a result still in flight waits for it (~100 cycles for this shape,
  // against ~32 between independent issues), so the d-sum of each block is split in two
  // halves: four independent accumulators, added at the end.
  auto s_product = [&](int BUF, f32x16_t (&s)[2]) {
    const char* sb = k_lds(BUF);
    constexpr int HS = NST / 2;
    f32x16_t s4[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) s4[mt][hh] = f32x16_t{};
    // round r: one MFMA on each of the four accumulators, its K fragments read a round ahead
    u32x4_t kf[2][4];
    auto load = [&](int r, u32x4_t (&f)[4]) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          f[2 * hh + mt] = *reinterpret_cast<const u32x4_t*>(sb + k_roff[r + hh * HS] + mt * 32 * D * 2);
    };
    load(0, kf[0]);
#pragma unroll
    for (int r = 0; r < HS; ++r) {
      if (r + 1 < HS) load(r + 1, kf[(r + 1) & 1]);
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          s4[mt][hh] = mfma32(as_bf16x8(kf[r & 1][2 * hh + mt]), qf[r + hh * HS], s4[mt][hh]);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) s[mt] = s4[mt][0] + s4[mt][1];
  };

  // ---- mask: only tiles that reach past the wave's lowest position, or past the end.
  // key = t0 + 32 mt + 8 (i/4) + 4 grp + i%4 is visible iff key <= min(plim, Tkv - 1).
  auto mask_tile = [&](f32x16_t (&s)[2], int t) {
    const int t0 = t * KT;
    bool need = (a.causal && t0 + KT - 1 > past + p_wlo) || t0 + KT > Tkv;
    if constexpr ((MASK & 1) != 0) need = need || t0 < wlo_hi;
    // with several query blocks in the workgroup, a visited tile may be hidden from a column
    if constexpr ((MASK & 2) != 0) need = need || qb_lo != qb_hi;
    if (need) {
      const int lim = (plim < Tkv - 1 ? plim : Tkv - 1) - t0 - 4 * grp;
      int lo = lane_lo - t0 - 4 * grp;  // keys below the window
      if constexpr ((MASK & 2) != 0) {
        if (qb_lo != qb_hi && !col_sees(t)) lo = 0x7fffffff;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kk = 32 * mt + 8 * (i >> 2) + (i & 3);
          if (kk > lim || (MASK != 0 && kk < lo)) s[mt][i] = -INFINITY;
        }
      }
    }
  };

  // ---- probabilities P = 2^(s - m_run); softmax does not depend on the reference m_run, it
  // only keeps P in range. It starts at 0, so while it stays there P = 2^s needs no
  // subtraction. A tile is accepted while every lane's tile sum is <= 2^32 (so no P or sum
  // can overflow) and every column's running sum is >= 2^-100 (so its largest P is a normal
  // number); otherwise the wave takes the exact path: the column max becomes the reference
  // (never lower than before, unless nothing has been summed yet), O and l are rescaled, P is
  // redone; once a reference has moved, the wave takes that path for every later tile. The
  // row sum is taken over the bf16-rounded P that also feeds the P.V product.
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
  auto probs = [&](const f32x16_t (&s)[2], uint32_t (&pk)[2][8], bool sub) {
    float ls4[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: no long dependency chain
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x0 = sub ? s[kb][2 * j] - m_run : s[kb][2 * j];
        const float x1 = sub ? s[kb][2 * j + 1] - m_run : s[kb][2 * j + 1];
        f32x2_t pp = {__builtin_amdgcn_exp2f(x0), __builtin_amdgcn_exp2f(x1)};
        const bf16x2_t pb2 = __builtin_convertvector(pp, bf16x2_t);
        pk[kb][j] = __builtin_bit_cast(uint32_t, pb2);
        ls4[j & 3] = __builtin_amdgcn_fdot2_f32_bf16(pb2, one2, ls4[j & 3], false);
      }
    }
    return (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
  };
  auto rescale = [&](const f32x16_t (&s)[2]) {
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s[0][i], s[1][i]));
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const float l_col = l_run + xor_shfl(l_run, 32);  // the column's sum before this tile
    float m_new = l_col > 0.f ? fmaxf(m_run, mx) : mx;
    if (m_new == -INFINITY) m_new = m_run;  // no visible key yet: keep the reference
    const float alpha = l_col > 0.f ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
    l_run *= alpha;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) o[mt] *= alpha;
    m_run = m_new;
  };

  // ---- O^T += V^T P^T from LDS buffer BUF: round (kb, hf) issues one MFMA on each of the
  // NMT accumulators (independent chains), its V^T fragments read a round ahead. The wave
  // runs this all-MFMA stretch at raised issue priority, so that on a SIMD shared with a
  // wave of the other workgroup its products go first whenever the matrix core is free and
  // the other wave's exponentials fill the VALU slots between them (measured 1-2% faster on
  // the dense, long and varlen workloads; the same raise on the S^T rounds was not).
  auto pv_product = [&](int BUF, const uint32_t (&pk)[2][8]) {
    const char* sb = v_lds(BUF);
    bf16x8_t pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
        pb[kb][hf] = as_bf16x8(u32x4_t{pk[kb][4 * hf], pk[kb][4 * hf + 1], pk[kb][4 * hf + 2], pk[kb][4 * hf + 3]});
    u32x4_t vf[2][NMT];
    auto load = [&](int r, u32x4_t (&f)[NMT]) {  // r = 2 kb + hf
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const u32x2_t lo = ds_read_tr16(sb + v_roff[mt] + (16 * r) * D * 2);
        const u32x2_t hi = ds_read_tr16(sb + v_roff[mt] + (16 * r + 8) * D * 2);
        f[mt] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
    };
    load(0, vf[0]);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r + 1 < 4) load(r + 1, vf[(r + 1) & 1]);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) o[mt] = mfma32(as_bf16x8(vf[r & 1][mt]), pb[r >> 1][r & 1], o[mt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- pipeline: the K and V tiles of step t+1 are in flight (DMA into buffer 1-P) while tile
  // t computes from buffer P; one barrier per tile. Past the last tile the loads repeat the
  // last tile, so the instruction stream is the same for every step.
  // With masks beyond causal a column may have seen no key yet: its sum is then exactly 0
  // without any underflow, so only columns that have started count for the exact-path test,
  // and a wave none of whose columns sees the tile skips it (it still takes part in the
  // loads and the barrier).
  bool started = MASK == 0;
  auto step = [&](int P, int t, int tn) {
    issue_k(1 - P, tn);
    issue_v(1 - P, tn);
    bool wave_on = true;
    if constexpr (MASK != 0) {
      const bool sees = col_sees(t);
      started = started || sees;
      wave_on = __any(sees);
    }
    if (wave_on) {
      f32x16_t sc[2];
      s_product(P, sc);
      mask_tile(sc, t);
      uint32_t pk[2][8];
      float ls = probs(sc, pk, false);
      const float lt = l_run + ls;
      bool exact = shifted || __any(!(ls <= 0x1p32f));
      // the column sums (lane pairs l, l^32) are only formed when some lane's own sum is
      // small, which happens on a column's first tiles
      if (!exact && __any(started && !(lt >= 0x1p-100f)))
        exact = __any(started && !(lt + xor_shfl(lt, 32) >= 0x1p-100f));
      if (exact) {
        rescale(sc);
        ls = probs(sc, pk, true);
        shifted = true;
      }
      l_run += ls;
      pv_product(P, pk);
    }
    wait_vmem();
    __syncthreads();
  };

  // ---- software-pipelined step of the unmasked variant: S^T of tile t+1 runs on the matrix
  // cores while the VALU does the softmax of tile t (one round of two MFMAs per slice of the
  // probabilities), then O^T += V^T P^T of tile t. K runs one tile ahead of V: at step t,
  // K(t+1) and V(t) are in LDS, K(t+2) and V(t+1) are in flight. sc holds S^T of tile t.
  // (The products and the softmax are independent within a step. Pinning them together
  // instruction by instruction needs more than 256 VGPRs and spills; left to itself the
  // compiler groups the MFMAs ahead of the exponentials. Four accumulator chains for S^T
  // here measured no better than two.)
  constexpr int PPR = 16 / NST;  // probability pairs per lane per S round
  const int t_end = t_hi < ntiles ? t_hi : ntiles;
  auto pstep = [&](int P, int t, f32x16_t (&sc)[2]) {
    const int tk = t + 2 < t_end ? t + 2 : t_end - 1;
    const int tv = t + 1 < t_end ? t + 1 : t_end - 1;
    issue_k(P, tk);      // K(t+2) -> kbuf P (K(t) was consumed by the previous step)
    issue_v(1 - P, tv);  // V(t+1) -> vbuf 1-P
    mask_tile(sc, t);
    // S^T of tile t+1 from K(t+1) in two accumulator chains, in rounds that each also take
    // a slice of tile t's probabilities
    const char* kb = k_lds(1 - P);
    f32x16_t sn[2] = {f32x16_t{}, f32x16_t{}};
    uint32_t pk[2][8];
    float ls4[4] = {0.f, 0.f, 0.f, 0.f};
    u32x4_t kf[2][2];
    auto kload = [&](int r, u32x4_t (&f)[2]) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        f[mt] = *reinterpret_cast<const u32x4_t*>(kb + k_roff[r] + mt * 32 * D * 2);
    };
    kload(0, kf[0]);
#pragma unroll
    for (int r = 0; r < NST; ++r) {
      if (r + 1 < NST) kload(r + 1, kf[(r + 1) & 1]);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) sn[mt] = mfma32(as_bf16x8(kf[r & 1][mt]), qf[r], sn[mt]);
#pragma unroll
      for (int q = 0; q < PPR; ++q) {
        const int pair = r * PPR + q, kk = pair >> 3, j = pair & 7;
        f32x2_t pp = {__builtin_amdgcn_exp2f(sc[kk][2 * j]), __builtin_amdgcn_exp2f(sc[kk][2 * j + 1])};
        const bf16x2_t pb2 = __builtin_convertvector(pp, bf16x2_t);
        pk[kk][j] = __builtin_bit_cast(uint32_t, pb2);
        ls4[j & 3] = __builtin_amdgcn_fdot2_f32_bf16(pb2, one2, ls4[j & 3], false);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    float ls = (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
    const float lt = l_run + ls;
    bool exact = shifted || __any(!(ls <= 0x1p32f));
    if (!exact && __any(!(lt >= 0x1p-100f))) exact = __any(!(lt + xor_shfl(lt, 32) >= 0x1p-100f));
    if (exact) {
      rescale(sc);
      ls = probs(sc, pk, true);
      shifted = true;
    }
    l_run += ls;
    pv_product(P, pk);  // V(t) from vbuf P
    sc[0] = sn[0];
    sc[1] = sn[1];
    wait_vmem();
    __syncthreads();
  };

  if constexpr (MASK == 0) {
    issue_k(0, t_lo);
    issue_v(0, t_lo);
    issue_k(1, t_lo + 1 < t_end ? t_lo + 1 : t_lo);
    fill_omega();
    if (rope_tab) {
      build_rope_table();
      __syncthreads();
    }
    make_q();
    wait_vmem();
    __syncthreads();
    f32x16_t sc[2];
    s_product(0, sc);  // S^T of tile t_lo
    __syncthreads();   // kbuf 0 is refilled by the first step
    int t = t_lo;
    for (; t + 1 < t_end; t += 2) {
      pstep(0, t, sc);
      pstep(1, t + 1, sc);
    }
    if (t < t_end) pstep(0, t, sc);
  } else {
    // visible tiles only; past the last one the loads repeat it (same instruction stream)
    int t = (MASK & 2) ? next_tile(t_first - 1) : t_first;
    issue_k(0, t);
    issue_v(0, t);
    fill_omega();
    if (rope_tab) {
      build_rope_table();
      __syncthreads();
    }
    make_q();
    wait_vmem();
    __syncthreads();
    while (true) {
      const int t1 = next_tile(t);
      step(0, t, t1 < ntiles ? t1 : t);
      if (t1 >= ntiles) break;
      const int t2 = next_tile(t1);
      step(1, t1, t2 < ntiles ? t2 : t1);
      if (t2 >= ntiles) break;
      t = t2;
    }
  }

  // ---- epilogue: O / l -> bf16
  float l_tot = l_run + xor_shfl(l_run, 32);
  if constexpr (PAIR) {
    if (slot >= 0) {
      // Paired schedule: store this part's state (this lane's O rows, then the column's
      // reference m and sum l) with device-coherent 16-byte stores (the partner may run on
      // another XCD), laid out so that each store instruction of a wave writes 1 KB in one
      // piece; then count the part in. The part counted second reads the other one back and
      // merges, the heavy block's own part always as the first operand, so the bits do not
      // depend on which part ends last. The heavy workgroup's part usually ends last, so it
      // looks at the count first: when its partner's part is in, it merges at once and its
      // own part is never stored.
      constexpr int PF = COLS * D + 2 * COLS;  // floats of one part
      constexpr int kCoherent = 16;            // cache policy: sc1 (device-coherent access)
      const __amdgpu_buffer_rsrc_t prs = make_rsrc(a.pair_part + (long)pair * 2 * PF, 2 * PF * 4);
      const int mine = slot * PF * 4, other = (1 - slot) * PF * 4;  // byte offsets of the parts
      const int cw = wave * 32 + l32;  // column inside the block
      auto o_off = [&](int mt, int r4) { return ((((mt * 4 + r4) * 2 + grp) * COLS + cw) * 4) * 4; };
      int partner_in = 0;
      if (slot == 0) {
        if (tid == 0) s_arrived = __hip_atomic_load(a.pair_arrive + pair, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        partner_in = __builtin_amdgcn_readfirstlane(s_arrived);
      }
      if (partner_in == 0) {
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4_t v = {o[mt][4 * r4], o[mt][4 * r4 + 1], o[mt][4 * r4 + 2], o[mt][4 * r4 + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), prs, mine + o_off(mt, r4), 0,
                                                   kCoherent);
          }
        if (grp == 0) {
          const f32x2_t ml = {m_run, l_tot};
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, ml), prs,
                                                mine + (COLS * D + 2 * cw) * 4, 0, kCoherent);
        }
        wait_vmem();
        __syncthreads();
        if (tid == 0)
          s_arrived = __hip_atomic_fetch_add(a.pair_arrive + pair, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(s_arrived) == 0) return;  // the other part merges
      }
      const f32x2_t mlo = __builtin_bit_cast(f32x2_t, __builtin_amdgcn_raw_buffer_load_b64(
          prs, other + (COLS * D + 2 * cw) * 4, 0, kCoherent));
      const float mA = slot == 0 ? m_run : mlo[0], mB = slot == 0 ? mlo[0] : m_run;
      const float lA = slot == 0 ? l_tot : mlo[1], lB = slot == 0 ? mlo[1] : l_tot;
      const float M = fmaxf(mA, mB);
      const float wA = __builtin_amdgcn_exp2f(mA - M), wB = __builtin_amdgcn_exp2f(mB - M);
      l_tot = fmaf(lB, wB, lA * wA);
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        f32x4_t ot[4];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4)
          ot[r4] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
              prs, other + o_off(mt, r4), 0, kCoherent));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float oth = ot[i >> 2][i & 3];
          const float oA = slot == 0 ? o[mt][i] : oth, oB = slot == 0 ? oth : o[mt][i];
          o[mt][i] = fmaf(oB, wB, oA * wA);
        }
      }
    }
  }
  // Output rows go out through LDS: straight from the accumulator layout every store
  // instruction would write 16-byte pieces of 32 different rows; staged, each writes 64 / DCH
  // whole rows. The wave writes its 32 columns as bf16 rows [column][d] (16-byte chunks
  // XOR-swizzled by column) into half of a K tile buffer, which nothing reads after the last
  // step's barrier, and reads them back row by row.
  const float inv = 1.0f / l_tot;
  char* const stg = (wave < 2 ? kbuf0 : kbuf1) + (wave & 1) * (32 * D * 2);
  static_assert(2 * 32 * D * 2 <= KBYTES, "two waves' rows fit one K tile buffer");
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int ch = 4 * mt + r4;  // 16-byte chunk of d = 32 mt + 8 r4 + [0, 8)
      const u32x2_t w = {pack_bf16x2(o[mt][4 * r4 + 0] * inv, o[mt][4 * r4 + 1] * inv),
                         pack_bf16x2(o[mt][4 * r4 + 2] * inv, o[mt][4 * r4 + 3] * inv)};
      *reinterpret_cast<u32x2_t*>(stg + l32 * D * 2 + ((ch ^ (l32 % DCH)) * 16) + 8 * grp) = w;
    }
  }
  __builtin_amdgcn_wave_barrier();
  {
    constexpr int RPI = 64 / DCH;  // rows per store instruction
    const int rl = lane / DCH, ch = lane % DCH;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int c = i * RPI + rl;  // column inside the wave
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(stg + c * D * 2 + ((ch ^ (c % DCH)) * 16));
      const int mc = wcol + c;
      if (mc < ncol) {
        const int p = (int)((unsigned)mc / (unsigned)h);
        const long row = (long)(seq0 + p) * a.H + g * h + (mc - p * h);
        *reinterpret_cast<u32x4_t*>(reinterpret_cast<bf16_t*>(a.out) + row * D + 8 * ch) = val;
      }
    }
  }
  // the light workgroup of a pair runs a second block, whose first DMA refills these buffers
  if constexpr (PAIR) __syncthreads();
  };  // run

  if constexpr (PAIR) {
    // Paired schedule of a one-round dense causal grid: heavy block n_blk - 1 - rh and light
    // block rh of the same (sequence, group) run side by side (block ids i and i + grid/2).
    // The heavy one alone would run most of its tiles without a partner on its CU, so its key
    // tiles are cut at a fixed point s: the heavy workgroup takes [0, s), the light one first
    // takes [s, n_h) of the heavy block and then its own block. s follows from the two tile
    // counts alone (the light workgroup runs at about 0.7 of the heavy one's rate beside it,
    // plus its second start), so both workgroups derive the same cut and the result does not
    // depend on timing: s = ceil(0.55 (n_h + n_l + 2)), the best of 0.5-0.7 measured.
    auto tiles_of = [&](int bk) {
      const int nc = a.T * a.h, c0 = bk * COLS;
      if (c0 >= nc) return 0;
      const int cmax = (c0 + COLS - 1 < nc) ? c0 + COLS - 1 : nc - 1;
      return ((int)((unsigned)cmax / (unsigned)a.h) + 1 + KT - 1) / KT;
    };
    const bool heavy = r < half_r;
    const int rh = heavy ? r : r - half_r;  // the pair's heavy rank; its light block is rh
    const int n_h = tiles_of(a.n_blk - 1 - rh);
    const int n_l = rh + half_r < a.n_blk ? tiles_of(rh) : 0;
    const int cut = n_l > 0 ? min(n_h, (11 * (n_h + n_l + 2) + 19) / 20) : n_h;
    const int pair = (rh * a.B + b) * a.G + g;
    // one copy of the block code: the light workgroup runs it twice (the heavy block's tiles
    // it takes, then its own block)
    const int nphase = (!heavy && cut < n_h) ? 2 : 1;
    for (int ph = 0; ph < nphase; ++ph) {
      const bool own_light = !heavy && ph == nphase - 1;
      const int bk = own_light ? rh : a.n_blk - 1 - rh;
      const int lo = (!heavy && !own_light) ? cut : 0;
      const int hi = heavy ? cut : 0x7fffffff;
      const int sl = own_light ? -1 : (heavy ? (cut < n_h ? 0 : -1) : 1);
      run(bk, lo, hi, pair, sl);
    }
  } else {
    run(blk, 0, 0x7fffffff, -1, -1);
  }
}

template <int D, int MASK, bool CACHE>
static hipError_t launch_t(const PrefillArgs& a, hipStream_t s) {
  const long grid = (long)a.B * a.G * a.n_blk;
  if constexpr (MASK == 0 && !CACHE) {
    if (a.pair_part) {
      hipLaunchKernelGGL((prefill_bf16_kernel<D, 0, false, true>), dim3((unsigned)grid), dim3(256),
                         0, s, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_bf16_kernel<D, MASK, CACHE, false>), dim3((unsigned)grid), dim3(256), 0,
                     s, a);
  return hipGetLastError();
}

template <int D, bool CACHE>
static hipError_t launch_dc(const PrefillArgs& a, hipStream_t s) {
  const int mask = (a.window > 0 ? 1 : 0) | (a.block_mask ? 2 : 0);
  switch (mask) {
    case 1: return launch_t<D, 1, CACHE>(a, s);
    case 2: return launch_t<D, 2, CACHE>(a, s);
    case 3: return launch_t<D, 3, CACHE>(a, s);
    default: return launch_t<D, 0, CACHE>(a, s);
  }
}

template <int D>
static hipError_t launch_d(const PrefillArgs& a, hipStream_t s) {
  return a.cache_lens ? launch_dc<D, true>(a, s) : launch_dc<D, false>(a, s);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, int d, hipStream_t s) {
  if ((long)a.B * a.G * a.n_blk <= 0) return hipSuccess;
  return d == 128 ? launch_d<128>(a, s) : launch_d<64>(a, s);
}

int prefill_bf16_cols_per_block() { return COLS; }

}  // namespace gqa
