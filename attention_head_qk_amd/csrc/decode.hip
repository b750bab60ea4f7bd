// Single-token GQA decode on gfx950: split-KV pass + cross-split combine.
//
// The new token's query (already normalised and rotated, its own K/V already in the cache:
// zhanghao0806.com "Qwen3系列1-理论基础&真实结构", D2-3, the layer writes K/V into the cache
// before attention) attends to every cached row of its sequence. Decode reads the whole
// cache once and does ~4 FLOP per byte, so it is bound by HBM bandwidth (same section: decode
// is memory-bound, prefill compute-bound).
//
// Split pass (fp32; the bf16 passes further down run on matrix cores). A workgroup takes one
// split of a.split keys of one sequence and one KV group (and a chunk of HC of the group's h
// query heads). The K/V cache is token-major
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
  const int k0 = s * a.split;
  if (k0 >= L) return;
  const int k1 = (k0 + a.split < L) ? k0 + a.split : L;

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

// ---------------------------------------------------------------------------- bf16: matrix cores
//
// bf16 split pass on v_mfma_f32_16x16x32_bf16. Per wave, 32 keys at a time:
//   S^T = K Q^T   A = K rows straight from global (lane: key l%16, 8 consecutive d), B = the
//                 group's query heads (one head per column, padded to 16 columns);
//   O^T += V^T P^T  A = V^T, read from the V rows staged in LDS (16-byte DMA) with
//                 ds_read_b64_tr_b16, which hands each lane 4 consecutive keys of one d;
//                 B = P^T, which is the S^T accumulator itself, exponentiated and packed.
// In the 16x16 accumulator lane l owns head l%16, so a head's online softmax lives in the 4
// lanes l%16 + 16q. The reference max only moves when a probability would exceed 2^32 (the
// same lazy rule as the prefill kernel). Each of the 4 waves covers a quarter of the split
// with its own state, keeping two 32-key steps of loads in flight (double-buffered V in LDS,
// K in registers); the states merge through LDS at the end.
// NTV: the V DMA carries the non-temporal hint. V is read in 256-byte row pieces, a pattern
// the hint speeds up (measured 8% on the whole pass over 5 GB of cache) as long as the caches
// do not fit the chip's last-level cache, which would otherwise keep them from one call to the
// next. The K loads never carry it: their pattern (64 bytes from each of 16 rows per
// instruction, forced by the A-operand layout) got slower with it.
namespace {

typedef short i16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: inside every 16-lane block, lane i receives element i%4 of the 8-byte
// values addressed by lanes 4j + i/4 of that block, j = 0..3.
__device__ __forceinline__ u32x2_t ds_read_tr16(const char* lds) {
  typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)const_cast<char*>(lds));
  return __builtin_bit_cast(u32x2_t, v);
}

// s_waitcnt vmcnt(n), expcnt and lgkmcnt left at their maxima (gfx9 encoding: vmcnt bits
// [3:0] and [15:14]).
constexpr int vmcnt_enc(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// XOR swizzle of the 16-byte chunk index of a staged V row: the four rows one transposing
// read touches land on four different chunk pairs, so the read is bank-conflict free.
__device__ __forceinline__ int v_swz(int row) { return 2 * (row & 3); }

}  // namespace

template <int D, int HT, bool NTV>
__global__ __launch_bounds__(256, 2) void decode_split_mfma_kernel(DecodeArgs a) {
  constexpr int KSTEP = D / 32;             // k-steps of S^T
  constexpr int NMT = D / 16;               // 16-row tiles of O^T
  constexpr int SUB = 32;                   // keys per step of a wave
  constexpr int ROWB = D * 2;               // bytes of one staged V row
  constexpr int SUBB = SUB * ROWB;          // one staged V sub-tile
  constexpr int NDMA = SUBB / 1024;         // 1 KB DMA instructions per sub-tile
  constexpr int DCH = D / 8;                // 16-byte chunks per row
  constexpr int NHEAD = 16 * HT;
  static_assert(4 * 16 * D * 4 <= 4 * SUBB, "merge scratch of one head tile fits a V buffer");
  static_assert(HT <= 2, "one merge tile per V buffer");
  // The two V buffers of every wave are separate LDS objects, so the compiler can tell that
  // the DMA into one never feeds reads of the other and keeps its waits exact.
  __shared__ __attribute__((aligned(16))) char vb0[4 * SUBB];
  __shared__ __attribute__((aligned(16))) char vb1[4 * SUBB];
  __shared__ float sm_ml[2][4][NHEAD];

  // grid: x = (group, head tile) fastest, y = split, z = sequence. The G workgroups of one
  // split run side by side and read the same token rows of the cache (one row holds all G
  // groups), which keeps DRAM pages open.
  const int s = blockIdx.y;
  const int b = blockIdx.z;
  const int nht = (a.h + NHEAD - 1) / NHEAD;
  const int g = blockIdx.x / nht;
  const int head0 = (blockIdx.x % nht) * NHEAD;  // first head (inside the group) of this block
  const int L = a.seq_lens[b];
  const int k0 = s * a.split;
  if (k0 >= L) return;
  const int k1 = (k0 + a.split < L) ? k0 + a.split : L;
  const int kpw = a.split / 4;  // keys per wave

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const int h = a.h;
  const float sl2e = a.scale_log2e;

  // ---- Q^T (B operand): column = head head0 + 16 ht + l16, d = 32 st + 8 q4 + [0, 8)
  bf16x8_t qf[HT][KSTEP];
  {
    const bf16_t* qt = reinterpret_cast<const bf16_t*>(a.qt) + ((long)b * a.H + (long)g * h) * D;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      const int hh = head0 + 16 * ht + l16;
#pragma unroll
      for (int st = 0; st < KSTEP; ++st) {
        u32x4_t w = {0u, 0u, 0u, 0u};
        if (hh < h) w = *reinterpret_cast<const u32x4_t*>(qt + (long)hh * D + 32 * st + 8 * q4);
        qf[ht][st] = as_bf16x8(w);
      }
    }
  }

  // ---- buffer descriptors over sequence b's rows of group g; rows >= L read as zero
  const int row_stride = a.G * D * 2;
  const long base_el = ((long)b * a.max_seq * a.G + g) * D;
  const int nrec = (L - 1) * row_stride + D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16_t*>(a.k_cache) + base_el, nrec);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16_t*>(a.v_cache) + base_el, nrec);

  f32x4_t o[HT][NMT];
  float m_run[HT], l_run[HT];
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    m_run[ht] = -INFINITY;
    l_run[ht] = 0.f;
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) o[ht][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  char* const vbw[2] = {vb0 + wave * SUBB, vb1 + wave * SUBB};  // this wave's two V buffers
  const int kw0 = k0 + wave * kpw;
  const int kw1 = (kw0 + kpw < k1) ? kw0 + kpw : k1;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  // Loads of one 32-key step: V rows by DMA into buffer `buf` (instruction n fills rows
  // n * RPD.., lane slot pos of row r receives logical chunk pos ^ v_swz(r)), K rows into
  // A-operand registers (tile tt: key kb + 16 tt + l16, d = 32 st + 8 q4 + [0, 8)).
  // 2 * KSTEP + NDMA = 16 vector-memory instructions per step (D = 128).
  u32x4_t kr[2][2][KSTEP];
  auto issue = [&](int kb, int buf, u32x4_t (&k)[2][KSTEP]) {
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int r = n * (1024 / ROWB) + lane / DCH;
      const int c = (lane % DCH) ^ v_swz(r);
      dma16<NTV ? kNonTemporal : 0>(vrs, vbw[buf] + n * 1024, (kb + r) * row_stride + c * 16, 0);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int st = 0; st < KSTEP; ++st)
        k[tt][st] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
            krs, (kb + 16 * tt + l16) * row_stride + (32 * st + 8 * q4) * 2, 0, 0));
  };

  auto step = [&](int kb, int buf, const u32x4_t (&k)[2][KSTEP], bool more) {
    // ---- S^T: keys (kb + 16 tt + 4 q4 + i) x heads
    f32x4_t sc[2][HT];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KSTEP; ++st) acc = mfma16(as_bf16x8(k[tt][st]), qf[ht][st], acc);
        sc[tt][ht] = acc;
      }
    if (kb + SUB > kw1) {  // the last step of the sequence: keys >= kw1 are not there
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kb + 16 * tt + 4 * q4 + i >= kw1)
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) sc[tt][ht][i] = -INFINITY;
    }
    // ---- probabilities (P^T as the B operand: slots 0-3 from tile 0, 4-7 from tile 1)
    bf16x8_t pb[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
      uint32_t pk[4];
      float ls;
      auto probs = [&]() {
        ls = 0.f;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            f32x2_t pp = {__builtin_amdgcn_exp2f(fmaf(sc[tt][ht][2 * j], sl2e, -m_run[ht])),
                          __builtin_amdgcn_exp2f(fmaf(sc[tt][ht][2 * j + 1], sl2e, -m_run[ht]))};
            const bf16x2_t pb2 = __builtin_convertvector(pp, bf16x2_t);
            pk[2 * tt + j] = __builtin_bit_cast(uint32_t, pb2);
            ls = __builtin_amdgcn_fdot2_f32_bf16(pb2, one2, ls, false);
          }
      };
      probs();
      if (__any(!(ls <= 0x1p32f))) {
        float mx = fmaxf(fmaxf(sc[0][ht][0], sc[0][ht][1]), fmaxf(sc[0][ht][2], sc[0][ht][3]));
        mx = fmaxf(mx, fmaxf(fmaxf(sc[1][ht][0], sc[1][ht][1]), fmaxf(sc[1][ht][2], sc[1][ht][3])));
        mx = fmaxf(mx, xor_shfl(mx, 16));
        mx = fmaxf(mx, xor_shfl(mx, 32)) * sl2e;
        const float m_new = fmaxf(m_run[ht], mx);
        if (m_new != -INFINITY) {  // padded or fully masked heads keep their state
          const float alpha = __builtin_amdgcn_exp2f(m_run[ht] - m_new);
          l_run[ht] *= alpha;
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) o[ht][mt] *= alpha;
          m_run[ht] = m_new;
        }
        probs();
      }
      l_run[ht] += ls;
      pb[ht] = as_bf16x8(u32x4_t{pk[0], pk[1], pk[2], pk[3]});
    }
    // ---- this step's V DMA must have landed: only the next step's NDMA + 2 KSTEP loads may
    // still be outstanding, or none at the last step (vmcnt(0))
    if (more) {
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(NDMA + 2 * KSTEP));
    } else {
      wait_vmem();
    }
    // ---- O^T += V^T P^T; V^T operand: lane (d = 16 mt + l16) gets keys 4 q4 + 0..3 from the
    // first transposing read and 16 + 4 q4 + 0..3 from the second
    const char* vbuf = vbw[buf];
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int r0 = 4 * q4 + (l16 >> 2);
      const int c = 2 * mt + ((l16 & 3) >> 1);
      const int off8 = (l16 & 1) * 8;
      const u32x2_t v0 = ds_read_tr16(vbuf + r0 * ROWB + ((c ^ v_swz(r0)) * 16) + off8);
      const u32x2_t v1 = ds_read_tr16(vbuf + (r0 + 16) * ROWB + ((c ^ v_swz(r0 + 16)) * 16) + off8);
      const bf16x8_t va = as_bf16x8(u32x4_t{v0[0], v0[1], v1[0], v1[1]});
#pragma unroll
      for (int ht = 0; ht < HT; ++ht) o[ht][mt] = mfma16(va, pb[ht], o[ht][mt]);
    }
  };

  // two steps in flight per wave: step u + 1's loads go out before step u computes. Inside
  // the loop every issue is unconditional, so the wait counts the compiler derives for the K
  // registers stay exact (a skipped issue on some path would make it wait for everything).
  const int nsteps = (kw1 - kw0 + SUB - 1) / SUB;
  if (nsteps > 0) issue(kw0, 0, kr[0]);
  int u = 0;
  for (; u + 2 < nsteps; u += 2) {
    issue(kw0 + (u + 1) * SUB, 1, kr[1]);
    step(kw0 + u * SUB, 0, kr[0], true);
    issue(kw0 + (u + 2) * SUB, 0, kr[0]);
    step(kw0 + (u + 1) * SUB, 1, kr[1], true);
  }
  if (u + 1 < nsteps) {
    issue(kw0 + (u + 1) * SUB, 1, kr[1]);
    step(kw0 + u * SUB, 0, kr[0], true);
    step(kw0 + (u + 1) * SUB, 1, kr[1], false);
  } else if (u < nsteps) {
    step(kw0 + u * SUB, 0, kr[0], false);
  }

  // ---- merge the 4 waves' states: sm_ml[0|1][w][head] = (m, l), and the O tile of head
  // tile ht as [w][16][D] floats in V buffer ht (staged V is no longer needed)
  __syncthreads();
#pragma unroll
  for (int ht = 0; ht < HT; ++ht) {
    float lt = l_run[ht] + xor_shfl(l_run[ht], 16);
    lt += xor_shfl(lt, 32);
    const int hh = 16 * ht + l16;
    if (q4 == 0) {
      sm_ml[0][wave][hh] = m_run[ht];
      sm_ml[1][wave][hh] = lt;
    }
    float* sm_o = reinterpret_cast<float*>(ht == 0 ? vb0 : vb1);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[(wave * 16 + l16) * D + 16 * mt + 4 * q4 + i] = o[ht][mt][i];
  }
  __syncthreads();
  const int nh = (h - head0 < NHEAD) ? h - head0 : NHEAD;
  for (int idx = tid; idx < nh * D; idx += 256) {
    const int hh = idx / D, d = idx % D;
    const float* sm_o = reinterpret_cast<const float*>(hh < 16 ? vb0 : vb1);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_ml[0][w][hh]);
    float Ls = 0.f, Os = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = __builtin_amdgcn_exp2f(sm_ml[0][w][hh] - M);  // empty waves: 0
      Ls = fmaf(sm_ml[1][w][hh], wt, Ls);
      Os = fmaf(sm_o[(w * 16 + (hh & 15)) * D + d], wt, Os);
    }
    const long pidx = ((long)b * a.H + (long)g * h + head0 + hh) * a.nsplit + s;
    a.part_o[pidx * D + d] = Os;
    if (d == 0) {
      a.part_ml[2 * pidx] = M;
      a.part_ml[2 * pidx + 1] = Ls;
    }
  }
}

// ------------------------------------------------------ bf16, whole K rows per load (h <= 16)
//
// The split pass for groups of at most 16 query heads with every K load instruction covering
// whole rows (64 lanes x 16 B = 1024 / 2D rows), as the V DMA does, instead of 64 bytes of each
// of 16 rows (measured: 64-sequence decode 824 -> 800 us, the 16-sequence loop's pass 21 ->
// 18 us). Each row (and each query) is cut into NQ = D / 32 interleaved parts: part c holds
// d = 8 (NQ q + c) + [0, 8) for q = 0..3. In S^T = K Q^T a row of A is one (key, part) pair,
// m = NQ k + c, so one product covers 16 / NQ keys and the 4 NQ lanes that hold one key read
// its 2D contiguous bytes; a column of B is one (head, part) pair, n = NQ j + c', for HPM =
// 16 / NQ heads of the group. Entry (m, n) is then the dot product of part c of key k with
// part c' of head j: the entries with c = c' are partial scores, summed over the NQ adjacent
// lanes of a head by DPP, and the others are dropped. Groups of more than HPM heads take NHQ
// such products per 32 keys, one per set of HPM heads; column n = NQ j + c' then follows head
// (c' mod NHQ) HPM + j from the scores on, so the softmax, P^T and O^T columns cover every
// head once or more. The rest is the kernel above: V by DMA with transposing reads, the lazy
// softmax reference, two steps in flight per wave, and the 4 waves' states merged through LDS.
namespace {

// XOR swizzle of the 16-byte chunk index of a staged V row for the key order of this kernel:
// the four rows one 16-lane block of a transposing read addresses differ in bits 2-3 of the
// row (d = 128) or in bits 0 and 3 (d = 64), and land on four different chunk pairs.
template <int D>
__device__ __forceinline__ int v_swz_rows(int row) {
  return D == 128 ? 2 * ((row >> 2) & 3) : 2 * ((row & 1) | ((row >> 2) & 2));
}

}  // namespace

template <int D, int NHQ, bool NTV>
__global__ __launch_bounds__(256, 2) void decode_split_rows_kernel(DecodeArgs a) {
  constexpr int NQ = D / 32;       // parts of a row
  constexpr int KPM = 16 / NQ;     // keys per S^T product
  constexpr int HPM = 16 / NQ;     // heads per S^T product
  constexpr int KQ = 4 / NQ;       // keys per lane per S^T product
  constexpr int NMF = 32 / KPM;    // S^T products per 32-key step
  constexpr int NMT = D / 16;      // 16-row tiles of O^T
  constexpr int SUB = 32;          // keys per step of a wave
  constexpr int ROWB = D * 2;      // bytes of one row
  constexpr int SUBB = SUB * ROWB; // one staged V sub-tile
  constexpr int NDMA = SUBB / 1024;
  constexpr int DCH = D / 8;
  constexpr int NLOAD = NDMA + NMF;  // vector-memory instructions per step
  static_assert(4 * 16 * D * 4 <= 4 * SUBB, "merge scratch fits a V buffer");
  static_assert(NHQ >= 1 && NHQ * HPM <= 16 && NHQ <= NQ, "at most 16 heads, each in a column");
  __shared__ __attribute__((aligned(16))) char vb0[4 * SUBB];
  __shared__ __attribute__((aligned(16))) char vb1[4 * SUBB];
  __shared__ float sm_ml[2][4][16];

  // grid: x = group, y = split, z = sequence (as above)
  const int g = blockIdx.x;
  const int s = blockIdx.y;
  const int b = blockIdx.z;
  const int L = a.seq_lens[b];
  const int k0 = s * a.split;
  if (k0 >= L) return;
  const int k1 = (k0 + a.split < L) ? k0 + a.split : L;
  const int kpw = a.split / 4;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const int part = l16 % NQ;  // the part of its key (A) or head (B) this lane holds
  const int hd = l16 / NQ;    // its key inside a product (A), its head inside a set (B)
  const int jq = part % NHQ;  // the head set of this lane's column from the scores on
  const int head = jq * HPM + hd;  // and its head
  const int h = a.h;
  const float sl2e = a.scale_log2e;

  // ---- Q^T (B operands, one per head set): column l16 = (head t HPM + hd, part)
  bf16x8_t qf[NHQ];
  {
    const bf16_t* qt = reinterpret_cast<const bf16_t*>(a.qt) + ((long)b * a.H + (long)g * h) * D;
#pragma unroll
    for (int t = 0; t < NHQ; ++t) {
      const int hh = t * HPM + hd;
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (hh < h) w = *reinterpret_cast<const u32x4_t*>(qt + (long)hh * D + 8 * (NQ * q4 + part));
      qf[t] = as_bf16x8(w);
    }
  }

  // ---- buffer descriptors over sequence b's rows of group g; rows >= L read as zero
  const int row_stride = a.G * D * 2;
  const long base_el = ((long)b * a.max_seq * a.G + g) * D;
  const int nrec = (L - 1) * row_stride + D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(reinterpret_cast<const bf16_t*>(a.k_cache) + base_el, nrec);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(reinterpret_cast<const bf16_t*>(a.v_cache) + base_el, nrec);

  f32x4_t o[NMT];
  float m_run = -INFINITY, l_run = 0.f;
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) o[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  char* const vbw[2] = {vb0 + wave * SUBB, vb1 + wave * SUBB};
  const int kw0 = k0 + wave * kpw;
  const int kw1 = (kw0 + kpw < k1) ? kw0 + kpw : k1;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  // key (inside a step) of probability slot e of this lane: product e / KQ, its key
  // KQ q4 + e % KQ
  auto key_of = [&](int e) { return KPM * (e / KQ) + KQ * q4 + e % KQ; };

  // Loads of one 32-key step: V rows by DMA (as above, with this kernel's swizzle) and, for
  // product mi, K row kb + KPM mi + hd, part `part` into A-operand registers.
  u32x4_t kr[2][NMF];
  auto issue = [&](int kb, int buf, u32x4_t (&k)[NMF]) {
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int r = n * (1024 / ROWB) + lane / DCH;
      const int c = (lane % DCH) ^ v_swz_rows<D>(r);
      dma16<NTV ? kNonTemporal : 0>(vrs, vbw[buf] + n * 1024, (kb + r) * row_stride + c * 16, 0);
    }
#pragma unroll
    for (int mi = 0; mi < NMF; ++mi)
      k[mi] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
          krs, (kb + KPM * mi + hd) * row_stride + (NQ * q4 + part) * 16, 0, 0));
  };

  auto step = [&](int kb, int buf, const u32x4_t (&k)[NMF], bool more) {
    // ---- scores of keys kb + key_of(e), e = 0..7, for this lane's head (the same in the
    // lanes of its column across q4). In a product's result lane (q4, n) slot i is row
    // 4 q4 + i: key KQ q4 + i / NQ, part i % NQ; the slots of the lane's own part are the
    // partial scores of head t HPM + hd.
    float sc[8];
#pragma unroll
    for (int t = 0; t < NHQ; ++t)
#pragma unroll
      for (int mi = 0; mi < NMF; ++mi) {
        const f32x4_t acc = mfma16(as_bf16x8(k[mi]), qf[t], f32x4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int u = 0; u < KQ; ++u) {
          float v = acc[NQ * u];
#pragma unroll
          for (int c = 1; c < NQ; ++c) v = part == c ? acc[NQ * u + c] : v;
          v = dpp_add<0xB1>(v);                 // + part c ^ 1
          if (NQ == 4) v = dpp_add<0x4E>(v);    // + parts c ^ 2, c ^ 3
          sc[KQ * mi + u] = (t == 0 || jq == t) ? v : sc[KQ * mi + u];
        }
      }
    if (kb + SUB > kw1) {  // the last step of the sequence: keys >= kw1 are not there
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (kb + key_of(e) >= kw1) sc[e] = -INFINITY;
    }
    // ---- probabilities (P^T as the B operand: slot e is key key_of(e))
    uint32_t pk[4];
    float ls;
    auto probs = [&]() {
      ls = 0.f;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        f32x2_t pp = {__builtin_amdgcn_exp2f(fmaf(sc[2 * p], sl2e, -m_run)),
                      __builtin_amdgcn_exp2f(fmaf(sc[2 * p + 1], sl2e, -m_run))};
        const bf16x2_t pb2 = __builtin_convertvector(pp, bf16x2_t);
        pk[p] = __builtin_bit_cast(uint32_t, pb2);
        ls = __builtin_amdgcn_fdot2_f32_bf16(pb2, one2, ls, false);
      }
    };
    probs();
    if (__any(!(ls <= 0x1p32f))) {
      float mx = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sc[e]);
      mx = fmaxf(mx, xor_shfl(mx, 16));
      mx = fmaxf(mx, xor_shfl(mx, 32)) * sl2e;
      const float m_new = fmaxf(m_run, mx);
      if (m_new != -INFINITY) {  // padded or fully masked heads keep their state
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) o[mt] *= alpha;
        m_run = m_new;
      }
      probs();
    }
    l_run += ls;
    const bf16x8_t pb = as_bf16x8(u32x4_t{pk[0], pk[1], pk[2], pk[3]});
    // ---- this step's V DMA must have landed: only the next step's loads may be outstanding
    if (more) {
      __builtin_amdgcn_s_waitcnt(vmcnt_enc(NLOAD));
    } else {
      wait_vmem();
    }
    // ---- O^T += V^T P^T; V^T operand: lane (d = 16 mt + l16) gets the keys of slots 0-3 from
    // the first transposing read and of slots 4-7 from the second (addressing lane 4j + r of a
    // 16-lane block supplies slot j (+4), d = 16 mt + 4 r + [0, 4))
    const char* vbuf = vbw[buf];
    const int r0 = key_of(l16 >> 2), r1 = key_of((l16 >> 2) + 4);
#pragma unroll
    for (int mt = 0; mt < NMT; ++mt) {
      const int c = 2 * mt + ((l16 & 3) >> 1);
      const int off8 = (l16 & 1) * 8;
      const u32x2_t v0 = ds_read_tr16(vbuf + r0 * ROWB + ((c ^ v_swz_rows<D>(r0)) * 16) + off8);
      const u32x2_t v1 = ds_read_tr16(vbuf + r1 * ROWB + ((c ^ v_swz_rows<D>(r1)) * 16) + off8);
      const bf16x8_t va = as_bf16x8(u32x4_t{v0[0], v0[1], v1[0], v1[1]});
      o[mt] = mfma16(va, pb, o[mt]);
    }
  };

  const int nsteps = (kw1 - kw0 + SUB - 1) / SUB;
  if (nsteps > 0) issue(kw0, 0, kr[0]);
  int u = 0;
  for (; u + 2 < nsteps; u += 2) {
    issue(kw0 + (u + 1) * SUB, 1, kr[1]);
    step(kw0 + u * SUB, 0, kr[0], true);
    issue(kw0 + (u + 2) * SUB, 0, kr[0]);
    step(kw0 + (u + 1) * SUB, 1, kr[1], true);
  }
  if (u + 1 < nsteps) {
    issue(kw0 + (u + 1) * SUB, 1, kr[1]);
    step(kw0 + u * SUB, 0, kr[0], true);
    step(kw0 + (u + 1) * SUB, 1, kr[1], false);
  } else if (u < nsteps) {
    step(kw0 + u * SUB, 0, kr[0], false);
  }

  // ---- merge the 4 waves' states: (m, l) per head and the O columns as [w][head][D] floats
  // in V buffer 0, from the first column of each head (part < NHQ)
  __syncthreads();
  {
    float lt = l_run + xor_shfl(l_run, 16);
    lt += xor_shfl(lt, 32);
    if (q4 == 0 && part < NHQ) {
      sm_ml[0][wave][head] = m_run;
      sm_ml[1][wave][head] = lt;
    }
    float* sm_o = reinterpret_cast<float*>(vb0);
    if (part < NHQ)
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sm_o[(wave * 16 + head) * D + 16 * mt + 4 * q4 + i] = o[mt][i];
  }
  __syncthreads();
  const float* sm_o = reinterpret_cast<const float*>(vb0);
  for (int idx = tid; idx < h * D; idx += 256) {
    const int hh = idx / D, d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm_ml[0][w][hh]);
    float Ls = 0.f, Os = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = __builtin_amdgcn_exp2f(sm_ml[0][w][hh] - M);  // empty waves: 0
      Ls = fmaf(sm_ml[1][w][hh], wt, Ls);
      Os = fmaf(sm_o[(w * 16 + hh) * D + d], wt, Os);
    }
    const long pidx = ((long)b * a.H + (long)g * h + hh) * a.nsplit + s;
    a.part_o[pidx * D + d] = Os;
    if (d == 0) {
      a.part_ml[2 * pidx] = M;
      a.part_ml[2 * pidx + 1] = Ls;
    }
  }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float sw[kMaxCombineSplits];
  __shared__ float s_inv;
  combine_one<T, D>(a, blockIdx.x, blockIdx.y, threadIdx.x, sw, s_inv);
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

template <int D, int HT>
static hipError_t launch_split_mfma(const DecodeArgs& a, hipStream_t s) {
  const int nht = (a.h + 16 * HT - 1) / (16 * HT);
  const dim3 grid(a.G * nht, a.nsplit, a.B);
  if (a.stream_v)
    hipLaunchKernelGGL((decode_split_mfma_kernel<D, HT, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_mfma_kernel<D, HT, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int D, int NHQ>
static hipError_t launch_split_rows(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.G, a.nsplit, a.B);
  if (a.stream_v)
    hipLaunchKernelGGL((decode_split_rows_kernel<D, NHQ, true>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((decode_split_rows_kernel<D, NHQ, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// Whole-row K loads with NHQ sets of 16 / (D / 32) heads for h <= 16. Four sets (d = 128,
// h > 8) take four times the score products of the tiled kernel, which only pays where the
// pass streams a large cache (measured: 64 sequences of up to 32768 keys 491 -> 476 us; 16
// sequences of about 1200 keys 13.8 -> 15.1 us); otherwise, and for h > 16, the tiled kernel.
template <int D>
static hipError_t split_mfma_d(const DecodeArgs& a, hipStream_t s) {
  constexpr int HPM = 16 / (D / 32);
  if (a.h <= HPM) return launch_split_rows<D, 1>(a, s);
  if (a.h <= 2 * HPM) return launch_split_rows<D, 2>(a, s);
  if constexpr (D == 128)
    if (a.h <= 16 && a.stream_v) return launch_split_rows<D, 4>(a, s);
  return a.h <= 16 ? launch_split_mfma<D, 1>(a, s) : launch_split_mfma<D, 2>(a, s);
}

hipError_t launch_decode_split(const DecodeArgs& a, int d, bool bf16, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (bf16) return d == 128 ? split_mfma_d<128>(a, s) : split_mfma_d<64>(a, s);
  return d == 128 ? split_td<float, 128>(a, s) : split_td<float, 64>(a, s);
}

hipError_t launch_decode_combine(const DecodeArgs& a, int d, bool bf16, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  if (bf16) return d == 128 ? combine_td<bf16_t, 128>(a, s) : combine_td<bf16_t, 64>(a, s);
  return d == 128 ? combine_td<float, 128>(a, s) : combine_td<float, 64>(a, s);
}

}  // namespace gqa
