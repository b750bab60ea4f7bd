// Host side of the libgqa C ABI (include/gqa.h): argument checks, workspace layout, launch
// geometry and the dtype / head-dim dispatch. Every check runs before the first HIP call, so
// a rejected call enqueues nothing and touches no device.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <new>

#include "gqa.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxHeads = 4096;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t elem_size(int dtype) { return dtype == GQA_BF16 ? 2 : 4; }

bool dtype_ok(int dtype) { return dtype == GQA_F32 || dtype == GQA_BF16; }

// Keys per split of the decode pass. Splits of 1024 keys stream long caches with few
// partials; when that would launch fewer than kDecodeMinBlocks workgroups (8 per CU over the
// longest possible caches) the split is halved, down to kDecodeSplitMin, so that short caches
// still spread over the chip. Only the host-visible sizes enter (seq_lens live on the device).
constexpr long kDecodeMinBlocks = 2048;

// Largest grid y or z dimension of a launch: the decode passes and the fp32 prefill put the
// sequence index there.
constexpr int kMaxGridYZ = 65535;

// Caches whose K and V allocations together exceed this are streamed (V read non-temporally):
// twice the 256 MB last-level cache, so a loop over a cache that fits keeps finding it there.
// Measured: 64 sequences over a 8.6 GB allocation (5 GB read) 893 -> 826 us for the split
// pass; 16 sequences over 268 MB (77 MB read per step) 20.0 -> 20.8 us with the hint.
constexpr double kDecodeStreamBytes = 512.0 * 1024 * 1024;

int decode_split_len(int B, int H, int G, int max_seq) {
  const long nht = (H / G + 31) / 32;  // head tiles of one group in the bf16 split pass
  int split = gqa::kDecodeSplit;
  while (split > gqa::kDecodeSplitMin &&
         (long)B * G * nht * (((long)max_seq + split - 1) / split) < kDecodeMinBlocks)
    split /= 2;
  return split;
}

// Paired schedule of the bf16 prefill (one-round dense causal grids of at most
// kMaxPairGrid workgroups): pairs of column blocks, and the floats of one partial state
constexpr long kMaxPairGrid = 512;
long prefill_pairs(int B, int T, int H, int G) {
  if (B <= 0 || T <= 0 || G <= 0 || H % G != 0) return 0;
  const long cpb = gqa::prefill_bf16_cols_per_block();
  const long n_blk = ((long)T * (H / G) + cpb - 1) / cpb;
  const long grid = (long)B * G * n_blk;
  return grid <= kMaxPairGrid ? (long)B * G * ((n_blk + 1) / 2) : 0;
}
size_t prefill_part_floats(int d) {
  const size_t cpb = (size_t)gqa::prefill_bf16_cols_per_block();
  return cpb * d + 2 * cpb;
}

int decode_nsplit(int B, int H, int G, int max_seq) {
  if (max_seq <= 0) return 0;
  const int split = decode_split_len(B, H, G, max_seq);
  return (max_seq + split - 1) / split;
}

// Checks shared by every entry point. Returns GQA_OK or the first failure.
gqa_status check_heads(int H, int G, int d) {
  if (H <= 0 || G <= 0 || H > kMaxHeads || G > kMaxHeads || H % G != 0) return GQA_EINVAL;
  if (d != 64 && d != 128) return GQA_ENOTSUP;
  return GQA_OK;
}

// The dtype field as the caller stored it. A C caller may have put any int there, and
// loading an enum object that holds a value outside the enumeration is undefined in C++, so
// its bytes are read as an int; once this check passed, p->dtype holds GQA_F32 or GQA_BF16.
int dtype_bits(const gqa_params* p) {
  static_assert(sizeof(p->dtype) == sizeof(int), "gqa_dtype is int-sized");
  int v;
  std::memcpy(&v, &p->dtype, sizeof v);
  return v;
}

gqa_status check_params(const gqa_params* p) {
  if (!p) return GQA_EINVAL;
  if (!dtype_ok(dtype_bits(p))) return GQA_ENOTSUP;
  if (!(p->eps >= 0.f) || !std::isfinite(p->eps)) return GQA_EINVAL;
  if (!(p->scale >= 0.f) || !std::isfinite(p->scale)) return GQA_EINVAL;
  if (!(p->rope_theta >= 0.0) || !std::isfinite(p->rope_theta)) return GQA_EINVAL;
  if (!aligned(p->q_norm_w, 16) || !aligned(p->k_norm_w, 16)) return GQA_EINVAL;
  return GQA_OK;
}

bool tensor_ok(const void* t) { return t != nullptr && aligned(t, 16); }
bool opt_tensor_ok(const void* t) { return aligned(t, 16); }
bool opt_int_ok(const void* t) { return aligned(t, 4); }
bool int_ok(const void* t) { return t != nullptr && aligned(t, 4); }

float eff_scale(const gqa_params* p, int d) {
  return p->scale > 0.f ? p->scale : (float)(1.0 / std::sqrt((double)d));
}

// RoPE frequencies into the kernel arguments: the caller's table when given, else
// theta^(-2j/d) computed here in fp64.
template <typename Args>
void fill_rope(Args& a, const gqa_params* p, int d) {
  a.use_rope = (p->rope_inv_freq || p->rope_theta > 0.0) ? 1 : 0;
  for (int j = 0; j < gqa::kMaxHalfD; ++j) {
    double w = 0.0;
    if (a.use_rope && j < d / 2)
      w = p->rope_inv_freq ? p->rope_inv_freq[j] : std::pow(p->rope_theta, -2.0 * j / d);
    a.omega[j] = w;
  }
}

// A caller's frequency table must hold d/2 finite values.
gqa_status check_rope_table(const gqa_params* p, int d) {
  if (!p->rope_inv_freq) return GQA_OK;
  for (int j = 0; j < d / 2; ++j)
    if (!std::isfinite(p->rope_inv_freq[j])) return GQA_EINVAL;
  return GQA_OK;
}

gqa_status from_hip(hipError_t e) { return e == hipSuccess ? GQA_OK : GQA_EHIP; }

// Mask variants of a prefill whose key indices run over [0, n_keys): window needs the causal
// mask; the block mask needs whole rows over ceil(n_keys / 64) key blocks; both are bf16 only.
gqa_status check_masks(const gqa_params* p, int causal, long long n_keys) {
  if (p->window < 0 || (p->window > 0 && !causal)) return GQA_EINVAL;
  if (p->block_mask) {
    if (!aligned(p->block_mask, 4) || p->block_mask_words <= 0) return GQA_EINVAL;
    if ((long long)p->block_mask_words * 32 * 64 < n_keys) return GQA_EINVAL;
  }
  if ((p->window > 0 || p->block_mask) && p->dtype != GQA_BF16) return GQA_ENOTSUP;
  return GQA_OK;
}

template <typename Args>
void fill_masks(Args& a, const gqa_params* p) {
  a.window = p->window;
  a.block_mask = p->block_mask;
  a.bm_words = p->block_mask ? p->block_mask_words : 0;
}

// Records the caller's optional profiling event on the stream.
hipError_t mark(void* ev, hipStream_t s) {
  return ev ? hipEventRecord(reinterpret_cast<hipEvent_t>(ev), s) : hipSuccess;
}

// Host checks of a decode call (gqa_decode and the decode graph).
gqa_status decode_check(const void* q, void* k_cache, void* v_cache, const int32_t* seq_lens,
                        void* out, int B, int H, int G, int d, int max_seq, const gqa_params* p) {
  gqa_status st = check_params(p);
  if (st != GQA_OK) return st;
  if ((st = check_heads(H, G, d)) != GQA_OK) return st;
  if ((st = check_rope_table(p, d)) != GQA_OK) return st;
  if (B < 0 || max_seq < 0) return GQA_EINVAL;
  if (p->window != 0 || p->block_mask) return GQA_ENOTSUP;
  if (B == 0) return GQA_OK;
  if (max_seq == 0) return GQA_EINVAL;
  if (B > kMaxGridYZ) return GQA_ENOTSUP;
  // one sequence's cache rows are addressed with 32-bit byte offsets, and the combine pass
  // merges at most kMaxCombineSplits splits per sequence
  if ((long long)max_seq * G * d * (long long)elem_size(p->dtype) > 0x7fffffffLL ||
      decode_nsplit(B, H, G, max_seq) > gqa::kMaxCombineSplits)
    return GQA_ENOTSUP;
  if (!tensor_ok(q) || !tensor_ok(k_cache) || !tensor_ok(v_cache) || !tensor_ok(out))
    return GQA_EINVAL;
  if (!seq_lens || !opt_int_ok(seq_lens) || !opt_int_ok(p->positions)) return GQA_EINVAL;
  if ((p->k_new == nullptr) != (p->v_new == nullptr)) return GQA_EINVAL;
  if (!opt_tensor_ok(p->k_new) || !opt_tensor_ok(p->v_new)) return GQA_EINVAL;
  const size_t need = gqa_workspace_bytes(GQA_OP_DECODE, B, max_seq, H, G, d, p->dtype);
  if (!p->workspace || !aligned(p->workspace, 16) || p->workspace_bytes < need)
    return GQA_EWORKSPACE;
  return GQA_OK;
}

// The kernel arguments of one decode step (prologue with the optional append; split and
// combine passes). With `advance` (a generation-loop step) every sequence first gains its new
// token: the prologue takes min(len_in[b] + 1, max_seq) as the length and writes it to
// lens_step, the split and combine passes read it there, and the combine pass copies it into
// seq_lens -- no launch of its own for the advance. len_in is seq_lens, or the previous
// step's lens_step inside a multi-step graph.
void decode_args(const void* q, void* k_cache, void* v_cache, const int32_t* seq_lens,
                 void* out, int B, int H, int G, int d, int max_seq, const gqa_params* p,
                 bool advance, const int32_t* len_in, int32_t* lens_step, gqa::PrologueArgs& pa,
                 gqa::DecodeArgs& da) {
  const size_t es = elem_size(p->dtype);
  const int split = decode_split_len(B, H, G, max_seq);
  const int ns = decode_nsplit(B, H, G, max_seq);
  char* ws = static_cast<char*>(p->workspace);
  void* qt = ws;
  float* part_o = reinterpret_cast<float*>(ws + align_up((size_t)B * H * d * es));
  float* part_ml = reinterpret_cast<float*>(reinterpret_cast<char*>(part_o) +
                                            align_up((size_t)B * H * ns * d * 4));

  pa = gqa::PrologueArgs{};
  pa.q = q;
  pa.k = p->k_new;
  pa.v = p->v_new;
  pa.q_out = qt;
  pa.k_out = k_cache;
  pa.v_out = v_cache;
  pa.positions = p->positions;
  pa.seq_lens = advance ? len_in : seq_lens;
  pa.gq = p->q_norm_w;
  pa.gk = p->k_norm_w;
  pa.eps = p->eps;
  pa.decode = 1;
  pa.B = B;
  pa.T = 1;
  pa.H = H;
  pa.G = G;
  pa.max_seq = max_seq;
  pa.lens_out = advance ? lens_step : nullptr;
  fill_rope(pa, p, d);

  da = gqa::DecodeArgs{};
  da.qt = qt;
  da.k_cache = k_cache;
  da.v_cache = v_cache;
  da.seq_lens = advance ? lens_step : seq_lens;
  da.lens_commit = advance ? const_cast<int32_t*>(seq_lens) : nullptr;
  da.part_o = part_o;
  da.part_ml = part_ml;
  da.out = out;
  da.B = B;
  da.H = H;
  da.G = G;
  da.h = H / G;
  da.max_seq = max_seq;
  da.nsplit = ns;
  da.split = split;
  da.stream_v = 2.0 * B * max_seq * G * d * (double)es > kDecodeStreamBytes;
  da.scale_log2e = (float)((double)eff_scale(p, d) * 1.4426950408889634074);
}

// The two per-step length buffers of the decode workspace (after q~ and the partials):
// a multi-step graph alternates between them, a single step uses the first.
int32_t* decode_lens_ws(const gqa_params* p, int B, int H, int G, int d, int max_seq, int which) {
  const size_t es = elem_size(p->dtype);
  const int ns = decode_nsplit(B, H, G, max_seq);
  char* ws = static_cast<char*>(p->workspace);
  const size_t off = align_up((size_t)B * H * d * es) + align_up((size_t)B * H * ns * d * 4) +
                     align_up((size_t)B * H * ns * 2 * 4) + (size_t)which * align_up((size_t)B * 4);
  return reinterpret_cast<int32_t*>(ws + off);
}

// The decode step's three launches on `stream`; `prof` records the caller's events around the
// split pass; `advance` as in decode_args.
gqa_status decode_enqueue(const void* q, void* k_cache, void* v_cache, const int32_t* seq_lens,
                          void* out, int B, int H, int G, int d, int max_seq,
                          const gqa_params* p, hipStream_t stream, bool prof,
                          bool advance = false) {
  gqa_status st;
  const bool bf16 = p->dtype == GQA_BF16;
  gqa::PrologueArgs pa;
  gqa::DecodeArgs da;
  decode_args(q, k_cache, v_cache, seq_lens, out, B, H, G, d, max_seq, p, advance, seq_lens,
              decode_lens_ws(p, B, H, G, d, max_seq, 0), pa, da);
  if ((st = from_hip(gqa::launch_prologue(pa, B, d, bf16, stream))) != GQA_OK) return st;
  if (prof && (st = from_hip(mark(p->prof_start, stream))) != GQA_OK) return st;
  if ((st = from_hip(gqa::launch_decode_split(da, d, bf16, stream))) != GQA_OK) return st;
  if (prof && (st = from_hip(mark(p->prof_stop, stream))) != GQA_OK) return st;
  return from_hip(gqa::launch_decode_combine(da, d, bf16, stream));
}

// `steps` generation-loop steps (multi-step decode graph): step i reads and writes its own
// input and output blocks. Between two steps one launch runs step i's combine beside step
// i + 1's prologue (their data are disjoint; see the fused kernel), so a graph of S steps is
// 2 S + 1 kernels. The step lengths alternate between the two workspace buffers: step i + 1's
// prologue reads step i's lengths from one while writing its own to the other.
gqa_status decode_steps_enqueue(const void* q, void* k_cache, void* v_cache, int32_t* seq_lens,
                                void* out, int B, int H, int G, int d, int max_seq, int steps,
                                const gqa_params* p, hipStream_t stream) {
  gqa_status st;
  const bool bf16 = p->dtype == GQA_BF16;
  const size_t es = elem_size(p->dtype);
  const size_t q_step = (size_t)B * H * d * es, kv_step = (size_t)B * G * d * es;
  int32_t* lens[2] = {decode_lens_ws(p, B, H, G, d, max_seq, 0),
                      decode_lens_ws(p, B, H, G, d, max_seq, 1)};
  auto step_args = [&](int i, gqa::PrologueArgs& pa, gqa::DecodeArgs& da) {
    gqa_params ps = *p;
    ps.k_new = static_cast<const char*>(p->k_new) + i * kv_step;
    ps.v_new = static_cast<const char*>(p->v_new) + i * kv_step;
    if (p->positions) ps.positions = p->positions + (size_t)i * B;
    decode_args(static_cast<const char*>(q) + i * q_step, k_cache, v_cache, seq_lens,
                static_cast<char*>(out) + i * q_step, B, H, G, d, max_seq, &ps, true,
                i == 0 ? seq_lens : lens[(i - 1) & 1], lens[i & 1], pa, da);
  };
  gqa::PrologueArgs pa, pn;
  gqa::DecodeArgs da, dn;
  step_args(0, pa, da);
  if ((st = from_hip(gqa::launch_prologue(pa, B, d, bf16, stream))) != GQA_OK) return st;
  for (int i = 0; i < steps; ++i) {
    if ((st = from_hip(gqa::launch_decode_split(da, d, bf16, stream))) != GQA_OK) return st;
    if (i + 1 == steps) return from_hip(gqa::launch_decode_combine(da, d, bf16, stream));
    step_args(i + 1, pn, dn);
    if ((st = from_hip(gqa::launch_decode_combine_prologue(da, pn, d, bf16, stream))) != GQA_OK)
      return st;
    da = dn;
  }
  return GQA_OK;
}

// most decode steps one graph records
constexpr int kMaxGraphSteps = 256;

// ---- scratch of gqa_decode_noalloc: one fixed device array per GPU, so that entry point
// allocates nothing. In host code `scratch` names a host-side stand-in, never the device
// memory: its device address comes from hipGetSymbolAddress, taken once per device (with the
// device current) on the first call there and kept in g_scratch_ptr.
constexpr size_t kScratchBytes = (size_t)GQA_DECODE_NOALLOC_MAX_BYTES;
__device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array.
gqa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GQA_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return GQA_ENOTSUP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GQA_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

void gqa_params_init(gqa_params* p) {
  if (!p) return;
  p->dtype = GQA_BF16;
  p->q_norm_w = nullptr;
  p->k_norm_w = nullptr;
  p->eps = 1e-6f;
  p->rope_theta = 1e6;
  p->scale = 0.f;
  p->cu_seqlens = nullptr;
  p->k_out = nullptr;
  p->k_new = nullptr;
  p->v_new = nullptr;
  p->positions = nullptr;
  p->workspace = nullptr;
  p->workspace_bytes = 0;
  p->stream = nullptr;
  p->prof_start = nullptr;
  p->prof_stop = nullptr;
  p->window = 0;
  p->block_mask = nullptr;
  p->block_mask_words = 0;
  p->rope_inv_freq = nullptr;
}

const char* gqa_status_str(gqa_status s) {
  switch (s) {
    case GQA_OK: return "GQA_OK: success";
    case GQA_EINVAL: return "GQA_EINVAL: invalid argument";
    case GQA_ENOTSUP: return "GQA_ENOTSUP: unsupported head dim or dtype";
    case GQA_EWORKSPACE: return "GQA_EWORKSPACE: workspace missing or too small";
    case GQA_EHIP: return "GQA_EHIP: HIP launch error";
  }
  return "unknown gqa_status";
}

gqa_status gqa_rope_freq_table(int kind, int d, double theta, double alpha, double train_len,
                               double infer_len, double scale, double* out) {
  if (!out || d < 2 || d > 2 * gqa::kMaxHalfD || d % 2 != 0) return GQA_EINVAL;
  if (!(theta > 0.0) || !std::isfinite(theta)) return GQA_EINVAL;
  const int half = d / 2;
  double base = theta;  // the base whose table is taken before any per-frequency factor
  switch (kind) {
    case GQA_ROPE_BASE:
      break;
    case GQA_ROPE_LINEAR:
      if (!(alpha > 0.0) || !std::isfinite(alpha)) return GQA_EINVAL;
      break;
    case GQA_ROPE_YARN:
      if (!(train_len > 0.0) || !(infer_len > 0.0) || !std::isfinite(train_len) ||
          !std::isfinite(infer_len) || !std::isfinite(scale))
        return GQA_EINVAL;
      break;
    case GQA_ROPE_NTK:
      if (!(alpha > 0.0) || !std::isfinite(alpha) || d <= 2) return GQA_EINVAL;
      // theta * alpha^(d / (d - 2)): the exponent makes the last frequency exactly 1/alpha
      // of its unscaled value
      base = theta * std::pow(alpha, (double)d / (double)(d - 2));
      if (!std::isfinite(base) || !(base > 0.0)) return GQA_EINVAL;
      break;
    default:
      return GQA_EINVAL;
  }
  // past the training length the YaRN-named rule tilts the table linearly in j
  const double tilt = (kind == GQA_ROPE_YARN && infer_len > train_len)
                          ? scale * std::log2(infer_len / train_len)
                          : 0.0;
  for (int j = 0; j < half; ++j) {
    const double frac = 2.0 * j / d;
    double w = std::pow(base, -frac);
    if (kind == GQA_ROPE_LINEAR) w /= alpha;
    if (kind == GQA_ROPE_YARN) w *= 1.0 - tilt * frac;
    out[j] = w;
  }
  return GQA_OK;
}

int gqa_decode_split_keys(int B, int H, int G, int max_seq) {
  if (B <= 0 || max_seq <= 0 || H <= 0 || G <= 0 || H % G != 0) return 0;
  return decode_split_len(B, H, G, max_seq);
}

size_t gqa_workspace_bytes(int op, int B, int T_or_max_seq, int H, int G, int d, int dtype) {
  if (B < 0 || T_or_max_seq < 0 || check_heads(H, G, d) != GQA_OK || !dtype_ok(dtype)) return 0;
  const size_t es = elem_size(dtype);
  if (op == GQA_OP_PREFILL) {
    // k~ [N, G, d]; the fp32 path also stages q~ [N, H, d] (the bf16 attention kernel
    // normalises and rotates Q itself). bf16: plus the attention kernel's counters and, for
    // grids that may run the paired schedule, its partial states
    const size_t N = (size_t)B * (size_t)T_or_max_seq;
    if (dtype != GQA_BF16) return align_up(N * H * d * es) + align_up(N * G * d * es);
    const long pairs = prefill_pairs(B, T_or_max_seq, H, G);
    return align_up(N * G * d * es) + align_up(((size_t)G + (size_t)pairs) * 4) +
           (size_t)pairs * 2 * prefill_part_floats(d) * 4;
  }
  if (op == GQA_OP_DECODE) {
    // q~ [B, H, d], fp32 partial O [B, H, ns, d], (m, l) [B, H, ns, 2], and the lengths of
    // a generation-loop step [B]
    const size_t ns = (size_t)decode_nsplit(B, H, G, T_or_max_seq);
    return align_up((size_t)B * H * d * es) + align_up((size_t)B * H * ns * d * 4) +
           align_up((size_t)B * H * ns * 2 * 4) + 2 * align_up((size_t)B * 4);
  }
  return 0;
}

gqa_status gqa_prefill(const void* q, const void* k, const void* v, const int32_t* positions,
                       void* out, int B, int T, int H, int G, int d, int causal,
                       const gqa_params* p) {
  gqa_status st = check_params(p);
  if (st != GQA_OK) return st;
  if ((st = check_heads(H, G, d)) != GQA_OK) return st;
  if ((st = check_rope_table(p, d)) != GQA_OK) return st;
  if (B < 0 || T < 0 || (causal != 0 && causal != 1)) return GQA_EINVAL;
  if ((long long)B * T > 0x7fffffffLL) return GQA_EINVAL;
  // the bf16 kernel addresses one sequence's K/V rows of a group with 32-bit buffer offsets
  if (p->dtype == GQA_BF16 && (long long)T * G * d * 2 > 0x7fffffffLL) return GQA_ENOTSUP;
  // the bf16 kernel numbers a sequence's (position, head) columns with 32-bit integers
  if (p->dtype == GQA_BF16 && (long long)T * (H / G) > 0x7fffffffLL) return GQA_ENOTSUP;
  if (p->dtype == GQA_F32 && B > kMaxGridYZ) return GQA_ENOTSUP;
  if ((st = check_masks(p, causal, T)) != GQA_OK) return st;
  if (B == 0 || T == 0) return GQA_OK;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(out)) return GQA_EINVAL;
  if (!opt_int_ok(positions) || !opt_int_ok(p->cu_seqlens) || !opt_tensor_ok(p->k_out))
    return GQA_EINVAL;
  const size_t need = gqa_workspace_bytes(GQA_OP_PREFILL, B, T, H, G, d, p->dtype);
  if (!p->workspace || !aligned(p->workspace, 16) || p->workspace_bytes < need)
    return GQA_EWORKSPACE;

  const bool bf16 = p->dtype == GQA_BF16;
  const size_t es = elem_size(p->dtype);
  const size_t N = (size_t)B * T;
  hipStream_t stream = reinterpret_cast<hipStream_t>(p->stream);
  char* ws = static_cast<char*>(p->workspace);
  void* qt = bf16 ? nullptr : ws;
  void* kt = p->k_out ? p->k_out : ws + (bf16 ? 0 : align_up(N * H * d * es));
  // bf16: [k~][G claim counters, one arrival counter per pair][partial states of the pairs]
  const long pairs = bf16 ? prefill_pairs(B, T, H, G) : 0;
  int32_t* claim = bf16 ? reinterpret_cast<int32_t*>(ws + align_up(N * G * d * es)) : nullptr;
  float* pair_part = bf16 ? reinterpret_cast<float*>(reinterpret_cast<char*>(claim) +
                                                     align_up(((size_t)G + (size_t)pairs) * 4))
                          : nullptr;
  (void)hipGetLastError();

  const long cols = (long)T * (H / G);
  const int cpb = gqa::prefill_bf16_cols_per_block();
  const int n_blk = (int)((cols + cpb - 1) / cpb);
  // Pair heavy and light causal blocks when the grid is at most 2.5 workgroups per CU (two
  // bf16 prefill workgroups are resident per CU; measured against heaviest first: 1-2% faster
  // at 584 and 640 workgroups, 5-12% slower at 704-1024); longer grids run heaviest first, and
  // when a group's blocks spread over several XCDs (G < 8) the workgroups of the unmasked
  // kernel claim their ranks (the counters are zeroed by the prologue launch before it).
  // Measured on T = 32768, H = 64 on two boxes: G = 1 1.4-1.7% faster, G = 4 0.2-0.8%; the
  // block-layout variant, whose workgroups see few tiles, lost 2% to the claim's round trip,
  // so the masked variants keep the fixed order.
  int zigzag = 0, n_cu = 0;
  {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return GQA_EHIP;
    const long grid = (long)B * G * n_blk;
    zigzag = (causal && !p->cu_seqlens && 2 * grid <= 5L * n_cu) ? 1 : 0;
  }
  // the paired schedule: grids of the unmasked causal kernel that are resident at once (two
  // workgroups per CU), whose heaviest blocks see at least 48 key tiles (measured: T = 4096
  // and 3072 (H = 16, G = 8) 8-11% faster, T = 2048 the same, T = 1024 10% slower: the light
  // workgroup's second start outweighs the tiles it takes; a grid of 584 workgroups 25%
  // slower: light workgroups that wait for a slot take their share of the heavy block last)
  const bool paired = bf16 && zigzag && causal && pairs > 0 && p->window <= 0 && !p->block_mask &&
                      (T + 63) / 64 >= 48 && (long)B * G * n_blk <= 2L * n_cu;
  int32_t* counters = claim;
  if (zigzag || G >= 8 || p->window > 0 || p->block_mask) claim = nullptr;

  gqa::PrologueArgs pa{};
  pa.q = bf16 ? nullptr : q;
  pa.k = k;
  pa.q_out = qt;
  pa.k_out = kt;
  pa.positions = positions;
  pa.cu_seqlens = p->cu_seqlens;
  pa.gq = p->q_norm_w;
  pa.gk = p->k_norm_w;
  pa.eps = p->eps;
  pa.decode = 0;
  pa.B = B;
  pa.T = T;
  pa.H = H;
  pa.G = G;
  pa.zero = (claim || paired) ? counters : nullptr;
  pa.zero_n = claim ? G : (paired ? G + (int)pairs : 0);
  fill_rope(pa, p, d);
  if ((st = from_hip(gqa::launch_prologue(pa, B * T, d, bf16, stream))) != GQA_OK) return st;

  gqa::PrefillArgs fa{};
  fa.qt = qt;
  fa.q = q;
  fa.positions = positions;
  fa.gq = p->q_norm_w;
  fa.eps = p->eps;
  fill_rope(fa, p, d);
  fa.kt = kt;
  fa.v = v;
  fa.out = out;
  fa.cu_seqlens = p->cu_seqlens;
  fa.B = B;
  fa.T = T;
  fa.H = H;
  fa.G = G;
  fa.h = H / G;
  fa.causal = causal;
  fill_masks(fa, p);
  fa.n_blk = n_blk;
  fa.zigzag = zigzag;
  fa.claim = claim;
  fa.pair_part = paired ? pair_part : nullptr;
  fa.pair_arrive = paired ? counters + G : nullptr;
  // several sequences: runs of 32 ranks per sequence keep fewer sequences' K/V in each
  // XCD's L2 at a time (measured: varlen 8 x [512, 8192] 1.68 -> 1.46 ms, chunked 1.63 ->
  // 1.54 ms)
  fa.rank_chunk = (fa.zigzag || B == 1) ? 1 : 32;
  fa.scale = eff_scale(p, d);
  fa.scale_log2e = (float)((double)fa.scale * 1.4426950408889634074);
  if ((st = from_hip(mark(p->prof_start, stream))) != GQA_OK) return st;
  st = from_hip(bf16 ? gqa::launch_prefill_bf16(fa, d, stream)
                     : gqa::launch_prefill_f32(fa, d, stream));
  if (st != GQA_OK) return st;
  return from_hip(mark(p->prof_stop, stream));
}

gqa_status gqa_prefill_cached(const void* q, const void* k, const void* v, void* k_cache,
                              void* v_cache, const int32_t* cache_lens,
                              const int32_t* positions, void* out, int B, int T, int H, int G,
                              int d, int max_seq, int causal, const gqa_params* p) {
  gqa_status st = check_params(p);
  if (st != GQA_OK) return st;
  if ((st = check_heads(H, G, d)) != GQA_OK) return st;
  if ((st = check_rope_table(p, d)) != GQA_OK) return st;
  if (B < 0 || T < 0 || max_seq < 1 || (causal != 0 && causal != 1)) return GQA_EINVAL;
  if ((long long)B * T > 0x7fffffffLL) return GQA_EINVAL;
  if (p->dtype != GQA_BF16) return GQA_ENOTSUP;
  if ((long long)max_seq * G * d * 2 > 0x7fffffffLL) return GQA_ENOTSUP;
  if ((long long)T * (H / G) > 0x7fffffffLL) return GQA_ENOTSUP;
  if ((st = check_masks(p, causal, max_seq)) != GQA_OK) return st;
  if (B == 0 || T == 0) return GQA_OK;
  if (!tensor_ok(q) || !tensor_ok(k) || !tensor_ok(v) || !tensor_ok(out) ||
      !tensor_ok(k_cache) || !tensor_ok(v_cache) || !int_ok(cache_lens))
    return GQA_EINVAL;
  if (!opt_int_ok(positions) || !opt_int_ok(p->cu_seqlens)) return GQA_EINVAL;

  hipStream_t stream = reinterpret_cast<hipStream_t>(p->stream);
  (void)hipGetLastError();

  // K of the new tokens: norm + RoPE at cache_lens[b] + t, written with their V into the caches
  gqa::PrologueArgs pa{};
  pa.k = k;
  pa.v = v;
  pa.k_out = k_cache;
  pa.v_out = v_cache;
  pa.positions = positions;
  pa.cu_seqlens = p->cu_seqlens;
  pa.seq_lens = cache_lens;
  pa.gk = p->k_norm_w;
  pa.eps = p->eps;
  pa.decode = 2;
  pa.B = B;
  pa.T = T;
  pa.H = H;
  pa.G = G;
  pa.max_seq = max_seq;
  fill_rope(pa, p, d);
  if ((st = from_hip(gqa::launch_prologue(pa, B * T, d, true, stream))) != GQA_OK) return st;

  gqa::PrefillArgs fa{};
  fa.q = q;
  fa.positions = positions;
  fa.gq = p->q_norm_w;
  fa.eps = p->eps;
  fill_rope(fa, p, d);
  fa.kt = k_cache;
  fa.v = v_cache;
  fa.out = out;
  fa.cu_seqlens = p->cu_seqlens;
  fa.cache_lens = cache_lens;
  fa.max_seq = max_seq;
  fa.B = B;
  fa.T = T;
  fa.H = H;
  fa.G = G;
  fa.h = H / G;
  fa.causal = causal;
  fill_masks(fa, p);
  const long cols = (long)T * fa.h;
  const int cpb = gqa::prefill_bf16_cols_per_block();
  fa.n_blk = (int)((cols + cpb - 1) / cpb);
  fa.zigzag = 0;
  // several sequences: runs of 32 ranks per sequence keep fewer sequences' K/V in each
  // XCD's L2 at a time (measured: varlen 8 x [512, 8192] 1.68 -> 1.46 ms, chunked 1.63 ->
  // 1.54 ms)
  fa.rank_chunk = (fa.zigzag || B == 1) ? 1 : 32;
  fa.scale = eff_scale(p, d);
  fa.scale_log2e = (float)((double)fa.scale * 1.4426950408889634074);
  if ((st = from_hip(mark(p->prof_start, stream))) != GQA_OK) return st;
  if ((st = from_hip(gqa::launch_prefill_bf16(fa, d, stream))) != GQA_OK) return st;
  return from_hip(mark(p->prof_stop, stream));
}

gqa_status gqa_decode(const void* q, void* k_cache, void* v_cache, const int32_t* seq_lens,
                      void* out, int B, int H, int G, int d, int max_seq,
                      const gqa_params* p) {
  const gqa_status st = decode_check(q, k_cache, v_cache, seq_lens, out, B, H, G, d, max_seq, p);
  if (st != GQA_OK || B == 0) return st;
  (void)hipGetLastError();
  return decode_enqueue(q, k_cache, v_cache, seq_lens, out, B, H, G, d, max_seq, p,
                        reinterpret_cast<hipStream_t>(p->stream), true);
}

gqa_status gqa_decode_noalloc(const void* q, void* k_cache, void* v_cache,
                              const int32_t* seq_lens, void* out, int B, int H, int G, int d,
                              int max_seq, const gqa_params* p) {
  if (!p) return GQA_EINVAL;
  // every host check of gqa_decode, with the scratch array standing in for the workspace
  // (a placeholder address until the checks pass, so a rejected call makes no HIP call)
  gqa_params sp = *p;
  sp.workspace = reinterpret_cast<void*>(kAlign);
  sp.workspace_bytes = kScratchBytes;
  gqa_status st = decode_check(q, k_cache, v_cache, seq_lens, out, B, H, G, d, max_seq, &sp);
  if (st != GQA_OK || B == 0) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != GQA_OK) return st;
  sp.workspace = ws;
  (void)hipGetLastError();
  return decode_enqueue(q, k_cache, v_cache, seq_lens, out, B, H, G, d, max_seq, &sp,
                        reinterpret_cast<hipStream_t>(p->stream), true);
}

// The generation loop's step, captured once: the caller refills q / k_new / v_new between
// launches, and each launch advances seq_lens on the device before the decode step.
struct gqa_decode_graph {
  hipGraphExec_t exec;
};

gqa_status gqa_decode_graph_create(const void* q, void* k_cache, void* v_cache,
                                   int32_t* seq_lens, void* out, int B, int H, int G, int d,
                                   int max_seq, const gqa_params* p, gqa_decode_graph** graph) {
  return gqa_decode_graph_create_steps(q, k_cache, v_cache, seq_lens, out, B, H, G, d, max_seq,
                                       1, p, graph);
}

gqa_status gqa_decode_graph_create_steps(const void* q, void* k_cache, void* v_cache,
                                         int32_t* seq_lens, void* out, int B, int H, int G,
                                         int d, int max_seq, int steps, const gqa_params* p,
                                         gqa_decode_graph** graph) {
  if (!graph) return GQA_EINVAL;
  *graph = nullptr;
  if (steps < 1 || steps > kMaxGraphSteps) return GQA_EINVAL;
  gqa_status st = decode_check(q, k_cache, v_cache, seq_lens, out, B, H, G, d, max_seq, p);
  if (st != GQA_OK) return st;
  if (!p->k_new || !p->v_new) return GQA_EINVAL;  // every step appends its token
  (void)hipGetLastError();
  const size_t es = elem_size(p->dtype);
  const size_t q_step = (size_t)B * H * d * es, kv_step = (size_t)B * G * d * es;

  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) return GQA_EHIP;
  hipGraph_t g = nullptr;
  hipGraphExec_t exec = nullptr;
  if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return GQA_EHIP;
  }
  if (B > 0) {
    // one step: its three kernels; several: 2 steps + 1 kernels with the fused passes between
    // steps (while the prologue rows of one launch stay below 2^22)
    if (steps == 1 || (long)B * (H + 2L * G) >= (1L << 22))
      for (int i = 0; i < steps && st == GQA_OK; ++i) {
        gqa_params ps = *p;
        ps.k_new = static_cast<const char*>(p->k_new) + i * kv_step;
        ps.v_new = static_cast<const char*>(p->v_new) + i * kv_step;
        if (p->positions) ps.positions = p->positions + (size_t)i * B;
        st = decode_enqueue(static_cast<const char*>(q) + i * q_step, k_cache, v_cache, seq_lens,
                            static_cast<char*>(out) + i * q_step, B, H, G, d, max_seq, &ps, cs,
                            false, /*advance=*/true);
      }
    else
      st = decode_steps_enqueue(q, k_cache, v_cache, seq_lens, out, B, H, G, d, max_seq, steps,
                                p, cs);
  }
  // the capture is ended whatever happened inside it
  const hipError_t ec = hipStreamEndCapture(cs, &g);
  if (st == GQA_OK && ec != hipSuccess) st = GQA_EHIP;
  if (st == GQA_OK && hipGraphInstantiate(&exec, g, nullptr, nullptr, 0) != hipSuccess)
    st = GQA_EHIP;
  if (g) (void)hipGraphDestroy(g);
  (void)hipStreamDestroy(cs);
  if (st != GQA_OK) {
    if (exec) (void)hipGraphExecDestroy(exec);
    return st;
  }
  gqa_decode_graph* h = new (std::nothrow) gqa_decode_graph{exec};
  if (!h) {
    (void)hipGraphExecDestroy(exec);
    return GQA_EHIP;
  }
  *graph = h;
  return GQA_OK;
}

gqa_status gqa_decode_graph_launch(gqa_decode_graph* graph, void* stream) {
  if (!graph || !graph->exec) return GQA_EINVAL;
  return from_hip(hipGraphLaunch(graph->exec, reinterpret_cast<hipStream_t>(stream)));
}

gqa_status gqa_decode_graph_destroy(gqa_decode_graph* graph) {
  if (!graph) return GQA_OK;
  const hipError_t e = graph->exec ? hipGraphExecDestroy(graph->exec) : hipSuccess;
  delete graph;
  return from_hip(e);
}

gqa_status gqa_qk_norm_rope(const void* q, const void* k, const int32_t* positions,
                            void* q_out, void* k_out, int N, int H, int G, int d,
                            const gqa_params* p) {
  gqa_status st = check_params(p);
  if (st != GQA_OK) return st;
  if ((st = check_heads(H, G, d)) != GQA_OK) return st;
  if ((st = check_rope_table(p, d)) != GQA_OK) return st;
  if (N < 0) return GQA_EINVAL;
  if (N == 0) return GQA_OK;
  if (!tensor_ok(q) || !tensor_ok(q_out)) return GQA_EINVAL;
  if ((k == nullptr) != (k_out == nullptr)) return GQA_EINVAL;
  if (!opt_tensor_ok(k) || !opt_tensor_ok(k_out) || !opt_int_ok(positions)) return GQA_EINVAL;
  (void)hipGetLastError();
  gqa::PrologueArgs pa{};
  pa.q = q;
  pa.k = k;
  pa.q_out = q_out;
  pa.k_out = k_out;
  pa.positions = positions;
  pa.gq = p->q_norm_w;
  pa.gk = p->k_norm_w;
  pa.eps = p->eps;
  pa.decode = 0;
  pa.B = 1;
  pa.T = N;
  pa.H = H;
  pa.G = G;
  fill_rope(pa, p, d);
  return from_hip(gqa::launch_prologue(pa, N, d, p->dtype == GQA_BF16,
                                       reinterpret_cast<hipStream_t>(p->stream)));
}

}  // extern "C"
