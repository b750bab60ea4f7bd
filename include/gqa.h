/*
 * gqa.h -- C ABI of the MI355X (gfx950) causal grouped-query attention library (libgqa.so).
 *
 * The operation (one transformer attention layer between the QKV projection and o_proj):
 *
 *   1. QK prologue.  For every token t and head: x_hat = x / sqrt(mean(x^2) + eps),
 *      x_bar = gamma (.) x_hat, then RoPE: each adjacent pair (x_2j, x_2j+1) is rotated
 *      counter-clockwise by pos[t] * omega_j, omega_j = theta^(-2j/d).  Applied to Q with
 *      gamma_q and to K with gamma_k; V is left alone.
 *        - RMSNorm: zhanghao0806.com "Qwen3系列1-理论基础&真实结构", D2-1 (formula).
 *        - per head, Q and K only, norm then RoPE, one gamma for all Q heads and one for
 *          all K heads: same page, D2-2; nano-vllm "Qwen3" page (selfknow.cn), Attention
 *          forward steps (4) and (5).
 *        - R(pos) as 2x2 rotation blocks: same page, D2-2 (matrix R(pos)); adjacent
 *          even/odd pairs: ewbang.com "深入剖析Qwen3模型架构", 3.1.2 (RoPE code);
 *          omega_j and base 1e6: same article, 3.4.1.
 *   2. Attention.  Query head i reads KV head g = floor(i / h), h = H / G (the article's
 *      3.1.2 GQA module repeats each K/V head h times); for each sequence
 *      out = softmax(Q K^T * scale + M) V with M = -inf where key index > query index
 *      (causal) and the row maximum subtracted inside the softmax.
 *        - zhanghao0806.com page, D1-4 (formula), D1-5 (causal mask), D1-2 (stable
 *          softmax), D2-3 (groups, KV cache, prefill / decode).
 *   Decode: one new token per sequence attends to all seq_lens[b] cached rows; its own K/V
 *   are written into the cache first (D2-3: the layer writes K/V into the cache before
 *   computing attention).
 *
 * Conventions for every entry point
 *   - Tensors are contiguous, row-major, token-major and live in device memory:
 *       q, out [N, H, d]; k, v [N, G, d]; decode q, out [B, H, d];
 *       caches [B, max_seq, G, d] holding K after norm + RoPE and raw V.
 *     Element type is params->dtype (fp32 or bf16) for q, k, v, out, caches, k_new, v_new,
 *     k_out and the two norm weights.  Integer arrays are device int32.
 *   - The caller owns all memory.  The library allocates nothing and keeps no state
 *     between calls, so it is re-entrant; the one exception is the decode graph object
 *     below, which the caller creates and destroys explicitly.  Work is enqueued on params->stream (a
 *     hipStream_t; NULL = the default stream) and the call returns without waiting.
 *     Buffers must stay valid until that stream work has finished.  Outputs must not
 *     alias inputs.
 *   - Errors found on the host are returned at once and nothing is enqueued:
 *       GQA_EINVAL    null required pointer, negative size, H, G or d <= 0, H % G != 0,
 *                     a device pointer not 16-byte aligned, an int array not 4-byte aligned,
 *                     a non-finite entry in rope_inv_freq;
 *       GQA_ENOTSUP   d not in {64, 128}, an unknown dtype, a bf16 prefill whose
 *                     T * G * d * 2 exceeds 2^31 - 1 bytes (one sequence's K rows) or
 *                     whose T * H / G exceeds 2^31 - 1 (its (position, head) columns), a
 *                     decode whose max_seq * G * d * element size exceeds 2^31 - 1 bytes
 *                     or max_seq exceeds 4096 splits of
 *                     gqa_decode_split_keys(B, H, G, max_seq) keys, a decode or fp32
 *                     prefill with B > 65535 (sequences index a grid dimension);
 *       GQA_EWORKSPACE workspace smaller than gqa_workspace_bytes() or NULL when needed;
 *       GQA_EHIP      a HIP launch error.
 *     A batch with B == 0 or T == 0 is valid and enqueues nothing.  Device faults show up
 *     at the caller's next synchronisation.  Values inside device int arrays (positions,
 *     seq_lens, cu_seqlens) are trusted: out-of-range values are undefined behaviour,
 *     except a sequence of length 0 (no rows; decode writes zeros).  Nothing is printed and
 *     no C++ exception crosses this interface.
 *   - Non-finite inputs.  A NaN or infinity in q (token t, head i) reaches out[t, i] only
 *     (after the RMSNorm an infinite element makes its head row NaN).  One in the K row of
 *     token t, group g reaches exactly the outputs of group g's query heads whose queries
 *     see key t (a K row already in a cache skips the norm: there an infinity gives scores
 *     of +-inf, and -inf only drops that key).  One in the V row of token t, group g reaches those outputs too; the fp32
 *     prefill and decode stop there, while the bf16 prefill may also turn NaN the outputs of
 *     group g's heads at the other query positions of the same 128-column block (128 / h
 *     consecutive positions) that do not see key t, because its products multiply whole
 *     64-key tiles of V by weights that are exactly 0 for the keys a query does not see
 *     (and 0 * inf = 0 * NaN = NaN).  Cache rows at or past a sequence's length are never
 *     read.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gqa_status {
  GQA_OK = 0,
  GQA_EINVAL = 1,
  GQA_ENOTSUP = 2,
  GQA_EWORKSPACE = 3,
  GQA_EHIP = 4
} gqa_status;

typedef enum gqa_dtype { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype;

typedef enum gqa_op { GQA_OP_PREFILL = 0, GQA_OP_DECODE = 1, GQA_OP_QK_NORM_ROPE = 2 } gqa_op;

typedef struct gqa_params {
  gqa_dtype dtype;           /* element type of every float tensor of the call              */
  const void *q_norm_w;      /* [d] gamma_q; NULL = no RMSNorm on Q                          */
  const void *k_norm_w;      /* [d] gamma_k; NULL = no RMSNorm on K                          */
  float eps;                 /* RMSNorm epsilon, added inside the square root                */
  double rope_theta;         /* RoPE base theta (Qwen3: 1e6); 0 = no RoPE                    */
  float scale;               /* score scale; 0 = 1/sqrt(d)                                   */
  const int32_t *cu_seqlens; /* prefill: device [B+1] packed offsets, cu[0] = 0;
                                NULL = dense, every sequence has length T                   */
  void *k_out;               /* prefill: optional [N, G, d] output of normalised, rotated K
                                (e.g. the KV cache); NULL = keep it in the workspace         */
  const void *k_new;         /* decode: optional [B, G, d] raw K of the new token            */
  const void *v_new;         /* decode: optional [B, G, d] V of the new token; with k_new,
                                RoPE(RMSNorm(k_new)) and v_new are written into cache slot
                                seq_lens[b]-1 before attention                               */
  const int32_t *positions;  /* decode: optional device [B] RoPE positions of the new
                                tokens; NULL = seq_lens[b]-1                                 */
  void *workspace;           /* device scratch, >= gqa_workspace_bytes(), 256-byte aligned  */
  size_t workspace_bytes;
  void *stream;              /* hipStream_t; NULL = default stream                           */
  void *prof_start;          /* optional hipEvent_t, recorded on the stream right before the
                                main kernel (prefill attention, or the decode split pass);
                                for callers that time that kernel alone. NULL = none       */
  void *prof_stop;           /* optional hipEvent_t, recorded right after that kernel       */
  int window;                /* bf16 prefill (and cached prefill), causal only: > 0 keeps
                                only the `window` most recent keys of each query (key index
                                > query index - window); 0 = no window                     */
  const uint32_t *block_mask; /* bf16 prefill (and cached prefill): optional device bit rows
                                over 64-key blocks.  Row qb (query indices 64 qb .. 64 qb +
                                63) has block_mask_words words; bit j of word w set = query
                                block qb sees key block 32 w + j.  The diagonal block is
                                always seen.  Rows: ceil(T / 64) for gqa_prefill, ceil(max_seq
                                / 64) for gqa_prefill_cached; one mask serves every sequence
                                (indices inside the sequence).  NULL = no block mask        */
  int block_mask_words;      /* words per block_mask row, >= ceil(ceil(T_keys / 64) / 32)   */
  const double *rope_inv_freq; /* optional HOST array of the d/2 RoPE frequencies omega_j
                                (a scaled variant: linear interpolation, the architecture
                                article's YaRN formula (3.4.2), an NTK base change...); read
                                during the call (a decode graph keeps the values it saw at
                                creation).  When set, RoPE is applied with it and rope_theta
                                is ignored.  NULL = omega_j = rope_theta^(-2j/d)            */
} gqa_params;

/* Fills p with defaults: bf16, no norm weights, eps 1e-6, theta 1e6, scale 1/sqrt(d),
 * dense, no workspace, default stream, no profiling events, no window, no block mask, no
 * frequency table. */
void gqa_params_init(gqa_params *p);

/* Prefill (prompt) attention with the QK prologue.
 *   q [N, H, d], k and v [N, G, d] raw projections; out [N, H, d].
 *   positions: device [N] RoPE positions, or NULL for 0..T_b-1 inside every sequence (the
 *     causal mask always uses the index inside the sequence; positions feed RoPE only).
 *   Dense: N = B*T and sequence b is tokens [b*T, (b+1)*T).  Packed: p->cu_seqlens given,
 *     N = cu_seqlens[B], sequence b is [cu[b], cu[b+1]) and T must be >= every length.
 *   causal: 1 = causal mask inside each sequence, 0 = every key of the sequence visible.
 *   Mask variants (bf16 only; zizhi168.cn Qwen3 technical-report summary, section 3.1:
 *   local attention inside a 512-token window, block-sparse attention over 64-token blocks):
 *     p->window > 0 (needs causal = 1) and / or p->block_mask narrow the visible keys
 *     further; key tiles no query of a workgroup sees are skipped.  GQA_EINVAL for a
 *     negative window, a window without the causal mask, a misaligned block_mask or
 *     block_mask_words too small for T; GQA_ENOTSUP for either with fp32.
 *   Needs p->workspace of gqa_workspace_bytes(GQA_OP_PREFILL, B, T, H, G, d, dtype).  The
 *   call keeps counters and, on grids that fit the chip at once, partial softmax states in
 *   it (reset by the call itself): calls that share one workspace must not overlap. */
gqa_status gqa_prefill(const void *q, const void *k, const void *v, const int32_t *positions,
                       void *out, int B, int T, int H, int G, int d, int causal,
                       const gqa_params *p);

/* Prefill of new tokens against a KV cache (chunked or multi-turn prefill), bf16 only.
 *   Sequence b has cache_lens[b] earlier tokens in k_cache / v_cache [B, max_seq, G, d] (K
 *   after norm + RoPE, raw V, as gqa_decode and gqa_prefill's k_out store them).  Its new
 *   tokens are q [N, H, d], k, v [N, G, d] (raw): dense N = B*T, token b*T + t; or packed
 *   with p->cu_seqlens as in gqa_prefill.  New token t of sequence b has RoPE position
 *   cache_lens[b] + t (or positions[token], device [N]).  Its K after the prologue and its V
 *   are first written into the caches at slot cache_lens[b] + t (zhanghao0806.com page,
 *   D2-3: the layer writes K/V into the cache before attention; nano-vllm "Qwen3" page,
 *   step (6)), then with causal = 1 it attends to keys 0 .. cache_lens[b] + t of its sequence
 *   (D1-5 with the query at key index cache_lens[b] + t); causal = 0: to all
 *   cache_lens[b] + T_b keys.  out [N, H, d].  cache_lens[b] + T_b <= max_seq is the
 *   caller's to ensure: rows past max_seq are neither written nor read.  p->window and
 *   p->block_mask work as in gqa_prefill over key indices of the whole sequence (cache rows
 *   first), the block mask with ceil(max_seq / 64) rows.  No workspace;
 *   p->k_out, k_new and v_new are not used.  GQA_ENOTSUP for fp32 and when
 *   max_seq * G * d * 2 exceeds 2^31 - 1 bytes. */
gqa_status gqa_prefill_cached(const void *q, const void *k, const void *v, void *k_cache,
                              void *v_cache, const int32_t *cache_lens,
                              const int32_t *positions, void *out, int B, int T, int H, int G,
                              int d, int max_seq, int causal, const gqa_params *p);

/* Single-token decode against a contiguous KV cache.
 *   q [B, H, d] raw query of the new token per sequence; out [B, H, d].
 *   k_cache, v_cache [B, max_seq, G, d]: rows 0..seq_lens[b]-1 are visible to sequence b;
 *     K rows are post-prologue.  With p->k_new and p->v_new the new row is written at
 *     slot seq_lens[b]-1 first (so k_cache and v_cache are written only then).
 *   seq_lens: device [B], 0 <= seq_lens[b] <= max_seq, counting the new token.
 *   p->window and p->block_mask are not supported here (GQA_ENOTSUP when set).
 *   When the two caches together exceed 512 MiB (2*B*max_seq*G*d*elem bytes) the bf16 pass
 *   reads V with a non-temporal cache hint; the results are the same bits either way.
 *   Needs p->workspace of gqa_workspace_bytes(GQA_OP_DECODE, B, max_seq, H, G, d, dtype), where
 *   the split partials live until the combine: calls that share one workspace must not
 *   overlap. */
gqa_status gqa_decode(const void *q, void *k_cache, void *v_cache, const int32_t *seq_lens,
                      void *out, int B, int H, int G, int d, int max_seq,
                      const gqa_params *p);

/* gqa_decode without a workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, checks and result bits as gqa_decode; p->workspace and p->workspace_bytes are
 * ignored.  The scratch (normalised queries, per-split partial results) lives instead in a
 * fixed device array of GQA_DECODE_NOALLOC_MAX_BYTES inside the library, one per GPU, held
 * from the first call on that GPU until the process ends; the call itself allocates nothing
 * and calls no allocating routine.  GQA_EWORKSPACE when the decode needs more scratch than
 * that (gqa_workspace_bytes(GQA_OP_DECODE, B, max_seq, H, G, d, dtype) above the maximum:
 * e.g. 64 sequences x 32 heads over a 32768-row cache need 34.1 MB).  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (two streams, two threads, or
 * one graph replay beside another call) race and give undefined results; calls ordered on
 * one stream do not.  Nothing in the array needs clearing: each call writes every value
 * it reads.  The first call on a GPU looks up the array's address (GQA_EHIP if that
 * fails). */
#define GQA_DECODE_NOALLOC_MAX_BYTES (64u * 1024u * 1024u)

gqa_status gqa_decode_noalloc(const void *q, void *k_cache, void *v_cache,
                              const int32_t *seq_lens, void *out, int B, int H, int G, int d,
                              int max_seq, const gqa_params *p);

/* Generation loop: the decode step captured once as a HIP graph and replayed per token.
 *   Generation runs one forward pass per new token, each seeing every earlier token
 *   (zhanghao0806.com page, D1-1, Q2 and Q5); the launches of one step are fixed, so they are
 *   recorded once (nano-vllm "Qwen3" page, the CUDA graph note beside compute_logits) and
 *   replayed without per-kernel launch cost.
 *
 *   gqa_decode_graph_create takes the arguments of gqa_decode; p->k_new and p->v_new are
 *   required (every step appends its token).  It records, on a private stream, a step that
 *     1. gives every sequence its new token: L_b = min(seq_lens[b] + 1, max_seq) (device
 *        side), then
 *     2. does exactly what gqa_decode does with seq_lens[b] = L_b: norm + RoPE of q and
 *        k_new, k_new / v_new written at slot L_b - 1, attention over L_b rows,
 *   and leaves seq_lens[b] = L_b when the step has finished (the step's three kernels carry
 *   the advance themselves: the prologue computes L_b, the last pass stores it).
 *   So before the first launch seq_lens[b] counts the tokens already in the cache.  Every
 *   pointer and size, and every field of *p except stream and the profiling events (which
 *   are ignored), is fixed at creation; the contents of q, k_new, v_new, positions and
 *   seq_lens are read at each launch, so the caller writes the next token's q / k_new /
 *   v_new into the same buffers between launches.  A sequence already at max_seq stays
 *   there and its next token overwrites slot max_seq - 1.  All buffers, including the
 *   workspace, must stay valid until the graph is destroyed and its launches have finished.
 *   Errors: those of gqa_decode, GQA_EINVAL without k_new / v_new or with graph == NULL,
 *   GQA_EHIP if HIP cannot capture or instantiate; on error *graph is NULL.  The graph
 *   object holds the instantiated HIP graph (no device memory of the library's own).
 *   B == 0 gives a graph whose launches do nothing.
 *
 *   gqa_decode_graph_launch enqueues the graph's step(s) on `stream` (a hipStream_t; NULL =
 *   default).
 *   Launches on one graph must not overlap (they share the workspace); in one stream they
 *   never do.
 *   gqa_decode_graph_destroy releases the graph (NULL is accepted); its launches must have
 *   finished. */
typedef struct gqa_decode_graph gqa_decode_graph;

gqa_status gqa_decode_graph_create(const void *q, void *k_cache, void *v_cache,
                                   int32_t *seq_lens, void *out, int B, int H, int G, int d,
                                   int max_seq, const gqa_params *p, gqa_decode_graph **graph);

/* Several generation steps in one graph (a HIP graph launch costs about 5 us more than the
 * stream launches of its kernels, measured on MI355X, so a graph of several steps spends it
 * once per `steps` tokens).  Arguments as gqa_decode_graph_create, with 1 <= steps <= 256
 * (else GQA_EINVAL): q and out hold `steps` consecutive [B, H, d] blocks, p->k_new and
 * p->v_new `steps` consecutive [B, G, d] blocks, p->positions (when set) `steps` consecutive
 * [B] blocks; step i reads and writes block i.  One launch runs the steps in order, each
 * doing what one launch of a one-step graph does (so seq_lens[b] grows by `steps`, capped at
 * max_seq).  gqa_decode_graph_create is this function with steps = 1. */
gqa_status gqa_decode_graph_create_steps(const void *q, void *k_cache, void *v_cache,
                                         int32_t *seq_lens, void *out, int B, int H, int G,
                                         int d, int max_seq, int steps, const gqa_params *p,
                                         gqa_decode_graph **graph);

gqa_status gqa_decode_graph_launch(gqa_decode_graph *graph, void *stream);

gqa_status gqa_decode_graph_destroy(gqa_decode_graph *graph);

/* The QK prologue alone (RMSNorm then RoPE), for step-level checks.
 *   q [N, H, d] -> q_out [N, H, d]; k [N, G, d] -> k_out [N, G, d]; positions device [N]
 *   or NULL for 0..N-1.  No workspace. */
gqa_status gqa_qk_norm_rope(const void *q, const void *k, const int32_t *positions,
                            void *q_out, void *k_out, int N, int H, int G, int d,
                            const gqa_params *p);

/* RoPE frequency tables for gqa_params.rope_inv_freq: writes the d/2 frequencies omega_j,
 * j = 0 .. d/2 - 1, of one rule into the caller's HOST array out[d/2], in fp64.
 *   GQA_ROPE_BASE    omega_j = theta^(-2j/d) (ewbang.com "深入剖析Qwen3模型架构", 3.4.1).
 *   GQA_ROPE_LINEAR  linear position interpolation by the extension factor alpha: every
 *                    position index divided by alpha, i.e. omega_j / alpha (zizhi168.cn
 *                    Qwen3 technical-report summary, 4.2).  alpha > 0.
 *   GQA_ROPE_YARN    the scaling the architecture article prints under the name YaRN (3.4.2):
 *                    when infer_len > train_len, omega_j * (1 - s * 2j / d) with
 *                    s = scale * log2(infer_len / train_len); otherwise the base table.  No
 *                    ramp and no attention temperature (it is not the published YaRN); past
 *                    infer_len / train_len = 2^(1/scale) the lowest frequencies turn negative,
 *                    which is what the formula gives.  train_len, infer_len > 0.
 *   GQA_ROPE_NTK     NTK-aware scaling read as a change of base (summary, 4.2): the base table
 *                    of theta * alpha^(d / (d - 2)), which keeps omega_0 and divides
 *                    omega_{d/2-1} by alpha.  alpha > 0, d > 2.
 * Arguments a rule does not use are ignored.  d must be even, 2 <= d <= 128; theta > 0 and
 * every used argument finite.  Returns GQA_EINVAL (nothing written) for a NULL out, an
 * unknown kind or an argument out of range, GQA_OK otherwise.  Pure host arithmetic: no HIP
 * call, no device needed. */
typedef enum gqa_rope_kind {
  GQA_ROPE_BASE = 0,
  GQA_ROPE_LINEAR = 1,
  GQA_ROPE_YARN = 2,
  GQA_ROPE_NTK = 3
} gqa_rope_kind;

gqa_status gqa_rope_freq_table(int kind, int d, double theta, double alpha, double train_len,
                               double infer_len, double scale, double *out);

/* Bytes of workspace an entry point needs (0 when none).  op is a gqa_op, T_or_max_seq is
 * T for prefill and max_seq for decode, dtype a gqa_dtype.  Returns 0 for invalid sizes. */
size_t gqa_workspace_bytes(int op, int B, int T_or_max_seq, int H, int G, int d, int dtype);

/* Keys per split of the decode pass (the split-KV partition of each sequence) for a decode
 * of B sequences, H query heads, G KV heads and a cache of max_seq rows: 1024, halved (down
 * to 256) while B * G * ceil(H / G / 32) * ceil(max_seq / split) stays below 2048
 * workgroups, so that short caches still spread over the chip.  0 for invalid sizes.  The
 * result does not depend on it beyond rounding (splits merge exactly). */
int gqa_decode_split_keys(int B, int H, int G, int max_seq);

/* Static text for a status code. */
const char *gqa_status_str(gqa_status s);

#ifdef __cplusplus
}
#endif
#endif /* GQA_H */
