/*
 * specverify.h -- C ABI of the MI355X (gfx950) verify/accept library for block
 * speculative decoding.
 *
 * One decode cycle hands the accept policy a target logit block [K+1, V] per
 * sequence: row 0 is p_1 from the anchor step, rows 1..K are p_2..p_{K+1}
 * from one verify forward over the K drafted tokens, row K being the bonus
 * position ("dspark-mlx 0.1.0" wheel diff, dspark_mlx/adapter.py, module
 * docstring "Logit conventions").  The policy exports greedy_accept and
 * speculative_sample_accept returning an AcceptResult (same page,
 * dspark_mlx/__init__.py); the accepted count is what
 * BaseModelAdapter.kv_rollback(n_keep) consumes (same page, adapter.py).
 *
 * Conventions shared by every entry point:
 *  - Logit pointers, token, seed and output pointers are DEVICE pointers; the
 *    caller owns every buffer, the workspace included.  The library never
 *    allocates, never synchronises, and enqueues its kernels only on
 *    `hip_stream` (a hipStream_t; NULL is the default stream).  Outputs are
 *    valid once the stream reaches that point.
 *  - Logits are fp32 or bf16 (dtype), laid out [b, rows, V] with V
 *    contiguous; strides are in ELEMENTS.  `*_row_stride` >= V,
 *    `*_batch_stride` >= 0.  Base pointers must be aligned to the element
 *    size.  Rows that start on 16-byte boundaries take 16-byte vector loads;
 *    other layouts take an element-wise path with identical results.
 *  - Argument errors are reported before anything is enqueued.  Per-sequence
 *    data errors never fail the call: a sequence whose rows hold NaN or +inf,
 *    or a row with no finite entry, or a draft token outside [0, V), gets
 *    n_accepted = -1, all its tokens -1 and NaN probabilities.  -inf logits
 *    (masked vocabulary) are allowed.
 *  - Calls are thread-safe and keep no state between calls.  Calls that share
 *    one workspace must be ordered on one stream.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPEC_OK = 0,
    SPEC_EINVAL = 1,   /* bad size, stride, temperature, null pointer, small or misaligned workspace */
    SPEC_EDTYPE = 2,   /* unknown dtype code */
    SPEC_EALIGN = 3,   /* a logit base pointer not aligned to its element size */
    SPEC_ELAUNCH = 4,  /* the HIP runtime refused a kernel launch */
    SPEC_ESCRATCH = 5  /* spec_mixed_accept_noalloc: the call needs more than SPEC_SCRATCH_BYTES */
} spec_status;

typedef enum {
    SPEC_F32 = 0,
    SPEC_BF16 = 1
} spec_dtype;

/* Largest block length K accepted by the entry points. */
#define SPEC_MAX_K 32

/*
 * Bytes of device workspace one call needs for batch b, block length K and
 * vocabulary V (sampling != 0 for spec_sample_accept).  Returns 0 when the
 * sizes are out of range (b < 1, K < 1, K > SPEC_MAX_K, V < 1) or the dtype
 * is unknown.  The workspace needs no initialisation and must be 256-byte
 * aligned (every entry point returns SPEC_EINVAL for a smaller or misaligned
 * workspace).
 */
size_t spec_workspace_bytes(int b, int K, int V, int dtype, int sampling);

/* Static description of a status code (never NULL). */
const char *spec_status_string(int status);

/*
 * Greedy accept: the committed tokens are the target's own argmax chain, so
 * the output equals plain greedy decoding up to exact ties ("mlx-dspark
 * 0.0.1" sdist diff, README "How it works"; benchmark.py's plain greedy token
 * is the argmax of the raw logits).
 *
 * For each sequence s: A_i = lowest index of the largest raw logit of target
 * row i (i = 0..K); n = length of the longest prefix with x_i == A_i;
 * tokens[s] = (x_0 .. x_{n-1}, A_n, -1, ..., -1) (K+1 entries).
 *
 *   target          [b, K+1, V] logits (device), element strides below
 *   draft_tokens    [b, K] int32 (device)
 *   n_accepted      [b] int32 out (device)
 *   tokens          [b, K+1] int32 out (device)
 *   target_argmax   [b, K+1] int32 out (device) or NULL: A_i of every row
 *   workspace       spec_workspace_bytes(b, K, V, dtype, 0) bytes (device)
 */
int spec_greedy_accept(const void *target, int dtype,
                       int64_t t_batch_stride, int64_t t_row_stride,
                       const int32_t *draft_tokens, int b, int K, int V,
                       int32_t *n_accepted, int32_t *tokens, int32_t *target_argmax,
                       void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Lossless speculative-sampling accept (the published rule of Leviathan,
 * Kalman & Matias 2023 and Chen et al. 2023; the pages call the policy
 * lossless: "dspark-mlx 0.1.0", adapter.py docstring, and the
 * "DeepSeek-V4-Flash DSpark drafter" model card).
 *
 * With p_i = softmax(target row i / T) and q_i = softmax(draft row i / T):
 * slot i < K accepts x_i iff u_i < min(1, p_i(x_i) / q_i(x_i)), where
 * u_i = U(seed_s, s, i, 0); n = index of the first rejected slot, else K.
 * When n < K the token at slot n is drawn from normalise(max(0, p_n - q_n));
 * when n == K it is drawn from p_{K+1} (the bonus); in both cases by inverse
 * CDF in ascending vocabulary order with t = U(seed_s, s, n, 1) * R, R the
 * total mass.  U(seed, row, pos, tag) = (w >> 8) * 2^-24 with w the first
 * output word of Philox4x32-10 (Salmon et al., SC'11) at counter
 * (pos, row, tag, 0) and key (low, high 32 bits of seed); `row` is the
 * sequence index inside this call.
 *
 *   target          [b, K+1, V] logits (device)
 *   draft           [b, K, V] logits of the same dtype (device)
 *   draft_tokens    [b, K] int32 (device), drawn by the caller from q
 *   temperature     T > 0, finite; divides the logits of both sides
 *   seeds           [b] uint64 (device), one Philox key per sequence
 *   n_accepted      [b] int32 out; tokens [b, K+1] int32 out (-1 padded)
 *   p_draft, q_draft  [b, K] float out or NULL: p_i(x_i), q_i(x_i) of every slot
 *   workspace       spec_workspace_bytes(b, K, V, dtype, 1) bytes (device)
 */
int spec_sample_accept(const void *target, const void *draft, int dtype,
                       int64_t t_batch_stride, int64_t t_row_stride,
                       int64_t d_batch_stride, int64_t d_row_stride,
                       const int32_t *draft_tokens, int b, int K, int V,
                       double temperature, const uint64_t *seeds,
                       int32_t *n_accepted, int32_t *tokens,
                       float *p_draft, float *q_draft,
                       void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Mixed batch: each sequence picks its rule by its own temperature, as a
 * serving batch mixes greedy and sampled requests.  temperatures[s] == 0
 * selects the greedy rule for sequence s (the drafter's temperature 0.0
 * default meaning greedy decoding, "dspark-mlx 0.1.0" wheel diff,
 * dspark_mlx/arch/gemma4.py, Gemma4DSparkArgs); a finite temperatures[s] > 0
 * selects the sampling rule at that temperature; any other value makes the
 * sequence invalid (n_accepted = -1).  Every sequence gets exactly what
 * spec_greedy_accept / spec_sample_accept give it, with its index s in THIS
 * batch as the Philox row.  Draft rows of greedy sequences are never read.
 *
 * Each sequence may also carry fewer than K draft tokens: a drafter's
 * confidence head truncates its block and a draft cap limits it ("mlx-dspark
 * 0.0.1" sdist diff, README "Tuning" and the --max-draft /
 * --confidence-threshold flags of its __main__.py; the confidence output of
 * "dspark-mlx 0.1.0", DraftBackbone.forward_spec).  Sequence s with draft
 * length Ks = draft_lengths[s], 0 <= Ks <= K, verifies target rows 0..Ks
 * (row Ks its bonus position), draft rows 0..Ks-1 and draft tokens
 * 0..Ks-1, exactly as a call with K = Ks would; Ks = 0 commits one token
 * (the argmax of row 0, or a draw from p_1).  Storage past its block is never
 * read; outputs past it are -1 (tokens, target_argmax) and NaN (p_draft,
 * q_draft).  Ks outside [0, K] makes the sequence invalid.  Strides and
 * output shapes stay those of K.
 *
 *   temperatures    [b] double (device)
 *   draft_lengths   [b] int32 (device), or NULL: every sequence has K
 *   p_draft, q_draft  [b, K] float out or NULL (NaN for greedy sequences)
 *   target_argmax   [b, K+1] int32 out or NULL (-1 for sampling sequences)
 *   workspace       spec_mixed_workspace_bytes(b, K, V, dtype) bytes (device)
 * Other arguments as for spec_sample_accept.  Four kernels, like the
 * sampling rule alone.
 */
size_t spec_mixed_workspace_bytes(int b, int K, int V, int dtype);

int spec_mixed_accept(const void *target, const void *draft, int dtype,
                      int64_t t_batch_stride, int64_t t_row_stride,
                      int64_t d_batch_stride, int64_t d_row_stride,
                      const int32_t *draft_tokens, int b, int K, int V,
                      const double *temperatures, const int32_t *draft_lengths,
                      const uint64_t *seeds,
                      int32_t *n_accepted, int32_t *tokens,
                      float *p_draft, float *q_draft, int32_t *target_argmax,
                      void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * spec_mixed_accept for callers that cannot allocate device memory: code
 * recorded under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels and results as
 * spec_mixed_accept, without the workspace: the call runs in a fixed array
 * of SPEC_SCRATCH_BYTES in device memory that the library holds on each GPU
 * it runs on until the process ends (its address is looked up once per
 * device, on the first call there).  The call allocates nothing.
 *
 * Limit: spec_mixed_workspace_bytes(b, K, V, dtype) must not exceed
 * SPEC_SCRATCH_BYTES, else SPEC_ESCRATCH before anything is enqueued (8 MiB
 * holds b = 128 at K = 7, V = 262144 in bf16 or in fp32).  Every call on one
 * GPU uses the same array: calls that may overlap on one GPU (several
 * streams, several host threads) race and must be ordered by the caller, for
 * example on one stream.  The array keeps the last call's contents; no call
 * needs it cleared.
 */
#define SPEC_SCRATCH_BYTES (8u << 20)

int spec_mixed_accept_noalloc(const void *target, const void *draft, int dtype,
                              int64_t t_batch_stride, int64_t t_row_stride,
                              int64_t d_batch_stride, int64_t d_row_stride,
                              const int32_t *draft_tokens, int b, int K, int V,
                              const double *temperatures, const int32_t *draft_lengths,
                              const uint64_t *seeds,
                              int32_t *n_accepted, int32_t *tokens,
                              float *p_draft, float *q_draft, int32_t *target_argmax,
                              void *hip_stream);

/*
 * Fused verify: the target logit block is formed inside the call from the
 * verify forward's final hidden states and the lm_head weight, and never
 * stored for greedy sequences.  The logits are those of the Gemma-4 drafter
 * code ("dspark-mlx 0.1.0" wheel diff, dspark_mlx/arch/gemma4.py): a
 * bias-free Linear(hidden_size, vocab_size) with weight [V, D] applied to
 * float32 hidden states, then the final-logit softcap c*tanh(a/c):
 *
 *   z[s, i, v] = softcap( sum_d hidden[s, i, d] * weight[v, d] ),  i = 0..K
 *
 * computed on the matrix cores from bf16 operands (products exact, sums in
 * float32, any order: within gamma_D * sum_d |hidden * weight| of the exact
 * sum, gamma_D = D 2^-24 / (1 - D 2^-24)); the softcap adds at most
 * 4 * 2^-23 * c.  Everything after the logits is spec_mixed_accept's
 * (per-sequence temperature, optional draft lengths), on float32 logits.
 *
 *   hidden        bf16 [b, K+1, D] (device), element strides h_batch_stride,
 *                 h_row_stride (multiples of 8), 16-byte aligned; it must span
 *                 fewer than 2^31 elements
 *   weight        bf16 [V, D] (device), row stride w_row_stride (a multiple of
 *                 8, >= D), 16-byte aligned
 *   D             a positive multiple of 64
 *   softcap       c >= 0 (0 = no softcap)
 *   draft         float32 [b, K, V] drafter logits (device), element strides
 *   workspace     spec_fused_workspace_bytes(b, K, V, D) bytes, 256-byte
 *                 aligned.  It holds, besides the partials, the float32 logits
 *                 of the sampling sequences (their residual or bonus draw
 *                 re-reads one row), b*(K+1)*ceil64(V)*4 bytes.
 * Other arguments and outputs as for spec_mixed_accept.  Seven kernels:
 * lm_head GEMM with statistics epilogue, tile merge, draft-row pass, scan,
 * residual pass, draw.  Errors as for spec_mixed_accept; misaligned
 * operands give SPEC_EALIGN.
 */
size_t spec_fused_workspace_bytes(int b, int K, int V, int D);

int spec_fused_mixed_accept(const void *hidden, int64_t h_batch_stride, int64_t h_row_stride,
                            const void *weight, int64_t w_row_stride, int D, float softcap,
                            const float *draft, int64_t d_batch_stride, int64_t d_row_stride,
                            const int32_t *draft_tokens, int b, int K, int V,
                            const double *temperatures, const int32_t *draft_lengths,
                            const uint64_t *seeds,
                            int32_t *n_accepted, int32_t *tokens,
                            float *p_draft, float *q_draft, int32_t *target_argmax,
                            void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * The fused call's GEMM alone: logits[r, v] = softcap(sum_d hidden[r, d] *
 * weight[v, d]) in float32 for rows r < rows, written with row stride
 * l_row_stride (a multiple of 4, >= V; logits 16-byte aligned).  Same
 * kernel, same arithmetic, as inside spec_fused_mixed_accept; for checking
 * the logits and for callers that want them.  hidden: bf16 [rows, D], row
 * stride h_row_stride.  Same argument rules otherwise.
 */
int spec_lm_head_logits(const void *hidden, int64_t h_row_stride, int rows,
                        const void *weight, int64_t w_row_stride, int V, int D, float softcap,
                        float *logits, int64_t l_row_stride, void *hip_stream);

/*
 * Vocabulary-sharded verify: the target and draft logits arrive split by
 * vocabulary column into G shards, as a tensor-parallel lm_head leaves them
 * (shard g holds columns [col0_g, col0_g + shard_V[g]) of every row, col0_g
 * the sum of the earlier widths), each shard in its own buffer.  The result
 * is spec_mixed_accept's on the concatenated vocabulary (global token ids).
 * Each shard runs the row pass and the residual pass on its own columns and
 * contributes one statistics record per row -- (max, first argmax) or (max,
 * sum of exp) -- and the draft-token logits it owns; the scan merges the G
 * records of a row in shard order; the G shard totals of the draw's weights
 * pick the shard that searches its columns for the drawn token.  On one GPU
 * the shards are plain buffers; across GPUs the records (b*(2K+1)*16 B), the
 * gathered logits (b*K*8 B) and the shard totals (b*G*8 B) are what would be
 * all-gathered, and the drawn tokens what would be broadcast.
 *
 *   G               1 .. SPEC_MAX_SHARDS
 *   target_shards   host array of G device pointers, shard g [b, K+1, shard_V[g]]
 *   draft_shards    host array of G device pointers, shard g [b, K, shard_V[g]]
 *   shard_V         host [G] widths (>= 1)
 *   t_strides       host [2G]: batch and row element strides of each target shard
 *   d_strides       host [2G]: same for the draft shards
 *   workspace       spec_sharded_workspace_bytes(G, shard_V, b, K, dtype) bytes
 * Other arguments and outputs as for spec_mixed_accept (V = sum of widths).
 */
#define SPEC_MAX_SHARDS 16

size_t spec_sharded_workspace_bytes(int G, const int *shard_V, int b, int K, int dtype);

int spec_sharded_mixed_accept(int G, const void *const *target_shards, const void *const *draft_shards,
                              const int *shard_V, const int64_t *t_strides, const int64_t *d_strides,
                              int dtype, const int32_t *draft_tokens, int b, int K,
                              const double *temperatures, const int32_t *draft_lengths,
                              const uint64_t *seeds, int32_t *n_accepted, int32_t *tokens,
                              float *p_draft, float *q_draft, int32_t *target_argmax,
                              void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Draft-side block decode with the Markov head -- the step that produces the
 * verify's draft block.  The parallel backbone's base logits L [b, K, V]
 * (float32) get, position by position, a rank-r correction conditioned on
 * the previous token ("dspark-mlx 0.1.0" README "How it works": a rank-256
 * previous-token correction sampled sequentially; "mlx-dspark 0.0.1"
 * __init__.py; the ds4 drafter card, "Files": the markov_w2 table read in
 * full per draft position):
 *
 *   u_i = w1[x_{i-1}]  (x_{-1} = anchors[s]),   q_i = L_i + w2 u_i,
 *   x_i = first argmax of q_i (temperature 0) or the inverse-CDF draw from
 *         softmax(q_i / T) at t = U R, U = Philox(seed, position i, row s, tag 2),
 *
 * the correction formed on the matrix cores (bf16 tables, fp32 sums).  With
 * hidden and conf_w, also the confidence head
 * conf_i = sigmoid(conf_w . [hidden_i ; u_i] + conf_b) and the draft length
 * = leading positions with conf_i >= threshold (K when threshold <= 0), the
 * draft_lengths input of spec_mixed_accept.
 *
 *   base            float32 [b, K, V] (element strides)
 *   anchors         int32 [b] (device): the last committed token
 *   w1, w2          bf16 [V, r] (device), r a positive multiple of 64, row
 *                   strides multiples of 8, 16-byte aligned; w2 row v holds the
 *                   table's entries for vocabulary entry v
 *   temperatures    double [b]: 0 greedy, > 0 sampling, else tokens -1
 *   seeds           uint64 [b]
 *   hidden          bf16 [b, K, D] and conf_w bf16 [D + r]; needed when confidence
 *                   or lengths is given (else SPEC_EINVAL), unused otherwise
 *   tokens          int32 [b, K] out; -1 from a position whose previous token
 *                   or logits are invalid on
 *   draft_logits    float32 [b, K, V] out (the corrected q_i), 16-byte aligned,
 *                   strides multiples of 4
 *   confidence      float [b, K] out or NULL; lengths int32 [b] out or NULL; the
 *                   confidence head runs when either is given
 *   workspace       spec_markov_workspace_bytes(b, K, V, r) bytes, 256-byte aligned
 * Two kernels per position (the correction on the matrix cores with the base
 * logits added, q_i stored and per-tile records; then per sequence the merge
 * of the tile records, the pick and the draw), then one kernel for the
 * confidences and the lengths.  For r <= 256 with 16-byte aligned base rows the correction kernel
 * is a persistent one-workgroup-per-CU stream; other shapes take a tiled
 * kernel with the same results.
 */
size_t spec_markov_workspace_bytes(int b, int K, int V, int r);

int spec_markov_block_decode(const float *base, int64_t base_batch_stride, int64_t base_row_stride,
                             const int32_t *anchors, const void *w1, int64_t w1_row_stride,
                             const void *w2, int64_t w2_row_stride, int r, int b, int K, int V,
                             const double *temperatures, const uint64_t *seeds,
                             const void *hidden, int64_t h_batch_stride, int64_t h_row_stride, int D,
                             const void *conf_w, float conf_b, float threshold,
                             int32_t *tokens, float *draft_logits, int64_t q_batch_stride,
                             int64_t q_row_stride, float *confidence, int32_t *lengths,
                             void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Profiling hook (not part of the accept semantics).  Registers, for the
 * calling host thread only, an array of n_events hipEvent_t handles.  While
 * registered, each accept call records events[0] before its first kernel and
 * events[k] after its k-th kernel on its stream (kernels: 1 row pass, 2 scan,
 * then for sampling and mixed calls 3 residual pass, 4 draw; for the fused
 * call 1 lm_head GEMM, 2 tile merge, 3 draft-row pass, 4 scan, 5 residual,
 * 6 draw; for the sharded call 1 row passes, 2 records + scan, 3 residual
 * passes + shard selection, 4 draws; for the Markov block decode 1 after all
 * positions, 2 after the confidence), for every k < n_events; n_events = 2
 * brackets the first kernel (the whole position loop for the Markov decode).  Pass NULL / 0 to
 * unregister.  Returns SPEC_OK.
 */
int spec_set_stage_events(void *const *events, int n_events);

/*
 * Diagnostic (not part of the accept semantics): the uniforms that the
 * accept test (tag 0) and the draws (tag 1; the Markov draft draws use tag 2)
 * take, from the library's own device Philox4x32-10, on a grid of counters:
 * out[r * npos + p] = U(seed, row0 + r, pos0 + p, tag), row and position
 * wrapping modulo 2^32.  out: device double [nrow * npos], 8-byte aligned.
 * For checking the device generator against an independent implementation.
 * Returns SPEC_EINVAL / SPEC_ELAUNCH on error.
 */
int spec_philox_uniforms(uint64_t seed, uint32_t row0, int nrow, uint32_t pos0, int npos, uint32_t tag,
                         double *out, void *hip_stream);

/*
 * Plain device copy of nbytes (a multiple of 16, 16-byte aligned pointers)
 * with the same 16-byte load path as the row pass, enqueued on hip_stream.
 * Used to calibrate hardware byte counters and to measure the achievable
 * streaming bandwidth.  Returns SPEC_EINVAL / SPEC_ELAUNCH on error.
 */
int spec_stream_copy(void *dst, const void *src, size_t nbytes, void *hip_stream);

/*
 * Read-only stream over nbytes at src (a multiple of 16, 16-byte aligned)
 * with the row pass's shape: one single-wave workgroup per 16 KiB, 16
 * nontemporal 16-byte loads per lane issued together.  It measures the
 * achievable read bandwidth that the row pass is compared with.  sink (a
 * device word, 4-byte aligned) is written only if the folded data equal one
 * fixed value, so the loads are kept; its contents are otherwise untouched.
 * Returns SPEC_EINVAL / SPEC_ELAUNCH on error.
 */
int spec_stream_read(const void *src, size_t nbytes, uint32_t *sink, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
