/*
 * mla.h - C ABI of the MI355X (gfx950) Multi-head Latent Attention hot path.
 *
 * The method (DeepSeek-V2 MLA) caches, per token, one joint KV latent
 * c^KV = W^DKV h (width d_c = 512) and one decoupled RoPE key k^R shared by
 * all heads (width d_R = 64), instead of per-head keys and values
 * ("A. Conclusion, Limitation, and Future" DeepSeek-V2 notes,
 * irregular6612.github.io, §2.1.2 eq. 9-11; DeepSeek-V2 MLA blog,
 * adg.csdn.net, part 2 §2.2.2).  Attention is evaluated in the weight-absorbed
 * form: W^UK is folded into the query, W^UV is applied after the softmax sum
 * (same blog, §2.2.1.1 and §2.2.2: by associativity neither keys nor values
 * need to be materialised).  Per query row t and head i:
 *
 *   q_lat_i = [ W^UK_i^T q_nope_i ; R_{pos t} q_rope_i ]           (576)
 *   row_j   = [ c^KV_j ; R_{pos j} k_rope_j ]                       (576, cached)
 *   s_ij    = scale * q_lat_i . row_j
 *   o_lat_i = sum_j softmax_j(s_ij) c^KV_j                           (512)
 *   o_i     = W^UV_i o_lat_i                                         (128)
 *
 * which equals eq. 7 ("standard MHA" softmax attention, §2.1.1 of the notes)
 * applied to the per-head keys [W^UK_i c^KV_j ; k^R_j] and values W^UV_i c^KV_j.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Widths are fixed by the pages for both DeepSeek-V2 and V2-Lite: d_c = 512,
 *   d_R = 64, d_h = 128 (blog part 3 §3.1.1 and the V2-Lite description in part 2).
 * - dtype: MLA_F32 (IEEE float) or MLA_BF16 (bfloat16 as raw 16-bit words).
 *   Arithmetic is fp32 in both cases (products of bf16 operands are exact in
 *   fp32; sums accumulate in fp32).  o_lat, lse, partials and the output are
 *   always fp32.
 * - RoPE (reading of blog §2.2.2, which only fixes R_m^T R_n = R_{n-m}): adjacent
 *   element pairs (x[2k], x[2k+1]) are rotated by angle pos * theta_k,
 *   k = 0..31, theta_k = base^(-2k/64); angles are formed in float64.  Every
 *   entry point that rotates takes `float rope_base` and
 *   `const double* rope_theta`: a host array of the 32 pair frequencies
 *   (radians per position) that, when not NULL, replaces base^(-2k/64)
 *   (rope_base is then unused), e.g. the YaRN table of mla_rope_theta.  Use
 *   one table for the keys and the queries of a model.  A table entry (or a
 *   rope_base) that is not finite and positive gives MLA_ERR_SHAPE.
 * - Paged cache: kv_cache is [num_blocks, block_size, 576] elements of dtype,
 *   rows contiguous (a bf16 row is 1152 bytes = 72 x 16 bytes).  Token j of
 *   sequence b lives in block block_table[b * max_blocks + j / block_size],
 *   row j % block_size.  block_size must be 64.
 * - Pointers named "device" are HIP device memory owned by the caller; the
 *   library never allocates, frees or synchronises.  "host" pointers are read
 *   or written synchronously during the call.
 * - stream: a hipStream_t (NULL = the null stream).  Every device call only
 *   enqueues work on it and returns.
 * - Errors: argument checks (null pointers, sizes, alignment, dtype) happen on
 *   the host before anything is enqueued and return a status != MLA_OK with
 *   nothing enqueued.  A failed launch returns MLA_ERR_HIP.  Device-resident
 *   integers (block ids, lengths, positions) cannot be checked on the host;
 *   the kernels skip entries that point outside the cache (a block id outside
 *   [0, num_blocks) contributes no keys and receives no rows) instead of
 *   faulting.  No C++ exception crosses this interface.  All entry points are
 *   thread-safe: the library holds no mutable global state, apart from the
 *   per-device scratch array of mla_decode_paged_noalloc and the per-thread
 *   timing events of mla_time_attention (see there).
 */
#ifndef MLA_LATENT_KV_MLA_H
#define MLA_LATENT_KV_MLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 5

#define MLA_D_C 512
#define MLA_D_R 64
#define MLA_D_H 128
#define MLA_ROW 576
#define MLA_BLOCK 64
/* Segment cost of mla_plan_decode's schedule, in blocks. */
#define MLA_PLAN_SEGMENT_COST 8

enum mla_dtype { MLA_F32 = 0, MLA_BF16 = 1 };

enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,   /* a required pointer is NULL */
  MLA_ERR_SHAPE = 2,  /* a size is out of range or inconsistent */
  MLA_ERR_ALIGN = 3,  /* a pointer is not 16-byte aligned */
  MLA_ERR_DTYPE = 4,  /* unknown dtype */
  MLA_ERR_HIP = 5,    /* the HIP runtime refused a launch */
  MLA_ERR_SCRATCH = 6 /* the problem needs more than the library's fixed scratch */
};

/* Static text for a status code (never NULL). */
const char* mla_status_string(int32_t status);

/* MLA_ABI_VERSION of the loaded library. */
int32_t mla_abi_version(void);

/*
 * mla_rope_theta - RoPE pair frequencies with YaRN's interpolation by parts.
 *
 * DeepSeek-V2 extends its 4K context to 128K by applying YaRN to the
 * decoupled shared key only, with scale s = 40, ramp bounds alpha = 1 and
 * beta = 32, aiming at 160K = 40 x 4K (DeepSeek-V2 MLA blog, part 3 §3.1.3).
 * Read as YaRN's by-parts rule: pair k of plain RoPE, f_k = base^(-2k/64),
 * makes r_k = orig_ctx * f_k / (2 pi) turns over the original window; with
 * g_k = clamp((r_k - alpha) / (beta - alpha), 0, 1),
 *   theta[k] = g_k * f_k + (1 - g_k) * f_k / scale,      k = 0..31,
 * so fast pairs (r_k >= beta) keep their frequency and slow pairs
 * (r_k <= alpha) are slowed by s.  scale = 1 gives plain RoPE.  YaRN's
 * attention-temperature factor multiplies every score, so it belongs in the
 * softmax scale the caller passes to the attention entry points.
 *
 * theta  host, double [32] (written)
 * Host arithmetic only: no device call.  MLA_ERR_NULL if theta is NULL;
 * MLA_ERR_SHAPE unless base > 1, scale >= 1, 0 <= alpha < beta and
 * orig_ctx > 0, all finite.
 */
int32_t mla_rope_theta(double base, double scale, double alpha, double beta, double orig_ctx,
                       double* theta);

/*
 * mla_kv_append - write n new tokens into the paged latent cache.
 *
 * The cache keeps c^KV unrotated and k^R already rotated at the token's
 * position, so attention needs no key RoPE (blog part 2 §2.2.2: the RoPE'd key
 * part is cached; RoPE may not touch the compressed latent).  For r < n:
 *   slot  = block_table[seq_idx[r] * max_blocks + pos[r] / 64] * 64 + pos[r] % 64
 *   cache[slot] = [ c_kv[r, 0:512] ; R_{pos[r]} k_rope[r, 0:64] ]
 * The RoPE position of a token is its index in its sequence.
 *
 * kv_cache    device, [num_blocks, 64, 576] dtype, 16-byte aligned (written)
 * block_table device, int32 [num_seqs, max_blocks]
 * c_kv        device, [n, 512] dtype (contiguous)
 * k_rope      device, [n, 64] dtype, before rotation
 * seq_idx     device, int32 [n]; pos device, int32 [n] (>= 0)
 * Rows whose seq_idx is outside [0, num_seqs), whose pos < 0 or
 * pos / 64 >= max_blocks, or whose block id is outside [0, num_blocks) are not
 * written.  Two rows aimed at one slot race.
 * n == 0 is a no-op.
 */
int32_t mla_kv_append(void* kv_cache, int32_t dtype, int32_t num_blocks, int32_t block_size,
                      const int32_t* block_table, int32_t num_seqs, int32_t max_blocks,
                      const void* c_kv, const void* k_rope,
                      const int32_t* seq_idx, const int32_t* pos, int32_t n,
                      float rope_base, const double* rope_theta, void* stream);

/*
 * mla_absorb_q - latent-space queries (W^UK absorbed into the query).
 *
 * For every row t < T and head i < n_h:
 *   q_lat[t, i, 0:512]   = W^UK_i^T q_nope[t, i, :]      (eq. 10 moved to the query)
 *   q_lat[t, i, 512:576] = R_{q_pos[t]} q_rope[t, i, :]  (decoupled RoPE query)
 * w_uk holds W^UK as [n_h, 128, 512]: head i's block is rows i*128..(i+1)*128
 * of eq. 10's matrix (eq. 4-6 head ordering).  Accumulation is fp32; q_lat is
 * rounded to dtype (round to nearest even for bf16).
 *
 * q_nope device [T, n_h, 128]; q_rope device [T, n_h, 64]; w_uk device
 * [n_h, 128, 512]; q_pos device int32 [T]; q_lat device out [T, n_h, 576];
 * all of dtype except q_pos, all contiguous and 16-byte aligned.
 * n_h must be a multiple of 16.  T == 0 is a no-op.
 */
int32_t mla_absorb_q(const void* q_nope, const void* q_rope, const void* w_uk,
                     const int32_t* q_pos, int32_t T, int32_t n_h, int32_t dtype,
                     float rope_base, const double* rope_theta, void* q_lat, void* stream);

/*
 * mla_append_absorb_q - the two calls that open a decode step, in one launch:
 * mla_kv_append (the step's n new rows into the cache) and mla_absorb_q (the
 * step's T latent queries), with the same dtype and RoPE frequencies.  The
 * arguments, layouts, results and skipped rows are those of the two calls;
 * each part is checked as its call checks it, and only when it is not empty
 * (n > 0, T > 0): an error in either returns its status with nothing
 * enqueued.  The two parts run concurrently, so the cache must not overlap
 * q_lat, q_nope, q_rope or w_uk.  Between the two operations of a step
 * (DeepSeek-V2 MLA blog, adg.csdn.net, part 2 §2.2.2: the new token's latent
 * row and rotated key are cached, and its query is absorbed into latent
 * space) there is no data dependence; one launch saves a kernel boundary.
 * bf16 runs as one kernel; fp32 as the two launches.
 */
int32_t mla_append_absorb_q(void* kv_cache, int32_t num_blocks, int32_t block_size,
                            const int32_t* block_table, int32_t num_seqs, int32_t max_blocks,
                            const void* c_kv, const void* k_rope, const int32_t* seq_idx,
                            const int32_t* pos, int32_t n, const void* q_nope,
                            const void* q_rope, const void* w_uk, const int32_t* q_pos,
                            int32_t T, int32_t n_h, int32_t dtype, float rope_base,
                            const double* rope_theta, void* q_lat, void* stream);

/*
 * mla_decode_paged - attention of latent queries over the paged cache.
 *
 * Query rows: q_lat [B, q_len, n_h, 576] (dtype).  Row m of sequence b sees
 * keys j < seq_lens[b] - (q_len - 1 - m): with q_len == 1 a decode query
 * sees all seq_lens[b] cached keys; with q_len > 1 (chunked prefill) the chunk
 * is the last q_len keys and each row sees keys up to its own position
 * (eq. 7's sum over j <= t).  seq_lens[b] is clamped to max_blocks * 64.
 *   s_j = softmax_scale * q_lat . row_j; o_lat = sum_j softmax_j(s) row_j[0:512]
 *   lse = log sum_j exp(s_j)   (natural log; -inf and o_lat = 0 for a row
 *                                that sees no key)
 *
 * Split-KV: with num_splits = S > 1 each row's keys are cut as in
 * mla_split_plan (per sequence, on seq_lens[b]; a row's range is further cut
 * at its own visible length) and every split writes its normalised partial
 * o_part [B, S, q_len, n_h, 512] and lse_part [B, S, q_len, n_h] (fp32);
 * o_lat/lse are then not written (run mla_splitkv_combine).  With S == 1
 * o_part/lse_part may be NULL and o_lat [B, q_len, n_h, 512], lse
 * [B, q_len, n_h] are written directly.
 *
 * n_h must be 16, 32 or a multiple of 64.  q_lat and kv_cache must be
 * 16-byte aligned.  softmax_scale is taken as given; the pages' reading is
 * 1/sqrt(d_h + d_R) = 1/sqrt(192), the width of the concatenated query/key.
 */
int32_t mla_decode_paged(const void* q_lat, const void* kv_cache, int32_t num_blocks,
                         int32_t block_size, const int32_t* block_table, int32_t max_blocks,
                         const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t n_h,
                         int32_t dtype, float softmax_scale, int32_t num_splits,
                         float* o_part, float* lse_part, float* o_lat, float* lse,
                         void* stream);

/*
 * mla_splitkv_combine - merge split-KV partials.
 *
 * Softmax over a partition of the keys is recovered exactly from per-split
 * normalised outputs and log-sum-exps:
 *   LSE = log sum_s exp(lse_s),  o = sum_s exp(lse_s - LSE) o_s.
 * Splits with lse_s = -inf carry weight 0; if every split is empty, o = 0 and
 * LSE = -inf.  o_part device fp32 [B, S, q_len, n_h, 512]; lse_part device fp32
 * [B, S, q_len, n_h]; o_lat device out fp32 [B, q_len, n_h, 512]; lse device
 * out fp32 [B, q_len, n_h] (may be NULL).
 */
int32_t mla_splitkv_combine(const float* o_part, const float* lse_part, int32_t B, int32_t S,
                            int32_t q_len, int32_t n_h, float* o_lat, float* lse, void* stream);

/*
 * mla_out_proj - per-head output o_i = W^UV_i o_lat_i (eq. 11's W^UV applied
 * after the softmax sum; the result is eq. 7's per-head output, the input of
 * eq. 8's W^O, which is not applied here).
 *
 * o_lat device fp32 [T, n_h, 512]; w_uv device [n_h, 128, 512] dtype (head i's
 * block is rows i*128..(i+1)*128 of eq. 11's matrix); out device fp32
 * [T, n_h, 128].  For bf16 weights o_lat is split as hi + lo with
 * hi = bf16(x), lo = bf16(x - hi), so 16 significant bits of o_lat enter the
 * product instead of 8.
 * T == 0 is a no-op.
 */
int32_t mla_out_proj(const float* o_lat, const void* w_uv, int32_t T, int32_t n_h,
                     int32_t dtype, float* out, void* stream);

/*
 * mla_split_plan - the split-KV key ranges, on the host.
 *
 * For sequence b with L = seq_lens[b] keys and nblk = ceil(L / 64) blocks,
 * c = ceil(nblk / S); split s covers keys [min(s*c*64, L), min((s+1)*c*64, L)).
 * begin_end (host, int32 [B, S, 2]) receives the ranges; empty splits have
 * begin == end.  seq_lens host int32 [B], each >= 0.
 */
int32_t mla_split_plan(const int32_t* seq_lens, int32_t B, int32_t block_size, int32_t num_splits,
                       int32_t* begin_end);

/*
 * mla_plan_decode - a load-balanced split-KV schedule, on the host.
 *
 * Rows r = b * q_len + m; row r sees n_r keys (the visibility rule of
 * mla_decode_paged, with seq_lens[b] clamped at 0) and spans T_r = ceil(n_r / 64)
 * blocks.  Lay the rows' blocks end to end (row 0 first): row r occupies
 * positions [S_r, S_r + T_r) of a sequence of N = sum_r T_r blocks.  With
 * G = n_h / 64 workgroups per unit of work when n_h is a multiple of 64 (else
 * G = 1), K = max(1, min(floor(num_slots / G), N)) lists (K = 1 when N = 0)
 * cover the positions in order, list k owning [b_k, b_{k+1}).  A list costs its
 * blocks plus C = MLA_PLAN_SEGMENT_COST per segment (the fixed price of
 * starting a row: its query, the first tiles, its output).  The boundaries
 * come from a greedy walk with capacity W: a list starts where the previous
 * one ended and takes the rest of the current row while its cost stays
 * <= W; the first rest that does not fit is cut after W - cost - C blocks when
 * that is >= 1, and the list closes.  W is the least capacity for which the
 * walk needs at most K lists (so the costliest list is as cheap as any
 * partition into K ordered lists allows); lists past the last one the walk
 * fills are empty (b_k = N).  A row whose blocks fall in lists k0..k1 is cut
 * at the list boundaries into k1 - k0 + 1 segments; a row with no block is one
 * empty segment in the last list with b_k <= S_r (the last list if S_r = N).
 * Segment keys are [64 t0, min(64 t1, n_r)) for its blocks [t0, t1) of the
 * row.
 *
 *   work  (host out, int32 [n_work, 4]) = {row, key_begin, key_end, slot},
 *         ordered by list, then row; slot = -1 for a row in one segment (its
 *         output goes straight to o_lat), else the segments of a cut row get
 *         consecutive partial slots (cut rows in increasing row order).
 *   lists (host out, int32 [n_lists + 1], at most num_slots + 1 entries):
 *         list k is work items lists[k] .. lists[k+1] - 1; lists[n_lists] = n_work.
 *   split (host out, int32 [n_split, 3]) = {row, first_slot, count} for every
 *         cut row, in row order; n_parts = number of partial slots.
 * max_work bounds work and split; if the plan needs more, MLA_ERR_SHAPE is
 * returned and *n_work holds the required size.  num_slots: workgroups the
 * device runs at once (e.g. its compute-unit count).  Pure integer host code.
 */
int32_t mla_plan_decode(const int32_t* seq_lens, int32_t B, int32_t q_len, int32_t block_size,
                        int32_t n_h, int32_t num_slots, int32_t max_work, int32_t* work,
                        int32_t* n_work, int32_t* lists, int32_t* n_lists, int32_t* split,
                        int32_t* n_split, int32_t* n_parts);

/*
 * mla_decode_paged_planned - mla_decode_paged over a schedule from
 * mla_plan_decode (work and lists copied to the device).  Item i scores its
 * row's query against keys [key_begin, key_end) of the row's sequence
 * (b = row / q_len) and writes o_lat/lse row `row` when slot < 0, else
 * o_part/lse_part row `slot` (fp32 [n_parts, n_h, 512] / [n_parts, n_h]).
 * n_parts >= 0 is the number of partial rows the caller provides (o_part and
 * lse_part may be NULL only when it is 0); an item whose slot is >= n_parts,
 * or whose row is outside [0, B * q_len), is skipped on the device and
 * writes nothing.
 * lists (device int32 [n_lists + 1], may be NULL): the items of each list are
 * run in order by one workgroup per 64 heads; results do not depend on it
 * (NULL runs one item per workgroup).  Other arguments as in
 * mla_decode_paged; key ranges are clamped to max_blocks * 64.
 */
int32_t mla_decode_paged_planned(const void* q_lat, const void* kv_cache, int32_t num_blocks,
                                 int32_t block_size, const int32_t* block_table,
                                 int32_t max_blocks, int32_t B, int32_t q_len, int32_t n_h,
                                 int32_t dtype, float softmax_scale, const int32_t* work,
                                 int32_t n_work, const int32_t* lists, int32_t n_lists,
                                 float* o_part, float* lse_part, int32_t n_parts, float* o_lat,
                                 float* lse, void* stream);

/*
 * mla_combine_planned - merge the partials of every split row of a plan
 * (split device int32 [n_split, 3] from mla_plan_decode), with the same
 * log-sum-exp rule as mla_splitkv_combine, into o_lat / lse rows.
 */
int32_t mla_combine_planned(const float* o_part, const float* lse_part, const int32_t* split,
                            int32_t n_split, int32_t n_h, float* o_lat, float* lse, void* stream);

/*
 * mla_out_proj_planned - mla_combine_planned followed by mla_out_proj, in one
 * launch for bf16 weights: the split rows of a plan (split device int32
 * [n_split, 3] from mla_plan_decode, rows distinct and increasing) are merged
 * from o_part / lse_part with the log-sum-exp rule of mla_splitkv_combine
 * (as they are loaded for T > 64; into on-chip memory, a few rows per
 * workgroup, for T <= 64), and their LSE is written to lse (device fp32
 * [T, n_h], may be NULL); every other row is read from o_lat.  The merged
 * rows of o_lat are scratch: after the call they hold either the merged value
 * (fp32 weights, where the two steps run one after the other) or what they
 * held before.
 * Other arguments, layouts and the bf16 hi + lo split of the operand as in
 * mla_out_proj.  0 <= n_split <= T; T == 0 is a no-op.
 */
int32_t mla_out_proj_planned(float* o_lat, const float* o_part, const float* lse_part,
                             const int32_t* split, int32_t n_split, const void* w_uv, int32_t T,
                             int32_t n_h, int32_t dtype, float* out, float* lse, void* stream);

/*
 * Producers: the projections that feed the path from a layer's hidden states
 * h [T, d_model] (notes §2.1.2 eq. 9 and 12-13; blog part 2 §2.2.2 for the
 * decoupled key and query, part 3 §3.1.1 for the RMSNorm after the compressed
 * latents).  The RMSNorm is the standard one over the latent's width:
 *   RMSNorm(x) = g * x / sqrt(mean(x^2) + eps), g a learned gain (fp32).
 * Weights are stored as the equations write them, [d_out, d_in] row-major,
 * in the element type dtype; h is [T, d_model] in dtype.  Products
 * accumulate in fp32.  d_model and d_cq are multiples of 64 (d_cq <= 2048),
 * and every operand's element count (T * d_model, T * d_cq, n_h * 128 * d_cq)
 * stays below 2^29 (else MLA_ERR_SHAPE).  q_nope and q_rope are 16-byte
 * aligned.
 * Each call takes a caller-owned device workspace of at least the size the
 * matching *_workspace function returns (-1 there: invalid sizes); a smaller
 * one is MLA_ERR_SHAPE.  The library allocates nothing.
 */

/* Workspace bytes of mla_kv_produce for T tokens of width d_model. */
int64_t mla_kv_produce_workspace(int32_t T, int32_t d_model);

/*
 * mla_kv_produce - cache rows of T new tokens, written like mla_kv_append:
 *   c^KV = RMSNorm(W^DKV h) (gain kv_gain [512], eps),  k^R = W^KR h,
 *   cache[slot(seq_idx[r], pos[r])] = [ c^KV_r ; R_{pos[r]} k^R_r ]
 * w_dkv [512, d_model], w_kr [64, d_model]; cache, block_table, seq_idx, pos,
 * rope_base and the skipping of out-of-range rows as in mla_kv_append.
 */
int32_t mla_kv_produce(const void* h, const void* w_dkv, const float* kv_gain, const void* w_kr,
                       int32_t T, int32_t d_model, int32_t dtype, float eps, float rope_base,
                       const double* rope_theta, void* kv_cache, int32_t num_blocks,
                       int32_t block_size,
                       const int32_t* block_table, int32_t num_seqs, int32_t max_blocks,
                       const int32_t* seq_idx, const int32_t* pos, void* workspace,
                       int64_t workspace_bytes, void* stream);

/* Workspace bytes of mla_q_produce. */
int64_t mla_q_produce_workspace(int32_t T, int32_t d_model, int32_t d_cq, int32_t dtype);

/*
 * mla_q_produce - per-head queries of T tokens through the compressed query:
 *   c^Q = RMSNorm(W^DQ h) (gain q_gain [d_cq], eps),
 *   q_nope = W^UQ c^Q  -> [T, n_h, 128],  q_rope = W^QR c^Q -> [T, n_h, 64]
 * (q_rope before rotation: mla_absorb_q rotates it).  w_dq [d_cq, d_model],
 * w_uq [n_h * 128, d_cq], w_qr [n_h * 64, d_cq], head i owning rows i*128..
 * and i*64..; c^Q is rounded to dtype before its up-projections.
 */
int32_t mla_q_produce(const void* h, const void* w_dq, const float* q_gain, const void* w_uq,
                      const void* w_qr, int32_t T, int32_t d_model, int32_t d_cq, int32_t n_h,
                      int32_t dtype, float eps, void* q_nope, void* q_rope, void* workspace,
                      int64_t workspace_bytes, void* stream);

/*
 * mla_q_produce_direct - per-head queries of T tokens for a model that does
 * not compress its queries (DeepSeek-V2-Lite: blog, the V2-Lite paragraph):
 *   q_nope = W^QC h -> [T, n_h, 128] (eq. 1's W^Q, head i owning rows i*128..),
 *   q_rope = W^QR h -> [T, n_h, 64] (before rotation; head i rows i*64..).
 * w_qc [n_h * 128, d_model], w_qr [n_h * 64, d_model], h [T, d_model], all
 * in dtype; fp32 accumulation.  No workspace.  d_model a multiple of 64.
 */
int32_t mla_q_produce_direct(const void* h, const void* w_qc, const void* w_qr, int32_t T,
                             int32_t d_model, int32_t n_h, int32_t dtype, void* q_nope,
                             void* q_rope, void* stream);

/*
 * mla_o_proj - the layer output of eq. 8 (notes §2.1.1):
 *   u[t] = W^O [o_{t,1}; ...; o_{t,n_h}]
 * out: fp32 [T, n_h, 128] as mla_out_proj writes it; w_o [d_model, n_h * 128]
 * in dtype; u [T, d_model] in dtype.  In bf16 the heads' outputs are rounded
 * to bf16 once to feed the MFMA (fp32 accumulation).  The caller's workspace
 * holds that copy and split-K partials: at least mla_o_proj_workspace bytes
 * (-1 there: invalid sizes; 0 is possible, then workspace may be NULL).
 * d_model a multiple of 64.
 */
int64_t mla_o_proj_workspace(int32_t T, int32_t n_h, int32_t d_model, int32_t dtype);
int32_t mla_o_proj(const float* out, const void* w_o, int32_t T, int32_t n_h, int32_t d_model,
                   int32_t dtype, void* u, void* workspace, int64_t workspace_bytes,
                   void* stream);

/*
 * Non-absorbed chunked prefill: the literal form of eq. 7 (notes §2.1.1) with
 * the per-head keys and values of eq. 10-11 (notes §2.1.2),
 *   k^C_{j,i} = W^UK_i c^KV_j,  v^C_{j,i} = W^UV_i c^KV_j,
 *   q_i = [q_nope_i ; R_{q_pos} q_rope_i],  k_{j,i} = [k^C_{j,i} ; k^R_j]
 * (k^R_j as cached, already rotated; blog part 2 §2.2.2), softmax over the
 * visible keys at `scale`, o_i = sum_j p_j v^C_{j,i}.  The blog keeps the
 * absorbed form for generation; for a chunk of many query rows this form
 * costs 2 (192 + 128) instead of 2 (576 + 512) flops per (row, head, key),
 * plus the up-projection of each key once.
 *
 * Same problem as mla_absorb_q + mla_decode_paged + mla_out_proj for one
 * chunk of q_len rows per sequence: q_nope [B * q_len, n_h, 128] and q_rope
 * [B * q_len, n_h, 64] (before rotation) in bf16, q_pos device int32
 * [B * q_len]; w_uk, w_uv bf16 [n_h, 128, 512]; the paged cache, block_table
 * and block_size as for mla_decode_paged; seq_lens a HOST int32 array [B]
 * (keys of each sequence; row m of sequence b sees keys
 * j < seq_lens[b] - (q_len - 1 - m)).  Outputs: out fp32 [B * q_len, n_h, 128]
 * (as mla_out_proj's), lse fp32 [B * q_len, n_h] (natural log; a row with no
 * visible key gets out = 0 and lse = -inf).  A block id outside
 * [0, num_blocks) contributes no keys.  bf16 only (else MLA_ERR_DTYPE).
 * seq_lens[b] <= max_blocks * 64 and num_blocks * 64 * 1152 < 2^32 bytes
 * (else MLA_ERR_SHAPE).  The workspace (caller-owned device memory of at
 * least mla_prefill_mha_workspace(max seq_len, n_h) bytes) holds k^C and
 * v^C of one sequence at a time; sequences run one after the other on the
 * stream.
 */
int64_t mla_prefill_mha_workspace(int32_t max_seq_len, int32_t n_h);
int32_t mla_prefill_mha(const void* q_nope, const void* q_rope, const int32_t* q_pos,
                        const void* w_uk, const void* w_uv, const void* kv_cache,
                        int32_t num_blocks, int32_t block_size, const int32_t* block_table,
                        int32_t max_blocks, const int32_t* seq_lens, int32_t B, int32_t q_len,
                        int32_t n_h, int32_t dtype, float scale, float rope_base,
                        const double* rope_theta, float* out, float* lse, void* workspace,
                        int64_t workspace_bytes, void* stream);

/*
 * Quantised latent cache (DeepSeek-V2 MLA blog, part 3 §3.1.4: the served
 * model's KV cache is quantised, about 6 bits per element on average, scheme
 * not given).  Here: OCP FP8 E4M3 per element (bias 7, subnormals, largest
 * finite 448, no infinities; the gfx950 conversion format) with two float32
 * scales per token, one for the 512 latent elements and one for the 64
 * rotated RoPE elements.
 *   kv_cache  device, uint8 [num_blocks, 64, 576] E4M3 codes, rows contiguous
 *             (576 bytes = 36 x 16), 16-byte aligned
 *   kv_scale  device, float32 [num_blocks, 64, 2] = {s_latent, s_rope} per
 *             row, 16-byte aligned
 * Row j stands for [s_latent * c ; s_rope * r], c and r its E4M3 values.
 * 584 bytes per token against 1152 for bf16.
 *
 * mla_kv_append_fp8 - mla_kv_append into the quantised cache.  The float32
 * row [c_kv ; R_pos k_rope] (rotation formed in float64, then rounded to
 * float32) is quantised per part: amax = max |x|, s = amax / 448 (float32
 * division; s = 1 when amax = 0), code = E4M3 nearest-even of the float32
 * quotient x / s, clamped to +-448.  c_kv / k_rope are dtype (MLA_F32 or
 * MLA_BF16); slot rule, skipping and RoPE table as in mla_kv_append.
 */
int32_t mla_kv_append_fp8(void* kv_cache, float* kv_scale, int32_t dtype, int32_t num_blocks,
                          int32_t block_size, const int32_t* block_table, int32_t num_seqs,
                          int32_t max_blocks, const void* c_kv, const void* k_rope,
                          const int32_t* seq_idx, const int32_t* pos, int32_t n, float rope_base,
                          const double* rope_theta, void* stream);

/*
 * mla_decode_paged_fp8 / mla_decode_paged_planned_fp8 - mla_decode_paged and
 * mla_decode_paged_planned over the quantised cache: the attention of
 * mla_decode_paged with row j replaced by its dequantised value.  q_lat is
 * bf16 [B * q_len, n_h, 576]; outputs and partials as there.  Scores take
 * s_latent and s_rope per token on the two parts of the product; the
 * softmax weight of token j in the value sum is rounded to bf16 after
 * multiplication by its s_latent (an MFMA operand), and the normaliser sums
 * those same weights divided by s_latent, so the output is an exact
 * weighted mean of the dequantised latents.  Head counts as in
 * mla_decode_paged; lists as in mla_decode_paged_planned (used with 64 heads
 * or more).
 */
int32_t mla_decode_paged_fp8(const void* q_lat, const void* kv_cache, const float* kv_scale,
                             int32_t num_blocks, int32_t block_size, const int32_t* block_table,
                             int32_t max_blocks, const int32_t* seq_lens, int32_t B,
                             int32_t q_len, int32_t n_h, float softmax_scale, int32_t num_splits,
                             float* o_part, float* lse_part, float* o_lat, float* lse,
                             void* stream);
int32_t mla_decode_paged_planned_fp8(const void* q_lat, const void* kv_cache,
                                     const float* kv_scale, int32_t num_blocks,
                                     int32_t block_size, const int32_t* block_table,
                                     int32_t max_blocks, int32_t B, int32_t q_len, int32_t n_h,
                                     float softmax_scale, const int32_t* work, int32_t n_work,
                                     const int32_t* lists, int32_t n_lists, float* o_part,
                                     float* lse_part, int32_t n_parts, float* o_lat, float* lse,
                                     void* stream);

/*
 * mla_decode_paged_noalloc - for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): mla_decode_paged followed, when num_splits > 1, by
 * mla_splitkv_combine, with the split partials kept in a device array that
 * the library itself holds, MLA_NOALLOC_SCRATCH_BYTES per GPU, from the
 * first call on that GPU until the process ends.  The caller passes only the
 * inputs and the merged outputs o_lat [B, q_len, n_h, 512] and lse
 * [B, q_len, n_h] (fp32, device).  Arguments, layouts and results are those
 * of mla_decode_paged with num_splits == 1 (the result of a split call
 * equals mla_decode_paged with num_splits partials merged by
 * mla_splitkv_combine).  The partials take B * num_splits * q_len * n_h *
 * 513 * 4 bytes; a call that needs more than MLA_NOALLOC_SCRATCH_BYTES
 * returns MLA_ERR_SCRATCH with nothing enqueued.  No allocation, free or
 * synchronisation happens.  All calls on one GPU share its array: calls that
 * overlap on one GPU (other streams or host threads) race and must be
 * ordered by the caller.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
int32_t mla_decode_paged_noalloc(const void* q_lat, const void* kv_cache, int32_t num_blocks,
                                 int32_t block_size, const int32_t* block_table,
                                 int32_t max_blocks, const int32_t* seq_lens, int32_t B,
                                 int32_t q_len, int32_t n_h, int32_t dtype, float softmax_scale,
                                 int32_t num_splits, float* o_lat, float* lse, void* stream);

/*
 * mla_time_attention - kernel timing, for benchmarks and profilers that time
 * the attention kernel inside a running pipeline.  The events (hipEvent_t
 * handles created by the caller on the current device, timing enabled) are
 * armed for the calling host thread: the next attention kernel that thread
 * launches (the paged-attention kernel of mla_decode_paged,
 * mla_decode_paged_planned, mla_decode_paged_fp8,
 * mla_decode_paged_planned_fp8 or mla_decode_paged_noalloc) is dispatched
 * with them (hipExtLaunchKernel): `start` records the time that kernel starts
 * and `stop` the time it ends, so hipEventElapsedTime(start, stop) is its
 * duration.  Unlike hipEventRecord around the call, no timing packet is queued
 * between the kernels, so the timed pipeline runs as it does untimed.  The
 * launch disarms; a call that launches no attention kernel (no work, or an
 * argument error) leaves the events armed.  Arming again replaces the armed
 * pair; mla_time_attention(NULL, NULL) disarms.  Either event may be NULL.
 * Returns MLA_OK; the events are not checked here (a launch with an invalid
 * event returns MLA_ERR_HIP).  Other host threads are unaffected.
 */
int32_t mla_time_attention(void* start_event, void* stop_event);

#ifdef __cplusplus
}
#endif

#endif /* MLA_LATENT_KV_MLA_H */
