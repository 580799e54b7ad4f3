/*
 * lrkv.h -- C ABI of the LRKV (low-rank key-value attention) decode library
 * for AMD Instinct MI355X (gfx950).
 *
 * The method: every head's key and value projections are a shared dense
 * projection plus a per-head rank-r residual, W_h = W_shared + U_h B_h^T
 * ("Low-Rank Key Value Attention: Chinese reading notes", sec. 2.1,
 * Eqs. (2)-(5); "Low-Rank Key Value Attention | What a shared cache can
 * preserve", sec. 3).  The decode cache therefore holds, per token, one shared
 * key row and one shared value row (d_h wide each) and, per head, a key latent
 * and a value latent (r wide each).  Decoding never rebuilds per-head keys or
 * values: it absorbs B^K into the query, adds the shared and private logits
 * before a single softmax, and maps the weighted private value sum through
 * B^V once per head (reading notes sec. 2.4, Eqs. (6)-(7); review sec. 3,
 * "Associative decode" and Algorithm 2).
 *
 * Conventions for every entry point
 * ---------------------------------
 * Pointers named "device" point to GPU memory allocated by the caller; the
 * library never allocates, frees or retains them after the call returns.
 * All tensors are dense, row-major, without padding between rows.  Unless a
 * function says otherwise, device pointers must be 16-byte aligned.
 * Element types: q, cache rows and B bases share one dtype (lrkv_dtype);
 * p and out are always fp32; seq_lens is int32.  Arithmetic is fp32 with fp32
 * accumulation for both dtypes.
 * `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 * call only enqueues work on that stream and never synchronises; device
 * faults surface at the caller's next synchronisation.
 * Argument checks run on the host before any HIP call; a rejected call
 * enqueues nothing.  Functions return LRKV_OK or an error code; the text of
 * the last error on the calling thread is available from lrkv_last_error().
 * The library has no global mutable state besides that per-thread message,
 * so calls from several threads on different streams are independent.
 */
#ifndef LRKV_H
#define LRKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    LRKV_OK = 0,
    LRKV_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, misaligned pointer, max_len > L_cap, ... */
    LRKV_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement (see lrkv_decode) */
    LRKV_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than lrkv_decode_workspace_bytes */
    LRKV_ERR_HIP = 4          /* a kernel launch failed */
} lrkv_status;

typedef enum {
    LRKV_F32 = 0,  /* IEEE binary32 */
    LRKV_BF16 = 1  /* bfloat16 (upper half of binary32) */
} lrkv_dtype;

/* Problem sizes, in the pages' notation (reading notes sec. 2.1 symbol table). */
typedef struct {
    int32_t batch; /* sequences, >= 1 */
    int32_t H;     /* query heads, >= 1 */
    int32_t d_h;   /* head width, >= 1 */
    int32_t r;     /* residual rank, >= 0; r = 0 is MQA-style sharing of one K/V */
    int32_t L_cap; /* rows allocated per sequence in every cache tensor, >= 1 */
    int32_t dtype; /* lrkv_dtype of q, the cache rows and B^K, B^V */
} lrkv_dims;

/* The factored cache of one layer (review sec. 3, Algorithm 1): device pointers.
 *   k_shared, v_shared  [batch][L_cap][d_h]   rows x W_shared^K, x W_shared^V
 *   z_k, z_v            [batch][L_cap][H][r]  latents x U_h^K, x U_h^V; may be NULL iff r == 0
 *   seq_lens            [batch] int32         live rows per sequence: rows 0 .. seq_lens[b]-1
 * The latents are stored token-major: element z[b][j][h][i] is head h's
 * coordinate i for token j, so one token's H x r latents form one contiguous
 * row (the logical per-head tensor z_h[b][j][i] of the pages, transposed).
 * This replaces the per-head layout [batch][H][L_cap][r] in which the pages'
 * notation (reading notes sec. 2.1) and a per-head cache would hold them:
 * latents in that layout are NOT accepted here -- the library cannot tell the
 * two apart, and per-head latents give wrong results.  Convert them once with
 * lrkv_latents_to_token_major.  The reason for the change: a decode step then
 * streams every cache tensor linearly, and per-head latent regions never sit at
 * a common large stride, whatever L_cap is (split pass 208 against 227 us at
 * the long-context shape with L_cap = 33024).
 * For decode the current query's own token must already be appended, so
 * seq_lens[b] counts it; every live row is visible to the query. */
typedef struct {
    void* k_shared;
    void* v_shared;
    void* z_k;
    void* z_v;
    int32_t* seq_lens;
} lrkv_cache;

/* A paged factored cache (review sec. 4, the paged allocation a serving system
 * uses; sec. 9, append after prefill across page boundaries): the same rows as
 * lrkv_cache, stored in fixed-size pages drawn from one pool per tensor.
 *   k_pages, v_pages    [n_pages][page_rows][d_h]     (dims->dtype)
 *   zk_pages, zv_pages  [n_pages][page_rows][H][r]    token-major as in lrkv_cache; may be NULL iff r == 0
 *   block_table         device [batch][max_pages] int32: logical page m of sequence b (rows
 *                       m*page_rows .. (m+1)*page_rows - 1) is pool page block_table[b][m]
 *   seq_lens            device [batch] int32, as in lrkv_cache
 *   page_rows           rows per page: a power of two, >= 32
 *   max_pages           entries per sequence in block_table; dims->L_cap must equal max_pages * page_rows
 *   n_pages             pages in each pool
 * Every table entry that covers a live row (or the row an append writes) must
 * be a valid page index in [0, n_pages); the library does not check device
 * contents.  Pages may be shared between sequences only if their live rows
 * are identical (e.g. a common prefix) and no append writes into them. */
typedef struct {
    void* k_pages;
    void* v_pages;
    void* zk_pages;
    void* zv_pages;
    int32_t* block_table;
    int32_t* seq_lens;
    int32_t page_rows;
    int32_t max_pages;
    int32_t n_pages;
} lrkv_paged_cache;

/* Latents from the per-head layout to the token-major layout lrkv_cache and
 * lrkv_paged_cache expect (see lrkv_cache):
 *   src  device [batch][H][L_cap][r]   (dims->dtype), per head
 *   dst  device [batch][L_cap][H][r]   (dims->dtype), token-major
 * dst[b][j][h][i] = src[b][h][j][i] for every row j < L_cap, copied bit for
 * bit; src and dst must not overlap.  r == 0: nothing to do (src, dst may be
 * NULL).  Apply it to z_k and z_v separately. */
lrkv_status lrkv_latents_to_token_major(const lrkv_dims* dims, const void* src, void* dst, void* stream);

/* Absorb the key basis into the query: p[b][h][i] = sum_c q[b][h][c] * B_k[h][c][i]
 * (reading notes sec. 2.4 Eq. (6); review sec. 3, Algorithm 2: one small
 * product per head per step).
 *   q    device [batch][H][d_h]  (dims->dtype)
 *   B_k  device [H][d_h][r]      (dims->dtype)
 *   p    device [batch][H][r]    fp32 out
 * r == 0: nothing to do, returns LRKV_OK (q, B_k, p may be NULL). */
lrkv_status lrkv_absorb_query(const lrkv_dims* dims, const void* q, const void* B_k, float* p, void* stream);

/* Append one token's projected rows to every sequence (review sec. 3,
 * Algorithm 1: shared rows once, both private latents per head at the
 * matching token index; reading notes sec. 2.3).
 *   k_new, v_new    device [batch][d_h]      (dims->dtype)
 *   zk_new, zv_new  device [batch][H][r]     (dims->dtype); may be NULL iff r == 0
 * For each b the row is written at index seq_lens[b] (read on the device) and
 * seq_lens[b] is then incremented on the device.  A sequence that is already
 * full (seq_lens[b] >= L_cap) or has a negative length is left unchanged and
 * nothing is written for it. */
lrkv_status lrkv_cache_append(const lrkv_dims* dims, const lrkv_cache* cache, const void* k_new, const void* v_new,
                              const void* zk_new, const void* zv_new, void* stream);

/* The two per-token operations of a decode step in one launch: lrkv_cache_append
 * of (k_new, v_new, zk_new, zv_new) and lrkv_absorb_query of (q, B_k) into p,
 * with the same arguments, layouts and results (bit for bit) as the two calls
 * (review sec. 3, Algorithms 1 and 2; reading notes secs. 2.3-2.4).  They
 * touch disjoint memory, so their workgroups run side by side and the step
 * pays one kernel launch instead of two.  r == 0: the append alone (q, B_k, p
 * may be NULL).  Shapes outside the absorb's vector path (r not a multiple of
 * 8 in bf16 or 4 in fp32, or d_h > 256) run the two kernels one after the
 * other. */
lrkv_status lrkv_append_absorb(const lrkv_dims* dims, const lrkv_cache* cache, const void* k_new, const void* v_new,
                               const void* zk_new, const void* zv_new, const void* q, const void* B_k, float* p,
                               void* stream);

/* Bytes of device workspace lrkv_decode / lrkv_decode_partial need for these
 * dims and this max_len: G x H x align4(d_h + r + 2) floats, G as returned by
 * lrkv_decode_num_splits.  Host arithmetic only.  Returns 0 for invalid dims. */
size_t lrkv_decode_workspace_bytes(const lrkv_dims* dims, int32_t max_len);

/* Split plan of the decode for these dims and max_len: returns G, the number
 * of partial records per head the workspace holds (the split kernel launches
 * G workgroups for the whole batch), and the split granule in rows
 * (*chunk_tokens, may be NULL).  On the device the G workgroups are dealt to
 * the sequences by their live lengths, at least one each.  With n_b the
 * 32-row blocks of sequence b and M the least multiple of granule / 32 for
 * which S_b = max(1, ceil(n_b / M)) add up to at most G: when M is at least
 * 8 * granule / 32, each sequence has one query set and the batch holds at
 * most 64 sequences, sequence b gets those S_b workgroups (workgroups past
 * the sum have no split); otherwise they are dealt in proportion to the n_b.
 * Split s of sequence b takes the granule-row tiles s, s + S_b, s + 2 S_b, ...
 * of the sequence and holds live rows iff s * granule < seq_lens[b].
 * Host arithmetic only.  Returns 0 for invalid dims or max_len == 0. */
int32_t lrkv_decode_num_splits(const lrkv_dims* dims, int32_t max_len, int32_t* chunk_tokens);

/* The plan above, evaluated for given lengths as the decode's kernels evaluate
 * it: first_wg[b] = W_b, the first of sequence b's workgroups (the index of its
 * first partial record), and splits[b] = S_b, for b < dims->batch.  seq_lens
 * (device, [batch]) are the lengths the decode reads; append = 1 gives the plan
 * of lrkv_decode_step, which decodes each length L with 0 <= L < L_cap as
 * L + 1 (append = 0: lrkv_decode).  first_wg and splits are device int32
 * arrays of batch entries, written by a kernel enqueued on `stream` (nothing
 * is written when max_len == 0: the decode launches no split workgroups).
 * For inspecting and testing how a batch is split; the decode needs no call.
 * Errors: invalid dims or max_len, append other than 0 or 1, NULL pointers,
 * shapes with no kernel. */
lrkv_status lrkv_decode_split_plan(const lrkv_dims* dims, int32_t max_len, const int32_t* seq_lens, int32_t append,
                                   int32_t* first_wg, int32_t* splits, void* stream);

/* One decode step against the factored history (review sec. 3, Algorithm 2
 * and its fused online-softmax form; reading notes sec. 2.4 Eqs. (6)-(7)):
 *   s_j = (q_h . k_shared[j] + p_h . z_k[h][j]) / sqrt(d_h),  j < seq_lens[b]
 *   a   = softmax(s)   (one softmax over the summed logits)
 *   out[b][h] = sum_j a_j v_shared[j] + (sum_j a_j z_v[h][j]) (B_v[h])^T
 * Inputs:
 *   cache      the factored cache; seq_lens[b] must lie in [0, max_len]
 *   max_len    host upper bound of seq_lens, 0 <= max_len <= L_cap
 *   q          device [batch][H][d_h] (dims->dtype)
 *   p          device [batch][H][r] fp32, from lrkv_absorb_query for this q and B_k; may be NULL iff r == 0
 *   B_v        device [H][d_h][r] (dims->dtype); may be NULL iff r == 0
 *   out        device [batch][H][d_h] fp32 (written completely; 0 for a sequence with no live rows)
 *   workspace  device, >= lrkv_decode_workspace_bytes(dims, max_len) bytes, 256-byte aligned
 * Lengths outside [0, max_len] are clamped into it on the device (memory safe,
 * result then undefined).  The work of every sequence is split along the
 * sequence (see lrkv_decode_num_splits) and the splits' partial softmax states
 * are merged in a fixed order, so results are bitwise reproducible for fixed
 * dims, max_len and seq_lens contents.
 * Supported: d_h <= 256, r <= 256, H * (d_h + r + 2) * 4 <= 64 KiB.  Matrix-core
 * kernels cover bf16 with d_h in {64, 128}, r in {0, 8, 16, 32, 48, 64} and fp32
 * with r = 0, d_h in {64, 128}, both for H in {8, 16, 32}, and bf16 with d_h = 128
 * at the reading notes' model-table shapes (H, r) = (6, 46), (12, 51), (18, 55),
 * (32, 54) (sec. 2.5, Table 7 ranks), all with L_cap a multiple of 32; other
 * valid shapes use the general kernels. */
lrkv_status lrkv_decode(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* q,
                        const float* p, const void* B_v, float* out, void* workspace, size_t workspace_bytes,
                        void* stream);

/* The two halves of lrkv_decode, for callers that time or distribute them.
 * lrkv_decode_partial writes the per-split softmax states (running max in
 * log2 units, denominator, shared-value sum, private-value sum) to the
 * workspace; lrkv_decode_merge combines them in split order and applies B_v.
 * Both must be given the same dims, cache.seq_lens contents and max_len. */
lrkv_status lrkv_decode_partial(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* q,
                                const float* p, void* workspace, size_t workspace_bytes, void* stream);
lrkv_status lrkv_decode_merge(const lrkv_dims* dims, const int32_t* seq_lens, int32_t max_len, const void* B_v,
                              float* out, const void* workspace, size_t workspace_bytes, void* stream);

/* A whole decode step in the fewest launches: lrkv_append_absorb(dims,
 * cache, k_new, v_new, zk_new, zv_new, q, B_k, p) followed by
 * lrkv_decode(dims, cache, max_len, q, p, B_v, out), with the same
 * arguments, layouts and results, bit
 * for bit (p and out written, the token appended, seq_lens advanced) -- the
 * per-token work of Algorithms 1 and 2 and the fused online-softmax decode of
 * the review's sec. 3 (reading notes secs. 2.3-2.4, Eqs. (6)-(7)).  On the bf16
 * matrix-core shapes the launch holds three kinds of workgroups: absorb
 * workgroups (p = q B^K), the decode's split workgroups (each sequence seen
 * with the appended token; the workgroup that reads the token's rows writes
 * them into the cache first) and merge workgroups, which start as soon as
 * every split of their sequence is done.  They hand work on through counters
 * in the workspace, each waiting only for workgroups placed before it in the
 * launch, so the absorb and the merge run beside the splits instead of in
 * launches of their own.  On the fp32 rank-0 matrix-core shapes (no absorb)
 * the split pass appends the token in the same way and its last workgroup
 * advances the lengths; the merge kernel follows (two launches, not three).
 * Other shapes run the two calls one after the other.
 *   max_len    bound of the lengths after the append (as for lrkv_decode)
 *   workspace  device, >= lrkv_decode_step_workspace_bytes(dims, max_len) bytes,
 *              256-byte aligned; the split records, then the step's counter
 *              words from byte offset lrkv_decode_step_sync_offset(dims,
 *              max_len).  The counter words must be zero before the first
 *              call (zero the whole workspace once after allocating it); every
 *              call leaves them zero, so one workspace serves any number of
 *              calls, including replays of a captured graph.  The word at
 *              sync offset + 4 counts waits that ran out of their bound (never
 *              in correct operation; the results of such a call are not
 *              valid); it is not cleared by the library.
 * Calls that overlap in time on one workspace race. */
size_t lrkv_decode_step_workspace_bytes(const lrkv_dims* dims, int32_t max_len);
size_t lrkv_decode_step_sync_offset(const lrkv_dims* dims, int32_t max_len);
/* 1 if lrkv_decode_step folds the append into the decode's launches (one
 * launch on the bf16 matrix-core shapes, two on the fp32 rank-0 ones), 0 if it
 * runs the two calls (or the arguments are invalid).  Host arithmetic only. */
int32_t lrkv_decode_step_fused(const lrkv_dims* dims, int32_t max_len);
lrkv_status lrkv_decode_step(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* k_new,
                             const void* v_new, const void* zk_new, const void* zv_new, const void* q,
                             const void* B_k, const void* B_v, float* p, float* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* lrkv_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation.  Same
 * arguments, kernels, split plan and results (bit for bit) as lrkv_decode,
 * without the workspace: the split records go to a static device array of
 * lrkv_decode_noalloc_max_bytes() bytes (32 MiB) inside the library.  Each GPU
 * holds its own copy of that array from the first call on it until the process
 * ends; the call itself allocates nothing and calls no allocating routine.
 * The array is looked up once per device (the device of `stream`, or the
 * current device for the NULL stream) and is never read before this call's
 * split pass has written the records it needs, so nothing needs clearing.
 * Calls that overlap in time on one GPU share the array and race: run them on
 * one stream, or order them.  A problem whose split records need more than
 * the array (lrkv_decode_workspace_bytes(dims, max_len) > the maximum) is
 * rejected with LRKV_ERR_WORKSPACE before anything is enqueued. */
size_t lrkv_decode_noalloc_max_bytes(void);
lrkv_status lrkv_decode_noalloc(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* q,
                                const float* p, const void* B_v, float* out, void* stream);

/* Decode Q query tokens per sequence at once (speculative decode, chunked
 * prefill): the last Q tokens of every sequence, already appended, each
 * attend to the rows before and at their own position -- query i sits at
 * position seq_lens[b] - Q + i and sees rows j <= seq_lens[b] - Q + i, the
 * causal mask inside the chunk (reading notes sec. 2.4, Eqs. (6)-(7) under
 * the causal softmax; review sec. 3).  Everything else is lrkv_decode's.
 *   n_queries  Q, 1 <= Q <= 64, batch * Q <= 65535
 *   q          device [batch][Q][H][d_h] (dims->dtype)
 *   p          device [batch][Q][H][r] fp32: lrkv_absorb_query with dims->batch = batch * Q
 *   out        device [batch][Q][H][d_h] fp32 (0 for a query that sees no row)
 *   workspace  >= lrkv_decode_multi_workspace_bytes(dims, Q, max_len) bytes, 256-byte aligned
 * It runs lrkv_decode's split-and-merge scheme on virtual sequences, each a
 * set of qw consecutive query tokens of one sequence with the causal length
 * of its last token.  On the bf16 matrix-core shapes qw = 2 (Q = 2) or 4
 * (Q >= 3; at most 2 for d_h = 128 and r = 64): one workgroup serves all qw
 * tokens from a single read of the rows.  Elsewhere qw = 1, one virtual
 * sequence per token.  The sets of one sequence share its block order, so
 * their workgroups read the same rows at about the same time and the repeats
 * are served by the GPU's caches.  The workspace holds qw records per split
 * workgroup and head, then the virtual lengths.  Q = 1 gives exactly
 * lrkv_decode's kernels and results.  LRKV_MULTI_QW (1, 2 or 4) overrides
 * qw; it is read at every call and must not change between the workspace
 * query and the decode. */
size_t lrkv_decode_multi_workspace_bytes(const lrkv_dims* dims, int32_t n_queries, int32_t max_len);
lrkv_status lrkv_decode_multi(const lrkv_dims* dims, int32_t n_queries, const lrkv_cache* cache, int32_t max_len,
                              const void* q, const float* p, const void* B_v, float* out, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Normalised variant: post-projection RMS normalisation of the keys and
 * queries, evaluated exactly on the factored cache (review sec. 8, the
 * paragraphs on post-projection normalisation and its cache cost; reading
 * notes sec. 2.7, last paragraph).  The key of head h at token j is the summed
 * key k_{h,j} = k_shared[j] + z_k[j][h] (B_k[h])^T; it is normalised as a whole
 * (the shared and private parts together), with a per-head gain g_k[h], and the
 * query with g_q[h]:
 *   rho_{h,j} = 1 / sqrt(|k_{h,j}|^2 / d_h + eps)       one scalar per (token, head), cached
 *   q_eff[b][h] = g_k[h] * g_q[h] * q[b][h] / sqrt(|q[b][h]|^2 / d_h + eps)   (the key gain folded in)
 *   s_j = rho_{h,j} * (q_eff . k_shared[j] + p . z_k[j][h]) / sqrt(d_h),  p = q_eff B_k[h]
 * Values are not normalised.  The scales are kept beside the cache:
 *   rho  device [batch][L_cap][H] (dims->dtype), token-major like the latents:
 *        2 bytes per (token, head) in bf16, 1/(2 d_h) of a per-head K/V payload.
 * A step: lrkv_cache_append (or lrkv_project_append), lrkv_key_scales with
 * n_last = 1, lrkv_norm_query, lrkv_absorb_query on q_eff, lrkv_decode_normed. */

/* Scales of the last n_last live rows of every sequence, rows
 * max(0, L_b - n_last) .. L_b - 1 (n_last = 1 after an append; n_last >= max_len
 * for the whole history, e.g. after a prefill).  Other rows of rho are not
 * written.  The key is rebuilt in fp32 from the stored factors (never stored)
 * and the scale rounded once to dims->dtype (nearest even).
 *   max_len  host bound of seq_lens, 0 <= max_len <= L_cap
 *   n_last   >= 0; B_k device [H][d_h][r] (may be NULL iff r == 0); eps finite, >= 0
 *            (with eps = 0 an all-zero key gets an infinite scale)
 * bf16 with d_h a multiple of 16 and r a multiple of 8 up to 64 runs on the
 * matrix cores; other shapes on a plain kernel. */
lrkv_status lrkv_key_scales(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, int32_t n_last,
                            const void* B_k, float eps, void* rho, void* stream);

/* The normalised query with the key gain folded in, q_eff as above, rounded
 * once to dims->dtype (nearest even):
 *   q, q_eff  device [batch][H][d_h];  g_q, g_k  device [H][d_h]  (all dims->dtype)
 * Arithmetic: fp32, the sum of squares reduced in a fixed order. */
lrkv_status lrkv_norm_query(const lrkv_dims* dims, const void* q, const void* g_q, const void* g_k, float eps,
                            void* q_eff, void* stream);

/* lrkv_decode with every logit multiplied by its cached scale (above).
 * Arguments as lrkv_decode with q = q_eff (and p from lrkv_absorb_query on
 * q_eff), plus rho as written by lrkv_key_scales; the workspace is
 * lrkv_decode_workspace_bytes(dims, max_len).  Rows j < seq_lens[b] need their
 * scale in rho. */
lrkv_status lrkv_decode_normed(const lrkv_dims* dims, const lrkv_cache* cache, const void* rho, int32_t max_len,
                               const void* q_eff, const float* p, const void* B_v, float* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/* lrkv_cache_append on a paged cache: row seq_lens[b] of sequence b goes to
 * pool page block_table[b][seq_lens[b] / page_rows], row seq_lens[b] %
 * page_rows, then seq_lens[b] is incremented; a sequence at L_cap or with a
 * negative length is left unchanged. */
lrkv_status lrkv_paged_append(const lrkv_dims* dims, const lrkv_paged_cache* cache, const void* k_new,
                              const void* v_new, const void* zk_new, const void* zv_new, void* stream);

/* lrkv_decode on a paged cache: the same arithmetic, plan and workspace
 * (lrkv_decode_workspace_bytes(dims, max_len)) as lrkv_decode on the
 * contiguous cache holding the same rows, and for the matrix-core bf16 shapes
 * bitwise the same result.  Each pool must hold fewer than 2^31 bytes. */
lrkv_status lrkv_decode_paged(const lrkv_dims* dims, const lrkv_paged_cache* cache, int32_t max_len, const void* q,
                              const float* p, const void* B_v, float* out, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Rotary variant: rotary position embedding applied exactly on the factored
 * cache (review sec. 8, "Full RoPE needs a stronger identity"; reading notes
 * sec. 2.7).  A rotation cannot be moved into the rank-r latent for a generic
 * B_k, so the cache keeps every factor unrotated and the decode turns each
 * head's whole key at its own position:
 *   ktilde_{h,j} = (k_shared[j] + z_k[j][h] (B_k[h])^T) D_j,   qtilde = q D_{L_b - 1}
 *   s_j = qtilde . ktilde_{h,j} / sqrt(d_h),  a = softmax(s),  values as in lrkv_decode (not rotated)
 * D_t turns coordinate pair k = (2k, 2k+1) by t * theta_k, theta_k = base^(-2k/d_h):
 *   (x_2k, x_2k+1) -> (x_2k cos - x_2k+1 sin, x_2k sin + x_2k+1 cos).
 * Row j of a sequence sits at position j; the query is its last row. */

/* table[t][k] = (cos, sin)(t * theta_k), t < n_pos, k < d_h / 2: device
 * [n_pos][d_h / 2][2] fp32, the angle and both values computed in fp64. */
lrkv_status lrkv_rope_table(int32_t d_h, int32_t n_pos, float base, float* table, void* stream);

/* Bytes of device workspace lrkv_decode_rope needs (its own plan: the
 * matrix-core rotary kernel runs one eight-wave workgroup per CU).  Returns 0 for
 * invalid dims or d_h not a multiple of 4.  Host arithmetic only. */
size_t lrkv_decode_rope_workspace_bytes(const lrkv_dims* dims, int32_t max_len);

/* Decode under the rotary variant.  Arguments as lrkv_decode, except:
 *   q      device [batch][H][d_h], unrotated (the kernel turns it at position seq_lens[b] - 1)
 *   B_k    device [H][d_h][r] (the keys are rebuilt; no absorbed query is used); NULL iff r == 0
 *   table  lrkv_rope_table output with n_pos >= max_len
 * Workspace: lrkv_decode_rope_workspace_bytes(dims, max_len).  d_h must be a
 * multiple of 4.  The key of every (row, head) is rebuilt, turned and dotted
 * in fp32: d_h * r extra multiply-adds per row and head, the cost the review
 * names for the exact contraction. */
lrkv_status lrkv_decode_rope(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* q,
                             const void* B_k, const float* table, const void* B_v, float* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Rebuild every head's keys and values from the factored cache (reading notes
 * sec. 2.1 Eqs. (2)-(5); review sec. 3, the materialised form training and
 * prefill use):
 *   K_out[b][h][j] = k_shared[b][j] + z_k[b][j][h] (B_k[h])^T
 *   V_out[b][h][j] = v_shared[b][j] + z_v[b][j][h] (B_v[h])^T,  j < seq_lens[b]
 *   K_out, V_out  device [batch][H][L_cap][d_h] (dims->dtype); rows j >= seq_lens[b] are not written
 *   max_len       host bound of seq_lens, 0 <= max_len <= L_cap
 * Arithmetic: fp32 sums rounded once to dims->dtype.  bf16 with d_h a multiple
 * of 16 and r a multiple of 8 up to 64 runs on the matrix cores. */
lrkv_status lrkv_materialize(const lrkv_dims* dims, const lrkv_cache* cache, int32_t max_len, const void* B_k,
                             const void* B_v, void* K_out, void* V_out, void* stream);

/* Project the new token of every sequence and append it to the cache, in one
 * stacked product (review sec. 3, Algorithm 1; reading notes sec. 2.1
 * Eqs. (2)-(5) and sec. 2.3):
 *   y = x W_in^T, the rows of W_in ordered
 *       [W_q (H*d_h rows) | W_S^K (d_h) | W_S^V (d_h) | U^K (H*r, head h at rows h*r) | U^V (H*r)]
 *   q_out[b] = y[b][0 .. H*d_h); the shared key/value rows and every head's
 *   latents are written to row seq_lens[b] of the cache, then seq_lens[b] is
 *   incremented (a full sequence, seq_lens[b] >= L_cap, or a negative length
 *   is left unchanged and nothing of its cache is written; its q_out is still
 *   written).
 *   x      device [batch][d_model]                       (dims->dtype)
 *   W_in   device [H*d_h + 2*d_h + 2*H*r][d_model]       (dims->dtype; one output feature per row)
 *   q_out  device [batch][H][d_h]                        (dims->dtype)
 * Arithmetic: fp32 accumulation in a fixed order, results rounded to
 * dims->dtype (nearest even).  bf16 weights with d_model a multiple of 512 run
 * on the matrix cores; other shapes on a plain fp32 kernel.  Enqueues two
 * kernels (the product, then the length update).  Fails with
 * LRKV_ERR_UNSUPPORTED when W_in has 2^31 elements or more. */
lrkv_status lrkv_project_append(const lrkv_dims* dims, int32_t d_model, const lrkv_cache* cache, const void* x,
                                const void* W_in, void* q_out, void* stream);

/* Output projection of the decode result (review sec. 3, the last step of
 * Algorithm 2; reading notes sec. 2.4, after Eq. (7)):
 *   y[b] = concat_h(o[b][h]) W_o^T
 *   o    device [batch][H][d_h] fp32 (the output of lrkv_decode)
 *   W_o  device [d_model][H*d_h] (dims->dtype; one output feature per row)
 *   y    device [batch][d_model] fp32
 * Arithmetic: fp32 accumulation in a fixed order.  With bf16 weights (and
 * H*d_h a multiple of 512) o enters the matrix cores as a bf16 high part plus a
 * bf16 low part, about 16 significant bits; otherwise a plain fp32 kernel. */
lrkv_status lrkv_output_project(const lrkv_dims* dims, int32_t d_model, const float* o, const void* W_o, float* y,
                                void* stream);

/* Measurement helper, not part of the method: read every byte of src once
 * with 16-byte non-temporal loads (the streaming-read bandwidth the decode is
 * compared with) and write one XOR checksum per workgroup to sink.
 *   src   device, 16-byte aligned; bytes a positive multiple of 16
 *   sink  device uint32 [1024] */
lrkv_status lrkv_read_probe(const void* src, size_t bytes, uint32_t* sink, void* stream);

/* Cache payload in bytes, counted as the pages count it (numel x element size
 * of the live rows): 2 * s * sum_b L_b * (d_h + H * r), s = 4 (fp32) or 2 (bf16)
 * (reading notes sec. 2.5 Eqs. (8)-(9); review sec. 4).  host_seq_lens is a
 * host array [batch]; NULL counts L_cap rows for every sequence.  Negative
 * lengths count as 0 and lengths above L_cap as L_cap.  Returns 0 for invalid dims. */
uint64_t lrkv_cache_bytes(const lrkv_dims* dims, const int32_t* host_seq_lens);

/* Static text for a status code. */
const char* lrkv_status_str(lrkv_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* lrkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LRKV_H */
