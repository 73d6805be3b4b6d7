/*
 * btk.h -- block top-k sparse decode attention on AMD MI355X (gfx950).
 *
 * The method: keys of each KV head are grouped into fixed-size blocks (one KV
 * cache page each), every block is summarised by its mean key (its centroid),
 * the query heads that share a KV head (one grouped-query "query group") score
 * every centroid together, keep the top-k blocks, and run exact softmax
 * attention over only those blocks.  Sources: Pith review of "Kinetics:
 * Rethinking Test-Time Scaling Laws" (pith.science), section "What carries the
 * argument"; paging, block = page and top-k counted in pages: Kinetics README
 * (GitLite mirror), section "Benchmark Block TopK Attention throughput".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every buffer argument is a DEVICE pointer owned by the caller, unless it is
 *    marked "host".  The library never allocates, frees or synchronises device
 *    memory; every call is enqueued asynchronously on `stream` (a hipStream_t,
 *    NULL = the default stream) and returns once its kernels are launched.
 *  - Arguments are validated on the host before any HIP call.  A rejected call
 *    returns an error status and touches nothing.  No C++ exception crosses the
 *    ABI.  A launch failure returns BTK_ERR_HIP (see btk_last_hip_error()).
 *  - Device-resident contents (page ids, lengths, indices) are not inspected on
 *    the host.  Kernels never read outside the caller's buffers for any input:
 *    an out-of-range page id, length or index is skipped, and, where the call
 *    has a workspace, sets a sticky bit in workspace word 0 (bit 0: a length
 *    outside [1, max_blocks_per_seq * page_size]; bit 1: a page id outside
 *    [0, num_pages); bit 2: a block index outside [0, n_b); bit 3: a bounded wait
 *    for data published inside a launch gave up, a safeguard that no call is
 *    expected to reach (every such wait ends once the work it waits for, which is
 *    never held by a workgroup that has not started, is done); bit 4: a declared
 *    shared prefix differs between group members).
 *    Results for such inputs are unspecified.
 *
 * Notation: B = batch, Hq / Hkv = query / KV heads, r = Hq / Hkv (the query
 * group size; query head h uses KV head h / r), D = head_dim, P = page_size,
 * L_b = seq_lens[b] (counts the newest token), n_b = ceil(L_b / P) blocks,
 * block j of sequence b holds logical tokens [j*P, min(L_b, j*P+P)).
 *
 * Layouts (row-major):
 *   q, out       [B][Hq][D]                dtype
 *   k_cache      [num_pages][Hkv][P][D]    dtype   token-major pages
 *   v_cache      [num_pages][Hkv][D][P]    dtype   dim-major pages
 *   block_table  [B][max_blocks_per_seq]   int32   logical block -> page id
 *   seq_lens     [B]                       int32
 *   centroids    [num_pages][Hkv][D]       float32
 *   indices      [B][Hkv][top_k]           int32
 *   scores       [B][Hkv][max_blocks_per_seq] float32
 *   lse          [B][Hq]                   float32 (natural log)
 */
#ifndef BTK_H
#define BTK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BTK_ABI_VERSION 1

typedef enum {
    BTK_OK = 0,
    BTK_ERR_NULL = 1,        /* a required pointer is NULL */
    BTK_ERR_SHAPE = 2,       /* a size is out of range or inconsistent */
    BTK_ERR_UNSUPPORTED = 3, /* valid, but not built: dtype, head_dim, page_size, limits */
    BTK_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than btk_workspace_bytes() */
    BTK_ERR_HIP = 5          /* the HIP runtime reported an error at launch */
} btk_status_t;

typedef enum { BTK_BF16 = 0, BTK_F32 = 1 } btk_dtype_t;

/* Problem description (host struct, read during the call only).
 * Supported: dtype BTK_BF16 or BTK_F32; head_dim 64 or 128; page_size 16;
 * 1 <= r <= 16; max_blocks_per_seq <= 8192 (contexts up to 131072 tokens).
 * sm_scale <= 0 selects 1/sqrt(head_dim); it scales both the block scores and
 * the attention logits. */
typedef struct {
    int32_t batch;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t page_size;
    int32_t num_pages;
    int32_t max_blocks_per_seq;
    int32_t dtype; /* btk_dtype_t */
    float sm_scale;
} btk_problem_t;

/* Version of this ABI (BTK_ABI_VERSION of the built library). */
int btk_abi_version(void);

/* Human-readable name of a status code (static storage). */
const char *btk_status_string(btk_status_t status);

/* hipError_t code of the last BTK_ERR_HIP returned on this host thread. */
int btk_last_hip_error(void);

/* Bytes of device workspace that btk_select, btk_sparse_attend,
 * btk_dense_attend, btk_local_attend (top_k = the window) and btk_decode_step
 * need for this problem and top_k (host; no HIP call).
 * Returns 0 if the problem is invalid.  The caller allocates it, ZERO-FILLS it
 * once before its first use, and may then reuse it for any number of calls of
 * the same or a smaller problem (batch * num_kv_heads and every size at most
 * those of the problem it was sized for): each completed call leaves its
 * internal counters at zero again.  Calls that may overlap in time (different
 * streams) need separate workspaces. */
size_t btk_workspace_bytes(const btk_problem_t *problem, int32_t top_k);

/* S1 -- centroid update.  (Pith review, "What carries the argument": blocks are
 * summarised by their averaged key vector.)
 * For every block j of sequence b with j >= first_pos[b] / P (every block of
 * every sequence when first_pos is NULL) and every KV head g:
 *     centroids[page][g][:] = (sum of the block's valid keys, in fp32) / v_j,
 * page = block_table[b][j], v_j = min(P, L_b - j*P).  Other pages are left
 * untouched.  In decode, pass first_pos[b] = position of the token just
 * appended (L_b - 1), so only the page holding it is recomputed.  A page shared
 * by several sequences must hold the same number of valid tokens in each;
 * rebuilding it from several sequences writes identical values.
 *   k_cache    in   [num_pages][Hkv][P][D] dtype
 *   first_pos  in   [B] int32 device pointer, or NULL
 *   centroids  in/out [num_pages][Hkv][D] float32 */
btk_status_t btk_centroid_update(const btk_problem_t *problem, const void *k_cache,
                                 const int32_t *block_table, const int32_t *seq_lens,
                                 const int32_t *first_pos, float *centroids, void *stream);

/* S2 + S3 -- block scoring and top-k selection.  (Pith review, "What carries
 * the argument": blocks are scored by their averaged keys per query group and
 * the top k blocks are kept; top-k counted in pages: Kinetics README, "Benchmark
 * Block TopK Attention throughput".)
 * For unit (b, g) and block j < n_b, the group score is
 *     s_j = sm_scale * qbar . centroids[block_table[b][j]][g],
 *     qbar = mean of q[b][h] over the r query heads h of group g,
 * computed in fp32 (equal to the mean of the heads' scaled logits up to
 * rounding).  The k_b = min(top_k, n_b) blocks with the largest s_j are kept;
 * equal scores go to the lower j (-0.0 equals +0.0).  indices[b][g][0..k_b) holds
 * them in ascending j, and indices[b][g][k_b..top_k) = -1.  NaN scores give
 * unspecified selections.
 *   q        in   [B][Hq][D] dtype
 *   top_k    1 .. 8192
 *   indices  out  [B][Hkv][top_k] int32
 *   scores   out  [B][Hkv][max_blocks_per_seq] float32, or NULL; entries
 *                 j >= n_b are not written
 *   workspace     btk_workspace_bytes(problem, top_k) bytes (see above) */
btk_status_t btk_select(const btk_problem_t *problem, const void *q, const float *centroids,
                        const int32_t *block_table, const int32_t *seq_lens, int32_t top_k,
                        int32_t *indices, float *scores, void *workspace,
                        size_t workspace_bytes, void *stream);

/* Block sketches: an 8-bit copy of every block's fp32 centroid, kept per
 * sequence in block-table order, from which btk_select_sketch rules blocks out
 * of the top-k before reading their fp32 centroid rows.  Its selections are
 * those of btk_select (the rule-out is provably safe, see btk_select_sketch).
 * (Pith review, "What carries the argument": the method's block scores and
 * top-k; the sketch is this library's way of reading fewer bytes for them.)
 * Layout (btk_sketch_bytes bytes, owned by the caller): for row
 * i = (b * num_kv_heads + g) * max_blocks_per_seq + j, an 8-byte header
 * {int32 page + 1 (0: none), float32 scale} at offset 8 i, and head_dim code
 * bytes at offset R + head_dim * i, R = 8 * rows rounded up to 256; code_d =
 * rint(c_d / scale) + 128 with scale = max_d |c_d| / 127.  A sketch belongs to
 * one (batch, num_kv_heads, max_blocks_per_seq, head_dim).  Any contents are
 * safe: a row whose header does not name block j's current page is simply not
 * used to rule it out; a row that names it must have been built from that
 * page's current centroid (call btk_sketch_update after every
 * btk_centroid_update, with the same first_pos).  Returns 0 for an invalid
 * problem. */
size_t btk_sketch_bytes(const btk_problem_t *problem);

/* Writes the sketch rows of every block j >= first_pos[b] / 16 (every block when
 * first_pos is NULL; negative positions count as 0) of every sequence and KV
 * head from centroids[block_table[b][j]][g] (fp32, as btk_centroid_update left
 * them).  A block whose page id is out of range gets an empty header and sets
 * workspace bit 2; an invalid length sets bit 1.
 *   sketch     in/out, sketch_bytes >= btk_sketch_bytes(problem)
 *   workspace  any workspace of this problem (its error word is used) */
btk_status_t btk_sketch_update(const btk_problem_t *problem, const float *centroids,
                               const int32_t *block_table, const int32_t *seq_lens,
                               const int32_t *first_pos, void *sketch, size_t sketch_bytes,
                               void *workspace, size_t workspace_bytes, void *stream);

/* S2 + S3 with the same indices as btk_select, reading each unit's sketch rows
 * and only the fp32 centroid rows of the blocks the sketch cannot rule out.
 * For unit (b, g) every block gets an interval [sa - e, sa + e] from its
 * sketch row (sa: the sketch's score; e = 0.51 * scale * sum_d |qs_d|, qs the
 * scaled mean query), which holds the block's fp32 score as btk_select computes
 * it, rounding included.  With tau the k_b-th largest lower end, blocks whose
 * upper end is below tau score below k_b others and are dropped; the others are
 * scored from their fp32 centroid rows exactly as btk_select scores them and the
 * k_b best are kept with btk_select's tie rule.  Rows that do not name the
 * block's current page are never dropped.
 *   sketch     as built by btk_sketch_update, sketch_bytes >= btk_sketch_bytes()
 *   indices    out [B][Hkv][top_k] int32, equal to btk_select's
 *   workspace  btk_workspace_bytes(problem, top_k) bytes, as btk_select */
btk_status_t btk_select_sketch(const btk_problem_t *problem, const void *q,
                               const float *centroids, const void *sketch, size_t sketch_bytes,
                               const int32_t *block_table, const int32_t *seq_lens,
                               int32_t top_k, int32_t *indices, void *workspace,
                               size_t workspace_bytes, void *stream);

/* S2 + S3 for Best-of-N batches, reading each shared prompt page once.  The
 * pages' cost model counts a prompt's KV as read once for all N samples (Pith
 * review, "What carries the argument", and its referee report on the
 * Best-of-N memory term); here the centroid rows of a group's shared prefix are
 * read once per KV head and scored against every member's mean query.  Results
 * (indices, scores) are bit-identical to btk_select's.
 *   num_groups     1 .. 64
 *   group_start    host [num_groups + 1]: group g is the sequences
 *                  group_start[g] .. group_start[g+1]-1 (1 .. 32 of them,
 *                  increasing, within [0, batch)); sequences outside every group
 *                  are scored alone
 *   prefix_blocks  host [num_groups]: the members of group g share their first
 *                  prefix_blocks[g] block-table entries (0 .. max_blocks_per_seq);
 *                  a member whose entries differ sets workspace bit 4 (results
 *                  are then unspecified)
 *   the rest as btk_select (same workspace size). */
btk_status_t btk_select_shared(const btk_problem_t *problem, const void *q,
                               const float *centroids, const int32_t *block_table,
                               const int32_t *seq_lens, int32_t num_groups,
                               const int32_t *group_start, const int32_t *prefix_blocks,
                               int32_t top_k, int32_t *indices, float *scores, void *workspace,
                               size_t workspace_bytes, void *stream);

/* S4 -- exact softmax attention over the selected blocks.  (Pith review, "What
 * carries the argument": attention runs over only the retrieved blocks.)
 * For query head h of sequence b, g = h / r, the token set is every valid token
 * of the blocks listed in indices[b][g][0..top_k) (entries < 0 are skipped; the
 * list must name at least one block and no block twice).  With
 * l_t = sm_scale * q[b][h] . K_t:
 *     out[b][h] = sum_t softmax(l)_t V_t,   lse[b][h] = ln sum_t exp(l_t).
 * Accumulation is fp32; out is rounded to dtype (bf16: nearest-even).
 *   out  out [B][Hq][D] dtype;  lse out [B][Hq] float32, or NULL */
btk_status_t btk_sparse_attend(const btk_problem_t *problem, const void *q, const void *k_cache,
                               const void *v_cache, const int32_t *block_table,
                               const int32_t *seq_lens, const int32_t *indices, int32_t top_k,
                               void *out, float *lse, void *workspace, size_t workspace_bytes,
                               void *stream);

/* S5 -- dense paged decode attention: the same computation as btk_sparse_attend
 * over all n_b blocks of every sequence (the comparison path; Kinetics README,
 * "Benchmark Block TopK Attention throughput", dense paged attention of one
 * decoder layer). */
btk_status_t btk_dense_attend(const btk_problem_t *problem, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *block_table,
                              const int32_t *seq_lens, void *out, float *lse, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Local (sliding-window) attention baseline: the same computation as
 * btk_sparse_attend over the most recent min(window_blocks, n_b) blocks of each
 * sequence, i.e. the newest KV instead of the selected blocks, at the same
 * per-unit block budget.  (scime summary of "Kinetics: Rethinking Test-Time
 * Scaling Law", table "Measured effects reported in the paper": the ablation
 * that replaces top-k KV selection by local attention, and "Experimental setup",
 * which lists local attention among the baselines; the block granularity and
 * the budget in pages follow the Kinetics README, "Benchmark Block TopK
 * Attention throughput".)
 *   window_blocks  1 .. 8192
 *   workspace      btk_workspace_bytes(problem, window_blocks) bytes, as above
 *   out out [B][Hq][D] dtype;  lse out [B][Hq] float32, or NULL */
btk_status_t btk_local_attend(const btk_problem_t *problem, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *block_table,
                              const int32_t *seq_lens, int32_t window_blocks, void *out,
                              float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* Token-level top-k attention baseline ("oracle top-k"): for unit (b, g) every
 * valid token t < L_b is scored like a one-token block,
 *     s_t = sm_scale * qbar . K_t,   qbar = mean of q[b][h] over the group,
 * the K_b = min(top_tokens, L_b) highest-scoring tokens are kept (equal scores
 * go to the lower position), and every query head of the group attends over
 * exactly those tokens as in btk_sparse_attend.  It reads every key (the
 * retrieval cost the block method avoids) and is the upper bound the block
 * method is compared with.  (scime summary of "Kinetics: Rethinking Test-Time
 * Scaling Law", "Experimental setup": oracle top-k attention among the
 * baselines; "Limitations": the sparse results use it as their upper bound.)
 *   top_tokens     1 .. 131072 (a budget of k blocks is top_tokens = 16 k)
 *   token_indices  out [B][Hkv][top_tokens] int32 logical positions of the kept
 *                  tokens, ascending, -1 padded; or NULL
 *   out out [B][Hq][D] dtype;  lse out [B][Hq] float32, or NULL
 *   workspace      btk_token_workspace_bytes(problem, top_tokens) bytes, zero-filled
 *                  once before the first use and reusable as for the other calls */
size_t btk_token_workspace_bytes(const btk_problem_t *problem, int32_t top_tokens);
btk_status_t btk_token_topk_attend(const btk_problem_t *problem, const void *q,
                                   const void *k_cache, const void *v_cache,
                                   const int32_t *block_table, const int32_t *seq_lens,
                                   int32_t top_tokens, int32_t *token_indices, void *out,
                                   float *lse, void *workspace, size_t workspace_bytes,
                                   void *stream);

/* One whole decode step in a single launch: S1 for the touched pages (as
 * btk_centroid_update with first_pos; none when first_pos is NULL), then S2+S3
 * (as btk_select) and S4 (as btk_sparse_attend), with results identical to
 * those three calls.  A persistent kernel first scores every centroid row (each
 * workgroup a share of the rows, the last rows handed out in chunks to the
 * workgroups that finish first), then each (sequence, KV head) selects and
 * attends once its scores are complete.  Every share is claimed before it is
 * scored, by its own workgroup or, if that one has not started, by one that has
 * finished its own scoring, so the call does not need its whole grid to be
 * resident: beside other kernels (other streams or processes) it is slower, not
 * wrong.  (Test hook: with the environment variable BTK_STEP_TEST_FLAGS=1 at the
 * call, every workgroup leaves its own share to be taken over; results are the
 * same.)
 * (Pith review, "What carries the argument"; the single-launch form is this
 * library's own design.)
 *   centroids  in/out   indices out [B][Hkv][top_k]   out/lse out as btk_sparse_attend
 *   batch      <= 65536, and batch * num_kv_heads * (max_blocks_per_seq + 520) < 2^32
 *              (BTK_ERR_UNSUPPORTED beyond; the separate calls have no such limits)
 *   workspace  btk_workspace_bytes(problem, top_k), zero-filled once, as above. */
btk_status_t btk_decode_step(const btk_problem_t *problem, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_table,
                             const int32_t *seq_lens, const int32_t *first_pos, float *centroids,
                             int32_t top_k, int32_t *indices, void *out, float *lse,
                             void *workspace, size_t workspace_bytes, void *stream);

/* btk_decode_step reading each unit's sketch rows (see btk_sketch_bytes) in
 * place of its fp32 centroid rows, with results identical to btk_decode_step
 * (indices, out, lse and centroids bit for bit).  When there are at least as
 * many (sequence, KV head) units as compute units and the problem fits one
 * workgroup per unit (max_blocks_per_seq <= 3072, top_k <= 256, at most 8 query
 * heads per KV head, one attention split), each unit is done whole by one
 * workgroup, and no workgroup waits for another: it computes every block's
 * sketch interval (as btk_select_sketch); recomputes the touched blocks' (j >=
 * first_pos[b] / 16) centroids from the keys and rebuilds their sketch rows
 * from them, as btk_centroid_update and btk_sketch_update with the same
 * first_pos would, keeping them as candidates; takes the k_b-th largest lower
 * end as threshold, scores the blocks whose upper end reaches it from their
 * fp32 centroid rows exactly as btk_select scores them (every block when more
 * than 1024 do), keeps the k_b best with btk_select's tie rule and attends.
 * With fewer units the step is btk_decode_step's persistent fp32 scan (faster
 * there), which also rebuilds the touched blocks' sketch rows.  The results do
 * not depend on which.
 * The sketch must hold rows for the blocks before first_pos built from their
 * current centroids (btk_sketch_update after prefill; every call keeps the
 * rows of the blocks it touches current); a row that does not name its block's
 * page is never used to drop it, so any contents give the same results, only
 * more slowly.  (Pith review, "What carries the argument": the method's block
 * scores and top-k; the sketch is this library's way of reading fewer bytes
 * for them.)
 *   sketch       in/out, sketch_bytes >= btk_sketch_bytes(problem)
 *   cand_counts  out [B][Hkv] int32, or NULL: per unit the number of blocks
 *                whose fp32 centroid row the selection read (0 when every
 *                block is kept; n_b in the fp32 scan)
 *   other arguments, limits and errors as btk_decode_step. */
btk_status_t btk_decode_step_sketch(const btk_problem_t *problem, const void *q,
                                    const void *k_cache, const void *v_cache,
                                    const int32_t *block_table, const int32_t *seq_lens,
                                    const int32_t *first_pos, float *centroids, void *sketch,
                                    size_t sketch_bytes, int32_t top_k, int32_t *indices,
                                    void *out, float *lse, int32_t *cand_counts, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* btk_decode_step with the KV append of the step fused in: the newest token of
 * each sequence, at position seq_lens[b] - 1 (seq_lens count it), is written
 * into its cache slot from k_new / v_new before it is averaged into its
 * block's centroid and attended, so no separate append precedes the call.  The
 * results, centroids and caches are identical to writing k_new / v_new into the
 * caches and then calling btk_decode_step with first_pos = seq_lens - 1.
 * (Pith review, "What carries the argument": each decode step adds one key and
 * value per sequence to the blocks that are summarised and selected.)
 *   k_new, v_new  [B][Hkv][D], same dtype as q, device, read only
 *   k_cache, v_cache  in/out: slot (seq_lens[b] - 1) % 16 of page
 *                 block_table[b][(seq_lens[b] - 1) / 16] is written for every KV
 *                 head; that page must belong to sequence b alone (a shared
 *                 prompt page is never the newest); a sequence whose page id
 *                 there is out of range is skipped and flagged like any invalid
 *                 page
 *   other arguments, limits and errors as btk_decode_step (first_pos is implied);
 *   BTK_ERR_NULL if k_new or v_new is NULL. */
btk_status_t btk_decode_step_append(const btk_problem_t *problem, const void *q,
                                    const void *k_new, const void *v_new, void *k_cache,
                                    void *v_cache, const int32_t *block_table,
                                    const int32_t *seq_lens, float *centroids, int32_t top_k,
                                    int32_t *indices, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream);

/* btk_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument; the step's scratch (arrival counters, ready words, claim
 * words, scores, split partials) lives in a device array of
 * BTK_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on, from its first call there until the process ends.  The call allocates
 * nothing; its first call on a GPU clears the array's state words with a small
 * fill kernel on `stream` (no memset).  Every call on one GPU shares that GPU's
 * array, which keeps the last call's contents: calls that may overlap in time on
 * one GPU (different streams) race and give unspecified results.  Results are
 * those of btk_decode_step.  Error bits of invalid device inputs are not
 * reported (there is no workspace to read them from).
 *   arguments, limits and errors as btk_decode_step, and
 *   BTK_ERR_WORKSPACE if batch * num_kv_heads > 16384 or the problem's scratch
 *                  (about 4 * batch * num_kv_heads * max_blocks_per_seq bytes of
 *                  scores plus the split partials) does not fit the array beside
 *                  its state words */
#define BTK_NOALLOC_SCRATCH_BYTES (64u << 20)
btk_status_t btk_decode_step_noalloc(const btk_problem_t *problem, const void *q,
                                     const void *k_cache, const void *v_cache,
                                     const int32_t *block_table, const int32_t *seq_lens,
                                     const int32_t *first_pos, float *centroids, int32_t top_k,
                                     int32_t *indices, void *out, float *lse, void *stream);

/* Measurement aid, not part of the method: reads `rows` rows of 512 bytes of
 * src with the request shape of the decode step's centroid scan (16 bytes per
 * lane, half a wavefront per row) and computes nothing, so that hardware byte
 * counters (FETCH_SIZE) can be scaled by a kernel of known traffic,
 * 512 * rows bytes (+ 4 * rows of row ids).
 *   src      device, src_bytes bytes; row i is bytes [512 i, 512 i + 512)
 *   row_ids  device [rows] int32 row numbers (ids outside [0, src_bytes / 512)
 *            are skipped), or NULL for rows 0 .. rows-1 in order
 *   sink     device, one uint32 that is written only by chance (keeps the loads)
 * BTK_ERR_SHAPE if rows < 0, or row_ids is NULL and rows > src_bytes / 512. */
btk_status_t btk_probe_row_read(const void *src, size_t src_bytes, const int32_t *row_ids,
                                int64_t rows, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BTK_H */
