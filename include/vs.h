/*
 * vs.h -- C ABI of the vertical-slash sparse prefill library (libvs.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (VSPrefill; gist.science summaries of arXiv 2603.04460, English
 * page, Technical Summary section 2 "Methodology") prefills causal attention
 * over a per-head index set made of "vertical" key columns and "slash"
 * diagonals (keys at a fixed relative offset i - j from the query, German
 * page section 2.A).  The index sets come from a small indexer over
 * concat(K with RoPE, V) (section 2, "Key Components 1. VSIndexer") followed
 * by cumulative-threshold budgeting (section 2, "3. Adaptive Inference
 * Pipeline, Dynamic Budgeting"), and attention runs over the merged index
 * lists (same section, "Fused Kernel Execution").  The three calls below are
 * those three steps.
 *
 * Conventions shared by every call
 *  - All pointers except `ws_bytes`-style sizes are DEVICE pointers into
 *    memory the caller allocated on the current HIP device.  The library
 *    never allocates, frees or synchronises; every call only enqueues work
 *    on `stream` (NULL = the default stream) and returns.
 *  - Tensors are dense row-major with batch 1: Q [h_q][n][d], K and V
 *    [h_kv][n][d]; nothing is strided.
 *  - Inputs are never written.  Outputs are fully overwritten.
 *  - Host-checkable problems (null pointers, bad sizes, unsupported shapes,
 *    too-small workspace) return a status before anything is launched.  A
 *    launch failure returns VS_ERR_HIP.  No C++ exception crosses the ABI.
 *  - Calls are stateless and reentrant; two calls may run concurrently on
 *    different streams if their outputs and workspaces do not overlap.
 */
#ifndef VS_H_
#define VS_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
/* In C++ the enums below get a fixed underlying type, so that any int a C
 * caller passes (also one that names no enumerator) is a valid value and the
 * library's range checks are well defined; in C they are plain int-sized
 * enums, the same ABI. */
#define VS_ENUM_BASE : int
#else
#define VS_ENUM_BASE
#endif

typedef enum VS_ENUM_BASE {
  VS_OK = 0,
  VS_ERR_INVALID = 1,     /* null pointer, size out of range, bad enum     */
  VS_ERR_UNSUPPORTED = 2, /* valid but not built: head dim, group size     */
  VS_ERR_WORKSPACE = 3,   /* workspace smaller than *_workspace_bytes()    */
  VS_ERR_HIP = 4          /* a HIP launch or runtime call failed           */
} vs_status;

typedef enum VS_ENUM_BASE { VS_BF16 = 0, VS_F32 = 1 } vs_dtype;

typedef enum VS_ENUM_BASE { VS_VERTICAL = 0, VS_SLASH = 1 } vs_kind;

/* ------------------------------------------------------------------ indexer
 * VSIndexer (English page, section 2, "Key Components 1. VSIndexer"): a
 * shared-weight two-layer linear network over x_j = [K_rope[g][j][:] | V[g][j][:]]
 * (2d values) with separate vertical and slash output heads:
 *     h_j = max(0, W1 x_j)            (hidden values, no bias)
 *     vlog[g][j] = W2[0] . h_j,  slog[g][j] = W2[1] . h_j
 * One weight set serves every KV head.
 *   k_rope, v : bf16 [h_kv][n][d]     (K after rotary embedding, and V)
 *   w1        : bf16 [hidden][2d]     (columns 0..d-1 act on K, d..2d-1 on V)
 *   w2        : bf16 [2][hidden]      (row 0 vertical head, row 1 slash head)
 *   vlog,slog : fp32 [h_kv][n]        (outputs, indexed by position j)
 * First layer: bf16 MFMA with fp32 accumulation.  Second layer: fp32.
 * Supported: d in {64, 128}; hidden a multiple of 32 from 32 to 256 (the
 * first-layer weights stay in registers); n >= 1, h_kv >= 1, and each of
 * k_rope and v below 4 GiB (h_kv * n * d * 2 < 2^32 bytes).  Other shapes
 * return VS_ERR_UNSUPPORTED -- for larger inputs call per group of KV heads. */
vs_status vs_index(const void* k_rope, const void* v, int h_kv, int n, int d, int hidden,
                   const void* w1, const void* w2, float* vlog, float* slog,
                   hipStream_t stream);

/* ---------------------------------------------------------------- selection
 * Cumulative-threshold budgeting (English page, section 2, "3. Adaptive
 * Inference Pipeline, Dynamic Budgeting"): per head, the fewest top-scored
 * candidates whose softmax mass reaches `mass` of the total, capped at `cap`,
 * found without a full sort.
 *   VERTICAL: candidate c is key column c, its score is logit[h][c].
 *   SLASH:    candidate c is the offset o = c, scored where its diagonal meets
 *             the last query row: logit[h][n-1-o].  idx then holds offsets.
 * The mass arithmetic is fixed exactly so that the budget is an exact
 * integer decision: m = max score (fp32, -0 == +0); x = score - m (fp32);
 * u = 0 if x < -32, else rint(e(x) * 2^32) as an unsigned 64-bit integer,
 * where e(x) is Cody-Waite range reduction with a two-piece ln 2 followed by
 * the degree-7 Taylor polynomial by fused multiply-adds in fp32; U = sum u;
 * T = ceil(mass * U) in double.  Candidates are ordered by (score
 * descending, candidate ascending); K is the length of the shortest prefix
 * whose u sum reaches T, then min(K, cap).
 *   logit : fp32 [heads][n] (finite values)
 *   idx   : int32 [heads][cap] -- the K chosen candidates ascending, then -1
 *   count : int32 [heads]       -- K
 *   ws    : device workspace of at least vs_select_workspace_bytes(heads, n)
 * Requires 0 < mass <= 1 and 1 <= cap <= n.  Bit-deterministic. */
size_t vs_select_workspace_bytes(int heads, int n);
vs_status vs_select(const float* logit, int heads, int n, vs_kind kind, double mass, int cap,
                    int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/* Max-based dynamic threshold (FlashPrefill summary, arXiv 2603.06199, Spanish
 * page, section 2.B "Umbralizacion Dinamica Basada en Maximos"): per head,
 * keep every candidate whose softmax score is at least `alpha` times the
 * largest one, with no sort and no cumulative sum -- at most `cap` of them,
 * the best first in (score descending, candidate ascending) order.  The test
 * exp(score - max) >= alpha is decided on the quantised masses defined for
 * vs_select: keep when u >= ceil(alpha * 2^32) (the maximum has u = 2^32).
 * Candidates, scores, outputs, workspace and errors as for vs_select;
 * 0 < alpha <= 1. */
vs_status vs_select_threshold(const float* logit, int heads, int n, vs_kind kind, double alpha,
                              int cap, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/* Both selections of a layer in one launch chain: vs_select of vlog as
 * VERTICAL (cap_v) and of slog as SLASH (cap_s), with the same mass.  The
 * two kinds run side by side as 2 * heads rows of one chain, so the call
 * costs about what one vs_select of `heads` heads costs (the chain is bound
 * by the latency of its passes, not by the candidates).  Outputs are
 * bit-identical to the two separate calls.
 *   vlog, slog      : fp32 [heads][n] (finite values)
 *   v_idx, v_cnt    : int32 [heads][cap_v], [heads] -- columns, as vs_select
 *   s_off, s_cnt    : int32 [heads][cap_s], [heads] -- offsets, as vs_select
 *   ws              : device workspace of at least
 *                     vs_select_both_workspace_bytes(heads, n)
 * Requires 0 < mass <= 1, 1 <= cap_v, cap_s <= n, heads <= 32767. */
size_t vs_select_both_workspace_bytes(int heads, int n);
vs_status vs_select_both(const float* vlog, const float* slog, int heads, int n, double mass,
                         int cap_v, int cap_s, int32_t* v_idx, int32_t* v_cnt, int32_t* s_off,
                         int32_t* s_cnt, void* ws, size_t ws_bytes, hipStream_t stream);

/* -------------------------------------------------------- sparse attention
 * Causal prefill attention restricted to the vertical-slash index set
 * (English page, section 2, "Core Concept: Vertical-Slash Pattern" and
 * "3. Adaptive Inference Pipeline, Fused Kernel Execution").  For query head
 * h, KV head g = h / (h_q / h_kv), row i:
 *     S_i = { j : 0 <= j <= i, j in V_g  or  (i - j) in O_g }
 *     out[h][i] = sum_{j in S_i} softmax_j(scale * q_i . k_j) v_j
 *     lse[h][i] = log sum_{j in S_i} exp(scale * q_i . k_j)
 * A key in both sets counts once.  A row with S_i empty gets out = 0 and
 * lse = -inf.  The index lists are merged on the fly per query block into
 * contiguous key tiles (slash ranges, with a per-element diagonal mask) and
 * gathered tiles (verticals no slash range covers); no n x n mask is built.
 *   q          : [h_q][n][d], k, v : [h_kv][n][d], all of dtype `dt`
 *   v_idx      : int32 [h_kv][cap_v] vertical columns, in any order (vs_select
 *                writes them ascending)
 *   v_cnt      : int32 [h_kv] number of valid entries (clamped to [0, cap_v])
 *   s_off      : int32 [h_kv][cap_s] slash offsets, in any order
 *   s_cnt      : int32 [h_kv]
 *   out        : [h_q][n][d] of dtype `dt`;  lse : fp32 [h_q][n] or NULL
 *   ws         : device workspace of at least
 *                vs_attn_workspace_bytes(h_kv, n, cap_v, cap_s)
 * The lists are read into bitmaps, so entries outside [0, n) are ignored and
 * duplicates count once.  bf16 (or fp32
 * rounded to bf16) MFMA products with fp32 softmax and accumulation.
 * `scale` may be any finite value (negative flips every score, zero makes
 * each row the plain mean of V over S_i); NaN or infinity is VS_ERR_INVALID.
 * Supported: d in {64, 128}; h_q / h_kv in {1, 2, 4, 8, 16}; each launch's
 * grid must fit 2^32 work-items per dimension (fewer than 2^22 index-set
 * rows, and fewer than 2^23 attention workgroups of 64 (G = 4) to 256
 * (G = 1) query positions per set), else VS_ERR_UNSUPPORTED. */
size_t vs_attn_workspace_bytes(int h_kv, int n, int cap_v, int cap_s);
vs_status vs_sparse_attn_prefill(const void* q, const void* k, const void* v, vs_dtype dt,
                                 int h_q, int h_kv, int n, int d, float scale,
                                 const int32_t* v_idx, const int32_t* v_cnt, int cap_v,
                                 const int32_t* s_off, const int32_t* s_cnt, int cap_s,
                                 void* out, float* lse, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* The same call for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * no `ws` argument -- the workspace is a static device array of the library,
 * VS_NOALLOC_SCRATCH_BYTES (64 MiB) per GPU, held by every GPU the library
 * runs on until the process ends.  The call allocates and frees nothing.
 * Shapes whose vs_attn_workspace_bytes() exceeds that return
 * VS_ERR_WORKSPACE before anything is launched (8 KV heads at n = 262144
 * with uncapped lists need about 34 MiB).  Every call on a GPU shares that
 * GPU's one array: calls that overlap on one GPU (other streams, other host
 * threads) race and give wrong results; calls on one stream are ordered.
 * The array keeps the last call's contents; the call clears what it needs
 * with its own kernels.  Outputs and other arguments as for
 * vs_sparse_attn_prefill; VS_ERR_HIP if the array's address cannot be had
 * on the current device. */
#define VS_NOALLOC_SCRATCH_BYTES (64u << 20)
vs_status vs_sparse_attn_prefill_noalloc(const void* q, const void* k, const void* v, vs_dtype dt,
                                         int h_q, int h_kv, int n, int d, float scale,
                                         const int32_t* v_idx, const int32_t* v_cnt, int cap_v,
                                         const int32_t* s_off, const int32_t* s_cnt, int cap_s,
                                         void* out, float* lse, hipStream_t stream);

/* Per-query-head index sets (the other reading of "per head": every query
 * head h has its own columns and offsets, S_i^h = { j <= i : j in V_h or
 * i - j in O_h }).  Arguments as vs_sparse_attn_prefill except that the
 * lists have h_q rows: v_idx [h_q][cap_v], v_cnt [h_q], s_off [h_q][cap_s],
 * s_cnt [h_q]; query head h still reads K/V head h / (h_q / h_kv).  Each
 * query head then has its own tile list, so K/V tiles are not shared
 * between the heads of a group.  Workspace: vs_attn_workspace_bytes(h_q, n,
 * cap_v, cap_s). */
vs_status vs_sparse_attn_prefill_qh(const void* q, const void* k, const void* v, vs_dtype dt,
                                    int h_q, int h_kv, int n, int d, float scale,
                                    const int32_t* v_idx, const int32_t* v_cnt, int cap_v,
                                    const int32_t* s_off, const int32_t* s_cnt, int cap_s,
                                    void* out, float* lse, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* Packed batch of independent causal sequences.  Sequence s holds rows
 * cu_seqlens[s] .. cu_seqlens[s+1]-1 of q [h_q][total_n][d], k/v
 * [h_kv][total_n][d], out and lse [h_q][total_n]; it attends only within
 * itself, with positions (and so columns and offsets) counted from its
 * first row.  cu_seqlens is a HOST array of nseq + 1 ascending entries from
 * 0 to total_n (empty sequences allowed).  Lists are per sequence:
 * v_idx [nseq][S][cap_v], v_cnt [nseq][S], s_off [nseq][S][cap_s], s_cnt
 * [nseq][S], with S = h_kv, or h_q when sets_per_query_head is nonzero.
 * The whole batch is one tile build and one attention launch on `stream`:
 * the workspace, of vs_attn_varlen_workspace_bytes(S, nseq, longest
 * sequence, cap_v, cap_s) bytes, holds the tile lists of all nseq * S
 * index-set rows and a table of the sequences, which the call writes there
 * with small kernels (no host buffer outlives the call).  The attention
 * grid takes the sequences longest first.  The tile counters sum over the
 * batch: vs_attn_tile_counts(ws, nseq * S, longest, cap_v, cap_s,
 * nseq * h_q, ...).  Supported: as vs_sparse_attn_prefill, with each
 * sequence's K/V of one head under 2 GiB, nseq * S below 2^22 and the
 * whole batch's attention grid below 2^23 workgroups; the workspace is too
 * small (VS_ERR_WORKSPACE) if sized for one sequence. */
size_t vs_attn_varlen_workspace_bytes(int sets, int nseq, int max_len, int cap_v, int cap_s);
vs_status vs_sparse_attn_prefill_varlen(const void* q, const void* k, const void* v, vs_dtype dt,
                                        int h_q, int h_kv, int total_n, int d, float scale,
                                        const int32_t* cu_seqlens, int nseq,
                                        int sets_per_query_head, const int32_t* v_idx,
                                        const int32_t* v_cnt, int cap_v, const int32_t* s_off,
                                        const int32_t* s_cnt, int cap_s, void* out, float* lse,
                                        void* ws, size_t ws_bytes, hipStream_t stream);

/* Work counters of the most recent vs_sparse_attn_prefill (or its _qh or
 * _varlen form, with the arguments given there) that used `ws`, read
 * synchronously after `stream` finishes:
 *   tiles[0] = contiguous key tiles computed, summed over KV heads and query
 *              blocks; tiles[1] = gathered vertical tiles; tiles[2] = query
 *              rows per tile (for every query head of a KV group together);
 *              tiles[3] = keys per tile.
 * The MFMA work issued is (tiles[0] + tiles[1]) * tiles[2] * tiles[3]
 * query-key products, each 4*d flops. */
vs_status vs_attn_tile_counts(const void* ws, int h_kv, int n, int cap_v, int cap_s,
                              int h_q, int64_t tiles[4], hipStream_t stream);

/* ------------------------------------------ vertical/slash ground truth
 * VSPrefill (English page, section 2, "Key Components, 2. Distillation
 * Training, Ground Truth Generation"; German page, 2.B.2): the indexer is
 * distilled from full attention weights aggregated along vertical columns
 * and slash diagonals, computed without materialising the n x n matrix.
 * This call runs dense causal attention (out, lse as vs_sparse_attn_prefill
 * would with every offset selected) and then, per KV head g,
 *     a_v[g][j] = sum over the group's query heads h and rows i >= j of P^h_ij
 *     a_s[g][o] = sum over h and rows i >= o of P^h_{i,i-o}
 * with P the attention weights (softmax of scale * q_i . k_j over j <= i).
 * The sums are not normalised: each of a_v[g], a_s[g] totals G * n.
 *   q, k, v   : bf16 as for vs_sparse_attn_prefill
 *   out, lse  : bf16 [h_q][n][d], fp32 [h_q][n] (lse is required)
 *   a_v, a_s  : fp32 [h_kv][n]
 * P is formed in fp32 from the bf16 products and the fp32 lse of the first
 * pass.  Column sums add fp32 partials; a diagonal's partial within a
 * workgroup (at most 512 rows) is kept in fixed point with 22 fraction bits,
 * each weight rounded to nearest (at most 2^-23 off), and the partials meet
 * through fp32 atomics, so the last bits of both may vary run to run.
 * Any finite scale.  Supported: d in {64, 128}; h_q / h_kv in {1, 2, 4, 8,
 * 16}; K per head under 2 GiB; h_kv <= 65535.  The workspace holds the list
 * of all offsets and the attention workspace. */
size_t vs_aggregate_workspace_bytes(int h_kv, int n);
vs_status vs_attn_aggregate(const void* q, const void* k, const void* v, int h_q, int h_kv, int n,
                            int d, float scale, void* out, float* lse, float* a_v, float* a_s,
                            void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------ FlashPrefill block discovery
 * FlashPrefill (gist.science summary of arXiv 2603.06199, Spanish page,
 * section 2.A "Estrategia de Aproximacion de Bloques", 2.B "Umbralizacion
 * Dinamica Basada en Maximos"): query and key blocks are 64 positions (the
 * last may be short), nb = ceil(n / 64).  For KV head g and query block I the
 * probes are rows 64 I + m (64 / skel), m < skel, below n, of every query
 * head of the group; each probe's distribution over the candidate blocks
 * J < I is the softmax of scale * q . kbar_J, kbar_J the mean key of block J
 * (its exponential is the geometric mean of the block's exponentials); the
 * block score is that probability averaged over the probes.  Kept: the J < I
 * with score >= alpha * max_J score (one fp32 product), and J = I always.
 *   q, k   : bf16, [h_q][n][d] and [h_kv][n][d], row-major, device memory
 *   skel   : probes per query head and block; divides 64; G * skel <= 32
 *   alpha  : (0, 1]
 *   mask   : out, uint32 [h_kv][nb][words_per_row], bit b of word w set when
 *            key block 32 w + b is kept for that query block (words past I
 *            are zero); words_per_row >= ceil(nb / 32)
 *   score  : optional out (NULL to skip), fp32 [h_kv][nb][nb], the block
 *            scores the mask was decided on (zero for J >= I)
 * Block means are summed in fp32 and held as a bf16 pair (about 16
 * significant bits); the scores run on the matrix cores with fp32
 * accumulation.  Any finite scale.  Supported: d in {64, 128}; h_q / h_kv
 * in {1, 2, 4, 8, 16}; nb <= 16384; h_kv <= 65535.  The workspace holds the block means (bf16 hi and lo,
 * 4 * h_kv * nb * d bytes) and every block score of the call (fp32
 * [h_kv][nb][nb], 134 MB at n = 131072 with 8 KV heads), which the threshold
 * pass reads back instead of computing them again.  Nothing is allocated;
 * the calls only enqueue. */
size_t vs_block_workspace_bytes(int h_kv, int n, int d);
vs_status vs_block_discover(const void* q, const void* k, int h_q, int h_kv, int n, int d,
                            float scale, int skel, float alpha, uint32_t* mask, int words_per_row,
                            float* score, void* ws, size_t ws_bytes, hipStream_t stream);

/* Block-sparse causal prefill (FlashPrefill, same page, section 3 item 3:
 * a block-sparse kernel that walks an index list of kept blocks instead of
 * branching past masked ones).  Row i of a query head of KV head g attends
 * to the keys j <= i whose block j / 64 is set in mask[g][i / 64]; bits above
 * a query block's diagonal are ignored.  A row with no key gets out = 0 and
 * lse = -inf.  Arguments as vs_sparse_attn_prefill, with the mask of
 * vs_block_discover (or any caller-made mask of that layout) in place of the
 * index lists.  The workspace (vs_block_attn_workspace_bytes() bytes) holds
 * work counters.  Supported: as vs_sparse_attn_prefill (any finite scale),
 * with n <= 2^30 - 64. */
size_t vs_block_attn_workspace_bytes(void);
vs_status vs_block_attn_prefill(const void* q, const void* k, const void* v, vs_dtype dt, int h_q,
                                int h_kv, int n, int d, float scale, const uint32_t* mask,
                                int words_per_row, void* out, float* lse, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* Static text for a status code. */
const char* vs_status_str(vs_status s);

#ifdef __cplusplus
}
#endif

#endif /* VS_H_ */
