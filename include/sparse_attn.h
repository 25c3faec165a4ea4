/*
 * sparse_attn.h -- C ABI of a dynamic-sparse ("DSA"-style) attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * The method follows the page "国产AI芯片完成前沿大模型Day-0适配:稀疏注意力与混合精度推理
 * 全解析" (ruibaoantu.com), section 2, cited below as [DSA-page]:
 *   §2.1  an indexer scores every cached key against each query on the GPU, and a
 *         reduction keeps the top-K key indices per query;
 *   §2.2  the KV cache is stored in fixed blocks (pages) of contiguous tokens and the
 *         selected rows are gathered out of them before computing;
 *   §2.3  prefill and decode run the selection + gather + attention with different
 *         parallel shapes (prefill overlaps the next block's gather with compute; decode
 *         loads only the active rows);
 *   §2.4  vision tokens form a prefix that is always attended in full and never enters the
 *         sparse screening.
 * Dense causal attention is the special case where every causal key is selected
 * (sparse_attn_fwd_prefill with indices == NULL).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Ownership   The caller owns every buffer. All array pointers are DEVICE pointers, except
 *              the descriptor itself, which is read on the host during the call and may be
 *              freed as soon as the call returns. The library keeps no state between calls
 *              and allocates no memory (sparse_attn_fwd_decode_noalloc alone uses a static
 *              device buffer of the library, described there).
 *  Streams     `stream` is a hipStream_t (NULL = the default stream). Every call only
 *              enqueues work on it and returns; nothing synchronises.
 *  Errors      Each call returns SA_OK (0) or an SA_ERR_* code. All argument checks run on
 *              the host before anything is enqueued; on an error nothing is launched and no
 *              output is touched. SA_ERR_HIP means a launch was rejected by the runtime;
 *              earlier launches of the same call may then already be enqueued.
 *  Device data The CONTENTS of device arrays (page ids, sequence lengths, indices) are the
 *              caller's contract and are not validated. Kernels still never read or write
 *              out of bounds: a page id outside [0, num_pages) or an index outside the
 *              query's causal range is skipped, which makes the result unspecified but safe.
 *              sparse_attn_validate reports such contents; with SPARSE_ATTN_CHECK=1 in the
 *              environment every call validates the device data it reads first, into a report
 *              of the library that sparse_attn_check_report reads back.
 *  Alignment   Every array pointer must be 16-byte aligned (SA_ERR_ALIGN otherwise).
 *  Threads     Calls are re-entrant; concurrent calls on different streams are safe as long
 *              as their output and workspace buffers do not overlap.
 *
 * Positions   A call processes a block of q_len query tokens per sequence. Query i of
 *             sequence b sits at position  pos = seq_lens[b] - q_tail + i  (q_tail >= q_len
 *             is the distance from the block's first query to the end of the sequence:
 *             q_tail = T for a whole prefill, q_tail = 1 for a decode step). The cache holds
 *             seq_lens[b] tokens including the queries themselves; a query attends to keys
 *             0..pos.
 * Selection   Forced keys F = {t : 0 <= t < min(P, pos+1)}; candidate keys
 *             C = {t : P <= t <= pos}. The index list of a (sequence, query, KV group) is
 *             F followed by the top-K of C by (indexer score descending, token ascending),
 *             all in ascending token order and padded with -1 to width P + K. Query head h
 *             belongs to KV group h / (H_q / H_kv).
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 1

enum sa_status {
  SA_OK = 0,
  SA_ERR_NULL = 1,         /* a required pointer is NULL */
  SA_ERR_SHAPE = 2,        /* inconsistent or out-of-range sizes */
  SA_ERR_UNSUPPORTED = 3,  /* a size the kernels are not built for (e.g. head_dim 96) */
  SA_ERR_WORKSPACE = 4,    /* workspace missing or smaller than the *_workspace_size value */
  SA_ERR_HIP = 5,          /* the HIP runtime rejected a launch */
  SA_ERR_ABI = 6,          /* descriptor abi_version differs from SA_ABI_VERSION */
  SA_ERR_ALIGN = 7,        /* a pointer is not 16-byte aligned */
  SA_ERR_SCRATCH = 8       /* the call needs more than the static scratch buffer holds (noalloc) */
};

/*
 * Paged KV-cache descriptor ([DSA-page] §2.2: fixed-size blocks of contiguous tokens).
 *
 * Pools are indexed [page][head][slot][...]: one page holds page_size consecutive tokens of
 * every head, and within a page each head's rows are contiguous, so one head of one page is
 * a single contiguous (page_size x row) block.
 *   k_pool, v_pool  bf16 (raw uint16 bits) [num_pages][num_kv_heads][page_size][head_dim]
 *   kidx_pool       int8                   [num_pages][num_idx_heads][page_size][idx_dim]
 *   page_table      int32 [batch][max_pages_per_seq]; logical page p of sequence b is
 *                   physical page page_table[b * max_pages_per_seq + p]
 *   seq_lens        int32 [batch]; tokens cached per sequence, each in [1, max_seq_len]
 * A contiguous cache is the same descriptor with page_size = the sequence length and an
 * identity page table.
 * kidx_pool may be NULL for calls that do not score (attention only); k_pool/v_pool may be
 * NULL for calls that only score/select.
 */
typedef struct sa_paged_kv {
  int32_t abi_version;        /* must be SA_ABI_VERSION */
  int32_t batch;              /* B >= 1 */
  int32_t num_kv_heads;       /* H_kv >= 1 */
  int32_t head_dim;           /* d: 64 or 128 */
  int32_t num_idx_heads;      /* H_idx: num_kv_heads, or 1 (one indexer key shared by all groups) */
  int32_t idx_dim;            /* d_idx: 32, 64 or 128 (ignored when kidx_pool is NULL) */
  int32_t page_size;          /* tokens per page: a power of two, >= 64 */
  int32_t max_pages_per_seq;  /* row length of page_table */
  int64_t num_pages;          /* pages in each pool; num_pages * page_size < 2^31 */
  int32_t max_seq_len;        /* host-side bound on seq_lens[b]; <= max_pages_per_seq * page_size */
  int32_t prefix_len;         /* P >= 0: forced always-attended prefix ([DSA-page] §2.4) */
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int8_t* kidx_pool;
  const int32_t* page_table;
  const int32_t* seq_lens;
} sa_paged_kv;

/* SA_ABI_VERSION of the built library. */
int32_t sparse_attn_abi_version(void);

/* A static, human-readable name for a status code (never NULL). */
const char* sparse_attn_status_string(int32_t status);

/*
 * Indexer ([DSA-page] §2.1): exact int8 scores of every candidate key.
 *
 *   scores[b][i][gi][t] = sum_j q_idx[b][i][gi][j] * kidx(b, t, gi)[j]   for P <= t <= pos
 *
 * accumulated in int32 (exact: |score| <= idx_dim * 2^14 <= 2^21).
 *   q_idx   int8  [batch][q_len][num_idx_heads][idx_dim]
 *   scores  int32 [batch][q_len][num_idx_heads][score_row_stride]; only the candidate
 *           columns are written, the rest of each row is left untouched.
 * Requires kidx_pool, page_table, seq_lens; score_row_stride >= max_seq_len and a multiple
 * of 4; 1 <= q_len <= q_tail <= max_seq_len.
 */
int32_t sparse_attn_index(const sa_paged_kv* kv, const int8_t* q_idx, int32_t q_len,
                          int32_t q_tail, int32_t* scores, int64_t score_row_stride,
                          void* stream);

/*
 * Top-K selection ([DSA-page] §2.1, with the forced prefix of §2.4).
 *
 * For every (b, i, gi) writes the index list described in the header comment:
 *   indices int32 [batch][q_len][num_idx_heads][prefix_len + top_k]
 * Ties are broken by the lower token index, so the result is unique and deterministic.
 *   scores  as written by sparse_attn_index (same q_len/q_tail/row stride); only the
 *           candidate columns are read.
 * workspace: at least sparse_attn_topk_workspace_size(...) bytes of device memory (may be
 * NULL when that size is 0). Its contents on entry do not matter.
 */
size_t sparse_attn_topk_workspace_size(const sa_paged_kv* kv, int32_t q_len, int32_t top_k);
int32_t sparse_attn_topk(const sa_paged_kv* kv, const int32_t* scores, int64_t score_row_stride,
                         int32_t q_len, int32_t q_tail, int32_t top_k, int32_t* indices,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused indexer + top-K ([DSA-page] §2.1): the index lists that sparse_attn_index followed by
 * sparse_attn_topk would produce (bit-identical), without materialising the score rows.
 *
 *   q_idx    int8  [batch][q_len][num_idx_heads][idx_dim]
 *   indices  int32 [batch][q_len][num_idx_heads][prefix_len + top_k]
 * For decode-shaped calls (q_len == 1, rows of >= 16384 candidates) it scores every key once
 * and writes only the keys at or above a per-chunk provisional threshold (taken from the
 * chunk's first 4096 keys); the selection checks that no threshold could have dropped a
 * selected key and rescores exactly the chunks whose threshold could have, so the result never
 * depends on the thresholds (on scores packed into few values or tied, the call takes up to
 * about twice its time on spread scores).
 * Many-query blocks (q_len >= 16) of rows up to 32768 candidates hold 16-bit order-preserving
 * keys of the scores in the workspace instead (half the traffic) and settle the keys that tie
 * at the K-th largest by recomputing their exact int8 scores. Other shapes run the two-step
 * path with the score rows held in the workspace.
 * workspace: sparse_attn_index_topk_workspace_size(kv, q_len, top_k) bytes of device memory;
 * its contents on entry do not matter.
 */
size_t sparse_attn_index_topk_workspace_size(const sa_paged_kv* kv, int32_t q_len, int32_t top_k);
int32_t sparse_attn_index_topk(const sa_paged_kv* kv, const int8_t* q_idx, int32_t q_len,
                               int32_t q_tail, int32_t top_k, int32_t* indices, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Hybrid index lists: the selection of sparse_attn_index_topk plus a local window. Global sparse
 * attention next to local sliding-window attention is the hybrid described on the page
 * "…在摩尔线程MTT S5000上的原生推理优化实践" (blog.csdn.net) §2.3; the window is read here as a
 * second forced set like the prefix of [DSA-page] §2.4. For a query at pos the forced keys are
 * the prefix (t < min(P, pos + 1)) and the window (max(0, pos - window + 1) <= t <= pos); the
 * top-K runs over the remaining causal keys, ties to the lower token. The list holds all of
 * them ascending, -1 padded:
 *   indices  int32 [batch][q_len][num_idx_heads][prefix_len + top_k + window]
 * window = 0 gives sparse_attn_index_topk's lists. The attention entry points take these lists
 * with index_width = prefix_len + top_k + window.
 * workspace: sparse_attn_index_topk_window_workspace_size(kv, q_len, top_k, window) bytes of
 * device memory; its contents on entry do not matter. window >= 0.
 */
size_t sparse_attn_index_topk_window_workspace_size(const sa_paged_kv* kv, int32_t q_len,
                                                    int32_t top_k, int32_t window);
int32_t sparse_attn_index_topk_window(const sa_paged_kv* kv, const int8_t* q_idx, int32_t q_len,
                                      int32_t q_tail, int32_t top_k, int32_t window,
                                      int32_t* indices, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * Prefill attention ([DSA-page] §2.3, prefill): online-softmax attention of a block of
 * queries over their index lists, or dense causal attention when indices == NULL.
 *
 *   q        bf16 [batch][q_len][num_q_heads][head_dim]
 *   indices  int32 [batch][q_len][num_idx_heads][index_width] lists as written by
 *            sparse_attn_topk (ascending, -1 padded), or NULL for dense causal attention
 *            (every key 0..pos; index_width is then ignored)
 *   out      bf16 [batch][q_len][num_q_heads][head_dim]
 *   lse      float [batch][q_len][num_q_heads] (natural-log sum of exp of the scaled
 *            logits), or NULL
 * For each query head h:  z_t = sm_scale * q_h . K[t];  out = sum_t softmax(z)_t V[t].
 * sm_scale must be positive and finite (SA_ERR_SHAPE otherwise; the same holds for decode).
 * fp32 accumulation; out is rounded to bf16 (nearest-even). num_q_heads must be a multiple
 * of num_kv_heads with group size H_q/H_kv in {1, 2, 4, 8} for the sparse path.
 */
int32_t sparse_attn_fwd_prefill(const sa_paged_kv* kv, const uint16_t* q, int32_t num_q_heads,
                                int32_t q_len, int32_t q_tail, const int32_t* indices,
                                int32_t index_width, float sm_scale, uint16_t* out, float* lse,
                                void* stream);

/*
 * Per-row selection thresholds ([DSA-page] §2.1): the top-K of every (b, i, gi) row as two
 * numbers instead of an index list. With C the row's candidates (see Selection above), tau
 * the K-th largest indexer score among them and t_cut the largest token scoring tau that the
 * lower-index rule still takes, a key t of C is selected exactly when
 *     s(t) > tau   or   (s(t) == tau and t <= t_cut).
 * Rows with at most top_k candidates take all of them (tau = INT32_MIN, t_cut = INT32_MAX);
 * t_cut = INT32_MAX also when every candidate scoring tau is taken.
 *   q_idx       int8  [batch][q_len][num_idx_heads][idx_dim]
 *   thresholds  int32 [batch][q_len][num_idx_heads][2]   (tau, t_cut)
 * Keys on pages missing from the table are not candidates. Requires max_seq_len <= 131072
 * (SA_ERR_UNSUPPORTED otherwise). No workspace.
 */
int32_t sparse_attn_select_thresholds(const sa_paged_kv* kv, const int8_t* q_idx, int32_t q_len,
                                      int32_t q_tail, int32_t top_k, int32_t* thresholds,
                                      void* stream);

/*
 * Sparse prefill in one call ([DSA-page] §2.3: prefill fuses index selection, the gather of the
 * selected keys and attention): indexer, top-K selection and attention of a block of queries,
 * the result of sparse_attn_index_topk followed by sparse_attn_fwd_prefill on its lists.
 *   q, out, lse  as for sparse_attn_fwd_prefill;  q_idx as for sparse_attn_index_topk
 * Two ways to compute it, chosen by `path`:
 *   SA_PREFILL_MASKED  no index lists: sparse_attn_select_thresholds' (tau, t_cut) per row, the
 *                      dense kernel's selection masks written from indexer scores recomputed
 *                      on the matrix units, then attention over every causal key with the
 *                      unselected ones masked. Cost follows the causal length. A block with
 *                      too few queries to fill the chip splits its key tiles among several
 *                      workgroups and merges their results.
 *   SA_PREFILL_GATHER  index lists (sparse_attn_index_topk) and attention over gathered rows.
 *                      Cost follows top_k.
 *   SA_PREFILL_AUTO    masked when q_len >= 64 and top_k is at least 1/20 of the block's mean
 *                      candidate count (the crossover measured on MI355X for blocks of 128 to
 *                      2048 queries); gathered otherwise.
 *                      sparse_attn_prefill_fused_choice tells which path AUTO takes (or -1 if
 *                      none applies).
 * The masked path needs max_seq_len <= 131072; the gathered one a group size H_q/H_kv in
 * {1, 2, 4, 8}; a forced path that does not apply returns SA_ERR_UNSUPPORTED.
 * workspace: sparse_attn_prefill_fused_workspace_size(kv, num_q_heads, q_len, q_tail, top_k,
 * path) bytes of device memory (0 when no path applies); its contents on entry do not matter.
 */
enum sa_prefill_path { SA_PREFILL_AUTO = 0, SA_PREFILL_GATHER = 1, SA_PREFILL_MASKED = 2 };
size_t sparse_attn_prefill_fused_workspace_size(const sa_paged_kv* kv, int32_t num_q_heads,
                                                int32_t q_len, int32_t q_tail, int32_t top_k,
                                                int32_t path);
int32_t sparse_attn_prefill_fused_choice(const sa_paged_kv* kv, int32_t num_q_heads, int32_t q_len,
                                         int32_t q_tail, int32_t top_k);
int32_t sparse_attn_prefill_fused(const sa_paged_kv* kv, const uint16_t* q, const int8_t* q_idx,
                                  int32_t num_q_heads, int32_t q_len, int32_t q_tail,
                                  int32_t top_k, float sm_scale, int32_t path, void* workspace,
                                  size_t workspace_bytes, uint16_t* out, float* lse, void* stream);

/*
 * Sparse prefill on dense matrix tiles ([DSA-page] §2.3, prefill): the result of
 * sparse_attn_fwd_prefill with the same index lists, computed by the dense causal kernel
 * over every key 0..pos with each key that is not in the query's list masked out of the
 * softmax. Its cost follows the causal length, not top_k, so it pays off when the lists are
 * a large share of the causal keys or the gather is the bottleneck (long prefill blocks:
 * matrix tiles instead of one 512-byte row gather per selected key).
 *   q, out, lse  as for sparse_attn_fwd_prefill
 *   indices      int32 [batch][q_len][num_idx_heads][index_width], entries -1 or token ids;
 *                ids outside 0..min(pos, seq_len-1) are skipped, and a key listed more than
 *                once counts once (lists from sparse_attn_topk never repeat a key)
 * A query whose list holds no key gets out = 0 and lse = -inf.
 * workspace: sparse_attn_prefill_masked_workspace_size(kv, q_len) bytes of device memory
 * (one 64-bit lane mask per (32 queries, 64-key tile, score slot): batch * num_idx_heads *
 * 8 * ceil(q_len / 256) * ceil(max_seq_len / 64) * 256 bytes); its contents on entry do not
 * matter. head_dim 64 or 128; any group size H_q/H_kv.
 */
size_t sparse_attn_prefill_masked_workspace_size(const sa_paged_kv* kv, int32_t q_len);
int32_t sparse_attn_fwd_prefill_masked(const sa_paged_kv* kv, const uint16_t* q,
                                       int32_t num_q_heads, int32_t q_len, int32_t q_tail,
                                       const int32_t* indices, int32_t index_width, float sm_scale,
                                       void* workspace, size_t workspace_bytes, uint16_t* out,
                                       float* lse, void* stream);

/*
 * KV-cache append ([DSA-page] §2.2: the cache is kept in fixed blocks of contiguous tokens,
 * found through the block table; §2.3: each decode step adds its token to the cache before
 * the selection and attention read it). Writes n_new new tokens per sequence into the pools:
 * token i of sequence b goes to position seq_lens[b] - n_new + i (seq_lens already counts the
 * new tokens), i.e. to page page_table[b][pos / page_size], slot pos % page_size.
 *   k_new, v_new  bf16 [batch][n_new][num_kv_heads][head_dim], both or neither (NULL: the K and
 *                 V pools are not written)
 *   kidx_new      int8 [batch][n_new][num_idx_heads][idx_dim], or NULL (indexer keys not written)
 * At least one of the two must be given. The pools named in the descriptor are written in
 * place, so they must be writable device memory for this call. Positions below 0 and tokens
 * whose page entry lies outside [0, num_pages) are skipped. 1 <= n_new <= max_seq_len.
 */
int32_t sparse_attn_kv_append(const sa_paged_kv* kv, const uint16_t* k_new, const uint16_t* v_new,
                              const int8_t* kidx_new, int32_t n_new, void* stream);

/*
 * KV-cache block allocator ([DSA-page] §2.4: a KV dynamic allocator hands out and takes back
 * cache blocks; in sparse mode it tracks layer and head and keeps an independent block map
 * per head, so that heads never write into each other's blocks). One call serves num_maps
 * independent maps, e.g. one per (layer, KV head), or one per layer when the heads of a
 * layer share pages as in sa_paged_kv.
 *   block_maps   uint32 [num_maps][ceil(num_pages / 32)]: bit p % 32 of word p / 32 set means
 *                block p of that map is taken; bits at or past num_pages are never touched
 *   page_tables  int32 [num_maps][batch][max_pages_per_seq]: each map's block tables
 *
 * sparse_attn_kv_alloc grows sequence b from old_lens[b] to new_lens[b] tokens: it needs the
 * logical blocks ceil(old / page_size) .. ceil(new / page_size) - 1 (none when new <= old).
 * Per map, the needs are served in (sequence, logical block) order by the free blocks in
 * ascending block number (first fit, so the result is deterministic); the blocks are marked
 * taken and written into the table. All or nothing per map: status[m] (int32 [num_maps]) is
 * 0 on success, the number of blocks missing when too few are free, or -1 when a length is
 * negative or needs more than max_pages_per_seq blocks; in the last two cases the map and
 * its table are left unchanged. Table entries other than the allocated ones are not written.
 *
 * sparse_attn_kv_release returns the blocks of every sequence b with release[b] != 0 (int32
 * [batch]): its logical blocks 0 .. ceil(seq_lens[b] / page_size) - 1 (at most
 * max_pages_per_seq) are cleared in the map and their table entries set to -1; an entry
 * outside [0, num_pages) clears nothing. A block must belong to one sequence only.
 *
 * 1 <= num_maps <= 65535, 1 <= batch <= 8192, page_size >= 1, max_pages_per_seq >= 1 and
 * batch * max_pages_per_seq < 2^31 (SA_ERR_SHAPE otherwise). Lengths and flags are device
 * arrays; maps and tables are updated in place on the stream.
 */
int32_t sparse_attn_kv_alloc(int32_t num_maps, int32_t num_pages, uint32_t* block_maps,
                             int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                             const int32_t* old_lens, const int32_t* new_lens,
                             int32_t* page_tables, int32_t* status, void* stream);
int32_t sparse_attn_kv_release(int32_t num_maps, int32_t num_pages, uint32_t* block_maps,
                               int32_t batch, int32_t page_size, int32_t max_pages_per_seq,
                               const int32_t* seq_lens, const int32_t* release,
                               int32_t* page_tables, void* stream);

/*
 * Decode attention ([DSA-page] §2.3, decode): one query token per sequence (pos =
 * seq_lens[b] - 1) attends to its index list. Each (b, KV group) list is cut into
 * num_splits chunks processed in parallel; partial softmax states (max, sum, weighted V in
 * fp32) are merged exactly in a fixed order, so results are deterministic.
 *
 *   q        bf16 [batch][num_q_heads][head_dim]
 *   indices  int32 [batch][num_idx_heads][index_width]
 *   out      bf16 [batch][num_q_heads][head_dim];  lse float [batch][num_q_heads] or NULL
 *   num_splits  0 = choose automatically, else 1..256
 * workspace: sparse_attn_decode_workspace_size(kv, num_q_heads, index_width, num_splits)
 * bytes of device memory.
 */
size_t sparse_attn_decode_workspace_size(const sa_paged_kv* kv, int32_t num_q_heads,
                                         int32_t index_width, int32_t num_splits);
int32_t sparse_attn_fwd_decode(const sa_paged_kv* kv, const uint16_t* q, int32_t num_q_heads,
                               const int32_t* indices, int32_t index_width, float sm_scale,
                               int32_t num_splits, void* workspace, size_t workspace_bytes,
                               uint16_t* out, float* lse, void* stream);

/*
 * Decode attention that allocates nothing, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 *
 * Computes exactly what sparse_attn_fwd_decode computes, with the same kernels and split
 * choice, but the split partials live in a static device buffer of the library instead of a
 * caller workspace: sparse_attn_decode_noalloc_max_bytes() bytes (16 MiB) on each GPU the
 * library runs on, held until the process ends. A call whose partials need more
 * (sparse_attn_decode_workspace_size(...) larger than that) returns SA_ERR_SCRATCH and
 * launches nothing. No hipMalloc/hipFree or other allocating routine is called; the first
 * call on a device looks up that device's copy of the buffer (hipGetSymbolAddress), so the
 * current device must be the one that owns `stream` and the pointers.
 * Every call on one GPU shares that GPU's buffer and it keeps the last call's contents (each
 * call rewrites every partial it reads, so nothing needs clearing): calls that overlap on one
 * GPU (different streams, or threads without ordering) race and give undefined results.
 * Arguments, layouts and the other status codes as for sparse_attn_fwd_decode.
 */
size_t sparse_attn_decode_noalloc_max_bytes(void);
int32_t sparse_attn_fwd_decode_noalloc(const sa_paged_kv* kv, const uint16_t* q,
                                       int32_t num_q_heads, const int32_t* indices,
                                       int32_t index_width, float sm_scale, int32_t num_splits,
                                       uint16_t* out, float* lse, void* stream);

/*
 * Workspace of any call in one function: the bytes the call `op` needs for these sizes
 * (0 when it needs none, or when the sizes are invalid for it). `extra` is the call's own
 * parameter: the local window (SA_OP_INDEX_TOPK_WINDOW), the path (SA_OP_PREFILL_FUSED) or
 * num_splits (SA_OP_DECODE, where top_k is the index width); it is ignored otherwise. q_tail
 * matters only for SA_OP_PREFILL_FUSED, num_q_heads for it and SA_OP_DECODE. Equal to the
 * per-call *_workspace_size functions.
 */
enum sa_op {
  SA_OP_TOPK = 1,
  SA_OP_INDEX_TOPK = 2,
  SA_OP_INDEX_TOPK_WINDOW = 3,
  SA_OP_PREFILL_MASKED = 4,
  SA_OP_PREFILL_FUSED = 5,
  SA_OP_DECODE = 6
};
size_t sparse_attn_workspace_size(int32_t op, const sa_paged_kv* kv, int32_t q_len, int32_t q_tail,
                                  int32_t top_k, int32_t num_q_heads, int32_t extra);

/*
 * Validation of device data (the checks SPARSE_ATTN_CHECK=1 runs before every call).
 * Report: int32 [8] of device memory, written on the stream:
 *   [0] sequence lengths outside [1, max_seq_len]
 *   [1] page-table entries outside [0, num_pages), among the pages each sequence's tokens use
 *   [2] index-list entries that are neither -1 nor a token in [0, pos] of their query
 *   [3] index-list entries that do not follow the list's ascending order (-1 only at the end)
 *   [4] flat position (b * max_pages_per_seq + p) of the first bad page-table entry, else INT32_MAX
 *   [5] flat position of the first bad list entry (row * index_width + k), else INT32_MAX
 *   [6] calls checked, [7] 0
 * sparse_attn_validate clears `report`, then checks the descriptor's sequence lengths and page
 * table and, when indices is not NULL, the lists indices [batch][q_len][num_idx_heads]
 * [index_width] of a block of q_len queries at q_tail (positions as for the other calls).
 * With SPARSE_ATTN_CHECK=1 in the environment, every entry point taking a descriptor (except
 * the block allocator's) runs the same checks on what it reads before its own launches, adding
 * to a report of the library (a static device array per GPU, so no allocation);
 * sparse_attn_check_report copies it into `report` on the stream and clears it. Calls that
 * overlap on one GPU add to the same report.
 */
int32_t sparse_attn_validate(const sa_paged_kv* kv, const int32_t* indices, int32_t index_width,
                             int32_t q_len, int32_t q_tail, int32_t* report, void* stream);
int32_t sparse_attn_check_report(int32_t* report, void* stream);

/*
 * Roofline micro-benchmarks. They measure what the device reaches on the operations the path is
 * bound by, with the instructions the kernels use, so that roofline fractions can be given
 * against measured ceilings as well as vendor peaks. The caller times them (e.g. with events on
 * `stream`); each workgroup writes at most one word of `sink` (uint32 [workgroups]).
 *   sparse_attn_calib_read    streams `bytes` (a multiple of 16, >= 16) of `buf` with 16-byte
 *                             nontemporal loads: bytes / time is the streaming read bandwidth.
 *   sparse_attn_calib_gather  loads n_rows random 256-byte rows of `pool` (pool_bytes a multiple
 *                             of 256), rows[k] = row number (int32; a number outside the pool
 *                             reads row 0): 256 * n_rows / time is the row-gather bandwidth.
 *   sparse_attn_calib_mfma    `iters` x 4 back-to-back matrix instructions per wave, 4 waves per
 *                             workgroup: kind 0 = v_mfma_f32_32x32x16_bf16 (32768 flop each),
 *                             kind 1 = v_mfma_i32_32x32x32_i8 (65536 op each).
 * 1 <= workgroups <= 65536. Pointers are device pointers, 16-byte aligned.
 */
int32_t sparse_attn_calib_read(const void* buf, size_t bytes, uint32_t* sink, int32_t workgroups,
                               void* stream);
int32_t sparse_attn_calib_gather(const void* pool, size_t pool_bytes, const int32_t* rows,
                                 int64_t n_rows, uint32_t* sink, int32_t workgroups, void* stream);
int32_t sparse_attn_calib_mfma(int32_t kind, int32_t iters, int32_t workgroups, uint32_t* sink,
                               void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
