/*
 * hyb.h - C ABI of the MI355X (gfx950) hybrid compressed/sparse + sliding-window attention step.
 *
 * The method (DeepSeek-V4-style hybrid attention) is described on these pages:
 *   [vLLM]  "Day-0 support for DeepSeek V4 Pro and Flash on vLLM" - the "four moves" list
 *           (shared K/V + inverse RoPE; c4a / c128a KV compression; DeepSeek Sparse Attention
 *           over compressed tokens; short sliding window), the fp8 attention cache / fp4 indexer
 *           cache remark, and the "vLLM side" list (one logical block of 256 native positions
 *           for every compression rate; fused compressor + RMSNorm + RoPE + cache insert; fused
 *           Q-norm + KV RoPE + K insert).
 *   [SGLang] "DeepSeek-V4 launch review" (SGLang/Miles day-0 blog), section "Shadow Radix":
 *           each layer is sliding-window attention over the newest 128 raw tokens plus either
 *           C4 (top-512 sparse over 4:1 compressed KV) or C128 (dense over 128:1 compressed KV);
 *           each compression layer keeps its in-progress compression state in a state pool.
 *
 * Conventions shared by every entry point
 *   - Every pointer is a device pointer unless it says "host". The caller owns all memory:
 *     inputs, outputs, pools, block tables, state and workspace. The library never allocates,
 *     frees or synchronises, keeps no global mutable state (apart from a thread-local error
 *     string and the process-wide settings of hyb_set_error_word) and is re-entrant.
 *   - HYB_LOG set to anything but "" or "0" in the environment (read once, at the first call)
 *     makes the entry points report on stderr what they launch: attention plans, the parts of
 *     a decode step and where its side work runs, one line per launch.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null stream).
 *   - Return value: HYB_OK, or an error code. All argument checks run on the host before any
 *     HIP call, so a non-OK status means nothing was enqueued and outputs are untouched
 *     (HYB_ELAUNCH: a launch failed; earlier kernels of the same call may have run).
 *     hyb_last_error() describes the most recent failure on the calling thread.
 *   - Faults inside kernels surface at the caller's next synchronisation. Kernels never
 *     dereference a block whose table entry is negative or >= num_blocks: such entries are
 *     treated as absent (skipped on write, masked out on read); hyb_set_error_word makes the
 *     kernels report entries >= num_blocks.
 *   - Positions are absolute, 0-based raw-token positions. A query at position p sees the
 *     raw window [max(0, p - window + 1), p] and the compressed entries 0 .. n_vis(p) - 1 with
 *     n_vis(p) = ceil(max(0, p - window + 1) / ratio) (every complete group that holds at least
 *     one position older than the window). Every entry point that takes a window and a ratio
 *     requires window >= ratio (HYB_EINVAL otherwise): then every visible group is complete,
 *     and the group a token at p completes is not yet visible at p.
 *   - RoPE rotates the last rope_dim dims in adjacent pairs: pair i = (D - rope_dim + 2i,
 *     D - rope_dim + 2i + 1) turns by pos * rope_base^(-2i / rope_dim). Angles are formed and
 *     reduced in double precision.
 */
#ifndef HYB_H
#define HYB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HYB_ABI_VERSION 5

/* [vLLM] "vLLM side": one logical block = 256 native (raw) positions for every compression
 * rate, i.e. 256 raw entries, 64 C4 entries or 2 C128 entries. */
#define HYB_BLOCK_POSITIONS 256
/* Largest top-k the selector supports ([SGLang] "Shadow Radix" uses k = 512). */
#define HYB_KMAX 2048

typedef enum hyb_status {
  HYB_OK = 0,
  HYB_EINVAL = 1,     /* bad argument (NULL pointer, size, ratio, dtype mismatch, ...) */
  HYB_ENOTSUP = 2,    /* valid but not implemented (dtype / shape combination) */
  HYB_EWORKSPACE = 3, /* workspace missing or smaller than the *_workspace_bytes() result */
  HYB_ELAUNCH = 4     /* a HIP launch failed */
} hyb_status;

/* Element storage types. FP8_E4M3 = OCP E4M3 ("fn": no inf, max 448) with one float32 scale per
 * entry; FP4_E2M1 = OCP MX E2M1 with one E8M0 scale byte per 32 elements (value =
 * e2m1 * 2^(scale - 127); scale bytes 27..187, i.e. 2^-100 .. 2^60, for which every value is
 * widened to bf16 exactly). [vLLM]: "fp8 attention cache + fp4 indexer cache". */
typedef enum hyb_dtype {
  HYB_F32 = 0,
  HYB_BF16 = 1,
  HYB_FP8_E4M3 = 2,
  HYB_FP4_E2M1 = 3
} hyb_dtype;

/* Compressor pooling of the r raw tokens of a group: arithmetic mean, or softmax over one scalar
 * logit per raw position followed by the weighted sum. */
typedef enum hyb_pool_mode { HYB_POOL_MEAN = 0, HYB_POOL_SOFTMAX_GATE = 1 } hyb_pool_mode;

/* A paged pool ([vLLM] "unified hybrid KV cache"; [SGLang] "three heterogeneous KV pools").
 * Entry g of a pool with compression `ratio` lives in logical block floor(g * ratio / 256), slot
 * g mod (256 / ratio). Physical layout, all row-major, contiguous:
 *   data  F32/BF16: [num_blocks][256/ratio][dim] elements
 *         FP8_E4M3: [num_blocks][256/ratio][dim] bytes
 *         FP4_E2M1: [num_blocks][256/ratio][dim/2] bytes, element 2j in the low nibble of byte j
 *   scale FP8_E4M3: float [num_blocks][256/ratio];  FP4_E2M1: uint8 [num_blocks][256/ratio][dim/32];
 *         NULL otherwise.
 *   block_table: int32 [batch][max_blocks], logical -> physical block, negative = absent.
 * The descriptor itself is read on the host during the call and may be freed afterwards. */
typedef struct hyb_paged {
  void* data;
  void* scale;
  const int32_t* block_table;
  int32_t dtype;      /* hyb_dtype */
  int32_t dim;
  int32_t ratio;      /* 1 (raw sliding-window entries), 4 (C4) or 128 (C128) */
  int32_t num_blocks; /* physical blocks in data; num_blocks * 256/ratio < 2^31 */
  int32_t max_blocks; /* columns of block_table */
  int32_t reserved;   /* must be 0 */
} hyb_paged;

int32_t hyb_abi_version(void);
const char* hyb_status_str(int32_t status);

/* hyb_set_error_word - optional detection of corrupt block tables: from now on, every kernel of
 * the calling thread's current device that meets a block-table entry >= its pool's num_blocks ORs
 * HYB_ERR_BAD_PAGE into *word (the entry still counts as absent, as the conventions say). word:
 * a 4-byte-aligned device address on that device, owned by the caller, who zeroes it and reads it
 * after synchronising; NULL turns the detection off for the device. Calls enqueued before this
 * one are not affected. HYB_ELAUNCH when there is no current device. */
#define HYB_ERR_BAD_PAGE 1u
int32_t hyb_set_error_word(uint32_t* word);
/* Thread-local description of the last non-OK status returned on this thread (host string,
 * owned by the library, valid until the next call on the thread). */
const char* hyb_last_error(void);

/* --------------------------------------------------------------------------------------------
 * hyb_compress - KV compressor: pool -> RMSNorm -> RoPE -> paged insert, with a state ring.
 * [vLLM] "c4a / c128a KV compression" and the fused "compressor + RMSNorm + RoPE + cache insert";
 * [SGLang] "Shadow Radix": in-progress groups wait in a per-layer compression-state pool.
 *
 * New raw tokens x[cu_seqlens[b] .. cu_seqlens[b+1]) of sequence b sit at positions
 * start_pos[b] + i. Every group g = floor(pos / ratio) completed by them is written to `out` as
 *   entry g = RoPE(RMSNorm(Pool(x_{g*r} .. x_{g*r+r-1})), g*r + r - 1),
 * RMSNorm over all dim dims with eps and unit gain, the pool per `mode`. Tokens of a group that
 * started in an earlier call are read from the state ring; the tokens of the trailing incomplete
 * group are written to it (slot = pos mod ratio). One call serves decode (one token per sequence)
 * and chunked prefill; calls for one sequence must come in position order.
 *   x             [T][dim], x_dtype F32 or BF16 (T = cu_seqlens[batch])
 *   gate_logits   float [T] for HYB_POOL_SOFTMAX_GATE; NULL for HYB_POOL_MEAN
 *   cu_seqlens    int32 [batch + 1], non-decreasing, cu_seqlens[0] = 0
 *   start_pos     int32 [batch], position of each sequence's first new token
 *   max_new_tokens host bound on cu_seqlens[b+1] - cu_seqlens[b] (sizes the grid)
 *   state         [batch][ratio][dim] in x_dtype: raw tokens of the in-progress group
 *   state_logits  float [batch][ratio] (gate mode), NULL for mean
 *   out           host descriptor of the C4 / C128 pool (ratio 4 or 128, dim = x's dim,
 *                 block_table rows indexed by b); dtype F32 or BF16, or quantised as stored
 *                 (quantise-on-insert, [vLLM] "fp8 attention cache + fp4 indexer cache"):
 *                 FP8_E4M3 - one float32 scale per entry, scale = amax / 448 (1 for an all-zero
 *                   entry), code = E4M3 nearest to value / scale (float32 quotient), ties to
 *                   the even code, saturating at 448;
 *                 FP4_E2M1 (dim % 32 == 0; compressed indexer keys) - per 32 values the E8M0
 *                   byte e + 127 with e = floor(log2 amax) - 2 clamped to [-100, 60], code =
 *                   E2M1 nearest to value * 2^-e, ties to the even code, saturating at 6.
 * ------------------------------------------------------------------------------------------ */
int32_t hyb_compress(const void* x, int32_t x_dtype, const float* gate_logits,
                     const int32_t* cu_seqlens, const int32_t* start_pos, int32_t batch,
                     int32_t max_new_tokens, void* state, float* state_logits, int32_t mode,
                     const hyb_paged* out, int32_t rope_dim, double rope_base, float eps,
                     void* stream);

/* The arguments of one hyb_compress call, as one struct (same meaning, layout and rules; the
 * stream is the caller's of the entry point that takes the struct). */
typedef struct hyb_compress_call {
  const void* x;
  int32_t x_dtype;
  const float* gate_logits;
  const int32_t* cu_seqlens;
  const int32_t* start_pos;
  int32_t batch;
  int32_t max_new_tokens;
  void* state;
  float* state_logits;
  int32_t mode;
  const hyb_paged* out;
  int32_t rope_dim;
  double rope_base;
  float eps;
} hyb_compress_call;

/* --------------------------------------------------------------------------------------------
 * hyb_swa_insert - raw sliding-window entries s_t = RoPE(x_t, t) (no norm) written to the raw
 * pool (ratio 1) at position t. The "KV RoPE + K insert" step of [vLLM]'s fused-kernel list.
 * Arguments as in hyb_compress; swa->dtype F32, BF16 or FP8_E4M3 (dim <= 2048; each entry
 * quantised as stored, with the FP8_E4M3 rule of hyb_compress).
 * ------------------------------------------------------------------------------------------ */
int32_t hyb_swa_insert(const void* x, int32_t x_dtype, const int32_t* cu_seqlens,
                       const int32_t* start_pos, int32_t batch, int32_t max_new_tokens,
                       const hyb_paged* swa, int32_t rope_dim, double rope_base, void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_q_norm_kv_insert - the step before the attention for new tokens, in one launch ([vLLM]
 * "vLLM side": fused "Q-norm + KV RoPE + K insert"). For token i of sequence b (position
 * pos = start_pos[b] + i, tokens ordered as in hyb_compress):
 *   q_out[tok][h] = RoPE(RMSNorm(q[tok][h]), pos)   for every head h (RMSNorm over dim, eps,
 *                                                    unit gain; RoPE on the last rope_dim dims)
 *   window entry pos of sequence b = RoPE(kv[tok], pos)   (exactly hyb_swa_insert of kv)
 *   q      [T][n_heads][dim], q_dtype F32 or BF16;  q_out the same shape and dtype (may be q)
 *   kv     [T][dim], kv_dtype F32 or BF16 (T = cu_seqlens[batch]);  1 <= n_heads <= 128
 *   swa    raw pool (ratio 1) of dim `dim` <= 2048, dtype F32, BF16 or FP8_E4M3 (quantised as
 *          in hyb_swa_insert)
 * The query rows it writes are what hyb_attn_decode / hyb_attn_prefill take at these positions.
 * ------------------------------------------------------------------------------------------ */
int32_t hyb_q_norm_kv_insert(const void* q, int32_t q_dtype, int32_t n_heads, const void* kv,
                             int32_t kv_dtype, const int32_t* cu_seqlens, const int32_t* start_pos,
                             int32_t batch, int32_t max_new_tokens, void* q_out,
                             const hyb_paged* swa, int32_t rope_dim, double rope_base, float eps,
                             void* stream);

/* The arguments of one hyb_q_norm_kv_insert call, as one struct (same meaning, layout and rules;
 * the stream is the caller's of the entry point that takes the struct). */
typedef struct hyb_prep_call {
  const void* q;
  int32_t q_dtype;
  int32_t n_heads;
  const void* kv;
  int32_t kv_dtype;
  const int32_t* cu_seqlens;
  const int32_t* start_pos;
  int32_t batch;
  int32_t max_new_tokens;
  void* q_out;
  const hyb_paged* swa;
  int32_t rope_dim;
  double rope_base;
  float eps;
} hyb_prep_call;

/* --------------------------------------------------------------------------------------------
 * hyb_gather_pages - fill pages of a device working set from a pinned host mirror in one launch
 * (the offload of [SGLang] "HiSparse": the C4 pool lives in CPU memory, missing pages are brought
 * to a device buffer every step). For j < n:
 *   dst + dst_page[j] * page_bytes  <-  src_host + src_page[j] * page_bytes   (page_bytes bytes)
 *   src_host     pinned host memory of n_src_pages pages (hipHostMalloc, or a pinned torch tensor);
 *                the kernel reads it through the device alias hipHostGetDevicePointer gives;
 *                HYB_EINVAL if it has none
 *   dst          device memory of n_dst_pages pages
 *   src_page, dst_page  int32 [n] in device memory. The indices are device data the host cannot
 *                see: a j whose src_page[j] is outside [0, n_src_pages) or dst_page[j] outside
 *                [0, n_dst_pages) is skipped (nothing read, nothing written). Destination pages
 *                must not repeat.
 *   page_bytes % 16 == 0; src_host and dst 16-byte aligned; n_src_pages, n_dst_pages >= 1.
 * ------------------------------------------------------------------------------------------ */
int32_t hyb_gather_pages(const void* src_host, int32_t n_src_pages, void* dst, int32_t n_dst_pages,
                         const int32_t* src_page, const int32_t* dst_page, int32_t n,
                         int64_t page_bytes, void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_offload_admit - one step's working-set update of an offloaded C4 pool, on the device.
 * [SGLang] "HiSparse": the C4 pool lives in a pinned host mirror; the device keeps a working set of
 * pages, brings in every page the step's selection misses and evicts the least recently used pages
 * the step does not need. Here no top-k row is read back: in stream order,
 *   1. every page (logical block of `entries_per_page` entries; key = sequence * max_blocks +
 *      block) that a row of topk selects, and every key in extra, is needed this step; a needed
 *      resident page's slot gets stamp `step`;
 *   2. the needed pages that are not resident, in ascending key order, take as many slots among
 *      those the step does not need, the least recently used first (smallest stamp, then lowest
 *      slot; a never-used slot has stamp 0), the i-th page the i-th of those slots in slot order;
 *      dev_table, slot_owner and slot_stamp are updated (an evicted page's entry becomes -1);
 *   3. each admitted page is copied from mirror page mirror_table[key] into its slot (and its
 *      scale page, when scale_page_bytes > 0).
 *   topk     int32 [batch][k] entry indices (device; < 0 ignored); k = 0 allowed
 *   extra    int32 [n_extra] page keys (device; e.g. the pages receiving new entries), or NULL
 *   dev_table    int32 [batch][max_blocks] (device): block -> slot, -1 absent (the working set's
 *                block table, as the attention entry points read it)
 *   mirror_table int32 [batch][max_blocks] (device): block -> mirror page
 *   slot_owner   int32 [n_slots] (device): page key or -1; slot_stamp uint32 [n_slots] (device)
 *   step     >= 1 and greater than every earlier call's step on this workspace
 *   mirror_host  pinned host pages [n_mirror_pages][page_bytes] (read through the device alias);
 *   pool     device pages [n_slots][page_bytes]; mirror_scale_host / pool_scale: the same for the
 *            per-entry scales (scale_page_bytes > 0), else NULL and 0
 *   workspace    hyb_offload_workspace_bytes(batch, max_blocks, n_slots) bytes, zero before its
 *            first use; calls that share it must not overlap
 *   result   int32 [2] (device): pages admitted, pages left out because the slots the step could
 *            free were too few (then their blocks stay absent: size the working set for a step)
 * 1 <= n_slots <= 16384; page_bytes and scale_page_bytes multiples of 16 and of entries_per_page;
 * pool and mirror 16-byte aligned. Out-of-range keys and table entries are skipped.
 *
 * hyb_offload_write_back - back up new entries to the mirror, on the device: for each sequence b
 * whose position p = seq_lens[b] - 1 completes a compressed entry ((p + 1) % ratio == 0), entry
 * (p + 1) / ratio - 1 (and its scale) goes from its resident slot to its mirror page through the
 * mirror's device alias (skipped when its page is not resident). Enqueued on any stream after the
 * compressor that wrote the entry, it runs asynchronously to the host and to the next step.
 * ------------------------------------------------------------------------------------------ */
size_t hyb_offload_workspace_bytes(int32_t batch, int32_t max_blocks, int32_t n_slots);
int32_t hyb_offload_admit(const int32_t* topk, int32_t batch, int32_t k, const int32_t* extra,
                          int32_t n_extra, int32_t* dev_table, const int32_t* mirror_table,
                          int32_t max_blocks, int32_t entries_per_page, int32_t* slot_owner,
                          uint32_t* slot_stamp, int32_t n_slots, uint32_t step, void* mirror_host,
                          int32_t n_mirror_pages, void* pool, int64_t page_bytes,
                          void* mirror_scale_host, void* pool_scale, int64_t scale_page_bytes,
                          void* workspace, size_t workspace_bytes, int32_t* result, void* stream);
int32_t hyb_offload_write_back(const int32_t* seq_lens, int32_t batch, int32_t ratio,
                               const int32_t* dev_table, const int32_t* mirror_table,
                               int32_t max_blocks, int32_t entries_per_page, int32_t n_slots,
                               const void* pool, int64_t page_bytes, void* mirror_host,
                               int32_t n_mirror_pages, const void* pool_scale,
                               void* mirror_scale_host, int64_t scale_page_bytes, void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_index_score - indexer scores over the visible compressed entries.
 * [vLLM] "DeepSeek Sparse Attention over compressed tokens"; [SGLang] "indexer top-k".
 *   score[i][g] = sum_h w[i][h] * max(0, q_idx[i][h] . key_g), g = 0 .. n_vis(q_pos[i]) - 1,
 * keys from `idx_pool` rows of sequence q_seq[i]; an entry whose block is absent scores -inf.
 * Entries g >= n_vis are not written.
 *   q_idx   [n_q][n_heads][idx_pool->dim], q_dtype F32 or BF16
 *   w       float [n_q][n_heads]
 *   q_seq   int32 [n_q] (NULL = identity);  q_pos int32 [n_q]
 *   max_pos host bound on q_pos;  scores float [n_q][scores_ld], scores_ld >= n_vis(max_pos)
 * idx_pool: dtype F32, BF16 or FP4_E2M1 (dim % 32 == 0), ratio 4 or 128.
 * ------------------------------------------------------------------------------------------ */
int32_t hyb_index_score(const void* q_idx, int32_t q_dtype, const float* w, const int32_t* q_seq,
                        const int32_t* q_pos, int32_t n_q, int32_t n_heads, int32_t max_pos,
                        int32_t window, const hyb_paged* idx_pool, float* scores,
                        int64_t scores_ld, void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_topk - exact top-k per row: the first min(k, len[i]) indices of row i under the order
 * (score descending, index ascending), -0.0 equal to +0.0, written ascending and padded with -1.
 * [SGLang] "Shadow Radix": C4 keeps the top-512 compressed entries.
 *   scores float [n_q][scores_ld];  lengths int32 [n_q] (valid prefix of each row, <= max_len)
 *   out_idx int32 [n_q][k];  1 <= k <= HYB_KMAX.  Scores must not be NaN.
 * ------------------------------------------------------------------------------------------ */
int32_t hyb_topk(const float* scores, int64_t scores_ld, const int32_t* lengths, int32_t n_q,
                 int32_t max_len, int32_t k, int32_t* out_idx, void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_index_score_keys / hyb_topk_keys - the two halves of hyb_index_topk, for callers that want
 * to place them (or time them) separately. Same selection as hyb_index_score + hyb_topk.
 * hyb_index_score_keys turns each score into its order key, a uint32 that sorts like the float
 * (non-negative: bits | 0x80000000; negative: ~bits; -0.0 stored as +0.0), and hands each block
 * p of 1024 entries of a row over as
 *   part_hist[p][b]  the number of the block's keys whose top 10 bits are >= b (b < 1024), and
 *   keys[2048 p ..]  the block's (key, entry index) pairs as uint32 pairs, ordered by the keys'
 *                    top 10 bits from high to low (order within equal bits unspecified);
 *   keys       uint32 [n_q][keys_ld], keys_ld >= 2048 * part_ld
 *   part_hist  uint16 [n_q][part_ld][1024], ceil(n_vis(max_pos) / 1024) <= part_ld <= 4096
 * so the selector reads only the pairs that can be chosen. Other arguments as in
 * hyb_index_score. hyb_topk_keys selects from them with the same q_pos,
 * max_pos, window and the pool's ratio (row i holds n_vis(q_pos[i]) entries), as hyb_topk does:
 *   out_idx int32 [n_q][k];  1 <= k <= HYB_KMAX.
 * ------------------------------------------------------------------------------------------ */
int32_t hyb_index_score_keys(const void* q_idx, int32_t q_dtype, const float* w,
                             const int32_t* q_seq, const int32_t* q_pos, int32_t n_q,
                             int32_t n_heads, int32_t max_pos, int32_t window,
                             const hyb_paged* idx_pool, uint32_t* keys, int64_t keys_ld,
                             uint16_t* part_hist, int64_t part_ld, void* stream);
int32_t hyb_topk_keys(const uint32_t* keys, int64_t keys_ld, const uint16_t* part_hist,
                      int64_t part_ld, const int32_t* q_pos, int32_t n_q, int32_t max_pos,
                      int32_t window, int32_t ratio, int32_t k, int32_t* out_idx, void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_index_topk - hyb_index_score followed by hyb_topk over n_vis(q_pos[i]) entries; the
 * scores live in the workspace (size from hyb_index_topk_workspace_bytes with the same n_q,
 * max_pos, window and ratio) in the hand-off form of hyb_index_score_keys, after a block of
 * per-row counts (1 MiB at the workspace's start) that the indexer adds to and the selector reads:
 * those bytes must be zero before the workspace's first use (allocate it zeroed once), and every
 * call leaves them zero, so the workspace can be reused for calls of any size, on one stream at a
 * time (also from a captured graph). At most 4096 * 1024 visible entries (HYB_ENOTSUP beyond).
 * ------------------------------------------------------------------------------------------ */
size_t hyb_index_topk_workspace_bytes(int32_t n_q, int32_t max_pos, int32_t window,
                                      int32_t ratio);
int32_t hyb_index_topk(const void* q_idx, int32_t q_dtype, const float* w, const int32_t* q_seq,
                       const int32_t* q_pos, int32_t n_q, int32_t n_heads, int32_t max_pos,
                       int32_t window, const hyb_paged* idx_pool, int32_t k, int32_t* out_idx,
                       void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_index_topk_noalloc - hyb_index_topk for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * arguments without the workspace, the same selection from the same kernels. Its scratch memory
 * is a static device array of HYB_NOALLOC_SCRATCH_BYTES per GPU, which the library holds from
 * the first call on that GPU until the process ends; the call allocates nothing. The scratch
 * that hyb_index_topk_workspace_bytes gives for these arguments must not exceed the array
 * (HYB_EINVAL otherwise; 64 MiB holds e.g. 16 queries at 2^20 positions or 64 at 2^18). Every
 * call on one GPU shares that GPU's array and its contents persist between calls: calls that
 * overlap on one GPU (other streams, other host threads) race, and the caller must order them.
 * The array starts at zero, and every call leaves the 1 MiB of per-row counts at its start zero
 * again, as hyb_index_topk needs.
 * The first call on a device looks up the array's address with that device current
 * (HYB_ELAUNCH if that fails).
 * ------------------------------------------------------------------------------------------ */
#define HYB_NOALLOC_SCRATCH_BYTES (64ull << 20)
int32_t hyb_index_topk_noalloc(const void* q_idx, int32_t q_dtype, const float* w,
                               const int32_t* q_seq, const int32_t* q_pos, int32_t n_q,
                               int32_t n_heads, int32_t max_pos, int32_t window,
                               const hyb_paged* idx_pool, int32_t k, int32_t* out_idx,
                               void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_attn_decode - one query token per sequence, p = seq_lens[b] - 1.
 * [vLLM] "Shared K/V + inverse RoPE", "short sliding window"; [SGLang] "Shadow Radix": SWA over
 * the newest `window` raw tokens plus either the selected C4 entries (topk_idx != NULL, sparse)
 * or every visible compressed entry (topk_idx == NULL, dense; the C128 case).
 * Per head h, with keys kappa_j = the raw window entries (positions ascending) then the chosen
 * compressed entries:  z_j = softmax_scale * q_h . kappa_j,  o_h = sum_j softmax(z)_j kappa_j
 * (values are the keys: one shared K=V head), then out_h = RoPE(o_h, -p).
 *   q        [batch][n_heads][dim] already rotated at p;  q_dtype F32 or BF16
 *   seq_lens int32 [batch] (>= 1);  max_seq_len host bound on seq_lens
 *   swa      raw pool (ratio 1);  comp compressed pool (ratio 4 or 128); same dtype, dim as q;
 *            pool dtype F32 (q F32), BF16 or FP8_E4M3 (q BF16)
 *   topk_idx int32 [batch][k] entries of comp (negative = unused), or NULL
 *   out      [batch][n_heads][dim], out_dtype F32, BF16 or FP8_E4M3. FP8_E4M3 (dim % 8 == 0,
 *            dim <= 2048) quantises each (query, head) row after the inverse RoPE ([vLLM] fused
 *            "inverse RoPE + fp8 quant"): uint8 E4M3 codes in out, the row's float32 scale in
 *            out_scale [batch][n_heads], with the FP8_E4M3 rule of hyb_compress (scale = amax /
 *            448, nearest code to value / scale, ties to even, saturating)
 *   out_scale float [batch][n_heads] for an FP8_E4M3 output, NULL otherwise
 *   workspace size from hyb_attn_decode_workspace_bytes with the same batch, n_heads, dim,
 *            max_seq_len, comp ratio, k (0 when topk_idx is NULL) and window.
 * ------------------------------------------------------------------------------------------ */
size_t hyb_attn_decode_workspace_bytes(int32_t batch, int32_t n_heads, int32_t dim,
                                       int32_t max_seq_len, int32_t comp_ratio, int32_t k,
                                       int32_t window);
int32_t hyb_attn_decode(const void* q, int32_t q_dtype, const int32_t* seq_lens, int32_t batch,
                        int32_t n_heads, int32_t max_seq_len, const hyb_paged* swa,
                        const hyb_paged* comp, const int32_t* topk_idx, int32_t k, int32_t window,
                        float softmax_scale, int32_t rope_dim, double rope_base, void* out,
                        int32_t out_dtype, float* out_scale, void* workspace,
                        size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_attn_decode_compress - hyb_attn_decode, then hyb_compress(*compress), on one stream.
 * [vLLM] "vLLM side" (multi-stream overlap of the step's kernels): with the 64 x 512 bf16
 * attention kernel and a compressor call that four waves run in four-dim chunks (dim <= 512,
 * dim % 4 == 0 for F32 x and % 8 for BF16 x, x / state / pool data 16-byte aligned), the
 * compressor's workgroups are launched together with the attention's split combine, so its
 * memory latency hides behind the combine; otherwise the compressor is launched after it.
 * The result is exactly that of the two calls in that order: the attention reads the pools as
 * they were before the call. In a decode step this equals compressing the new token first, as
 * an entry that a group completes at position p is not yet visible to the query at p
 * (n_vis(p) <= floor(p / ratio) for window >= ratio). compress's buffers must not overlap `out`
 * or the workspace. Arguments: those of hyb_attn_decode, then compress (non-NULL), then stream.
 * ------------------------------------------------------------------------------------------ */
int32_t hyb_attn_decode_compress(const void* q, int32_t q_dtype, const int32_t* seq_lens,
                                 int32_t batch, int32_t n_heads, int32_t max_seq_len,
                                 const hyb_paged* swa, const hyb_paged* comp,
                                 const int32_t* topk_idx, int32_t k, int32_t window,
                                 float softmax_scale, int32_t rope_dim, double rope_base,
                                 void* out, int32_t out_dtype, float* out_scale, void* workspace,
                                 size_t workspace_bytes, const hyb_compress_call* compress,
                                 void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_decode_step - one whole decode step of a hybrid attention layer for a batch of sequences
 * (one query token each, at p = seq_lens[b] - 1), with its kernels fused as far as the data flow
 * allows. [SGLang] "Shadow Radix": each layer is the window plus C4 top-k (sparse) or C128
 * (dense); [vLLM] "vLLM side": the compressor, indexer and window work of a step overlap.
 *   C4 layer (comp->ratio 4; q_idx, w and idx_pool given): the results of hyb_index_topk over
 *     n_vis(p) indexer keys (decode form: the query of sequence b is b at p), written to
 *     topk_out [batch][k] when that is not NULL, then hyb_attn_decode over those rows;
 *   C128 layer (comp->ratio 128; q_idx, w and idx_pool NULL): hyb_attn_decode, dense;
 *   then the n_compress <= 2 compressor calls compress[0 .. n_compress), as hyb_compress (e.g.
 *     the new tokens into the C4 pool and their indexer-key rows into the indexer-key pool);
 *   and first of all, when prep is not NULL, hyb_q_norm_kv_insert(*prep): the new tokens' query
 *     RMSNorm + RoPE (into prep->q_out, normally the step's q) and their window entries. On a C4
 *     layer its waves run as extra workgroups at the end of the indexer's launch, on the compute
 *     units that the indexer's first finishers leave ([vLLM] "vLLM side": the window insert and
 *     query prep overlap the indexer); the indexer reads nothing they write, so prep->q_out and
 *     the window pool's data must not overlap q_idx, w, the indexer-key pool or seq_lens.
 *     Otherwise it is launched first.
 * The result equals those calls made one after another (the prep first). The compressor calls may run beside the
 * indexer or the attention: that is exact because nothing else in the step reads what they write
 * (the entry a token at p completes is not visible at p, for window >= ratio) or writes what they
 * read. Their x, state and output pools must not overlap q, out, topk_out or the workspace.
 * Arguments as in hyb_index_topk (q_idx [batch][idx_heads][idx_pool->dim], w [batch][idx_heads])
 * and hyb_attn_decode; workspace sized by hyb_decode_step_workspace_bytes with the same batch,
 * n_heads, dim, max_seq_len, comp ratio, k (ignored for C128) and window. A C4 step's workspace
 * starts with HYB_STEP_ZERO_BYTES that must be zero before its first use (per-row counts; every
 * call leaves them zero). With the MFMA attention (64 heads x 512 dims, bf16 query) and batch
 * <= 256 the attention workgroups select their rows' top k themselves from the indexer's
 * hand-off (no separate selection kernel); the rows are the same.
 * ------------------------------------------------------------------------------------------ */
#define HYB_STEP_ZERO_BYTES ((1ull << 20) + 1024ull)
size_t hyb_decode_step_workspace_bytes(int32_t batch, int32_t n_heads, int32_t dim,
                                       int32_t max_seq_len, int32_t comp_ratio, int32_t k,
                                       int32_t window);
int32_t hyb_decode_step(const void* q, int32_t q_dtype, const int32_t* seq_lens, int32_t batch,
                        int32_t n_heads, int32_t max_seq_len, const hyb_paged* swa,
                        const hyb_paged* comp, const void* q_idx, int32_t q_idx_dtype,
                        const float* w, int32_t idx_heads, const hyb_paged* idx_pool, int32_t k,
                        int32_t* topk_out, int32_t window, float softmax_scale, int32_t rope_dim,
                        double rope_base, void* out, int32_t out_dtype, float* out_scale,
                        const hyb_prep_call* prep, const hyb_compress_call* compress,
                        int32_t n_compress, void* workspace, size_t workspace_bytes, void* stream);

/* --------------------------------------------------------------------------------------------
 * hyb_attn_prefill - causal attention for a chunk of query tokens: query i of sequence q_seq[i]
 * at position q_pos[i] attends to its own window and its own top-k row (or, with topk_idx NULL,
 * to every compressed entry visible at q_pos[i]). Same arithmetic and pools as hyb_attn_decode.
 *   q [n_q][n_heads][dim] rotated at q_pos;  q_seq int32 [n_q] (NULL = identity);  q_pos int32 [n_q]
 *   max_pos host bound on q_pos;  topk_idx int32 [n_q][k] or NULL;  out [n_q][n_heads][dim]
 *   (out_dtype and out_scale [n_q][n_heads] as in hyb_attn_decode)
 * ------------------------------------------------------------------------------------------ */
size_t hyb_attn_prefill_workspace_bytes(int32_t n_q, int32_t n_heads, int32_t dim,
                                        int32_t max_pos, int32_t comp_ratio, int32_t k,
                                        int32_t window);
int32_t hyb_attn_prefill(const void* q, int32_t q_dtype, const int32_t* q_seq,
                         const int32_t* q_pos, int32_t n_q, int32_t n_heads, int32_t max_pos,
                         const hyb_paged* swa, const hyb_paged* comp, const int32_t* topk_idx,
                         int32_t k, int32_t window, float softmax_scale, int32_t rope_dim,
                         double rope_base, void* out, int32_t out_dtype, float* out_scale,
                         void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HYB_H */
