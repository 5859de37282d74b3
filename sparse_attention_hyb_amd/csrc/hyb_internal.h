// Internal interface between the C-ABI front end (hyb_api.cpp) and the HIP kernels.
// Plain structs passed to kernels by value, and one launcher per kernel family. Launchers
// assume validated arguments and return the hipError_t of their launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace hyb {

// A paged pool as the kernels see it (see hyb_paged in include/hyb.h).
struct PoolDev {
  uint8_t* data;
  const void* scale;
  const int32_t* block_table;
  int32_t dtype;
  int32_t dim;
  int32_t ratio;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t per_block;     // 256 / ratio
  int64_t entry_bytes;   // bytes of one entry in data
  // Optional device word: a kernel that meets a table entry >= num_blocks ORs kErrBadPage into
  // it (the entry still counts as absent). NULL: nothing is recorded.
  uint32_t* err;
};
constexpr uint32_t kErrBadPage = 1u;

// Query i -> (sequence, position): decode form (seq_lens != nullptr: seq = i, p = len - 1) or
// prefill form (seq = q_seq ? q_seq[i] : i, p = q_pos[i]).
struct QueryDev {
  const int32_t* seq_lens;
  const int32_t* q_seq;
  const int32_t* q_pos;
};

enum Dtype : int32_t { F32 = 0, BF16 = 1, FP8 = 2, FP4 = 3 };

// ---- compressor and raw-window insert -------------------------------------------------------
struct CompressArgs {
  const void* x;
  int32_t x_dtype;
  const float* gate;
  const int32_t* cu_seqlens;
  const int32_t* start_pos;
  int32_t batch;
  int32_t max_new_tokens;
  void* state;          // [batch][ratio][dim] in x_dtype
  float* state_logits;
  int32_t mode;
  PoolDev out;
  int32_t rope_dim;
  double rope_base;
  float eps;
  double theta[64];   // RoPE frequencies base^(-2i / rope_dim), i < rope_dim / 2 (host-formed)
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t s);

// Query RMSNorm + RoPE of new tokens, with their window entries (kv: the tokens' K=V rows in x,
// their window pool in out, positions and RoPE as in the insert).
struct QNormArgs {
  CompressArgs kv;
  const void* q;       // [T][n_heads][dim]
  int32_t q_dtype;
  void* q_out;         // same shape and dtype (may be q)
  int32_t n_heads;
  float eps;
};
// Up to two compressor calls riding along as extra workgroups of another launch (the indexer's or
// the attention's): n[j] workgroups for call j, or 0. A call runs there only when nothing else in
// that launch reads what it writes or writes what it reads. Kernels take the two calls as two
// separate arguments (c0, c1): an array indexed at run time would be copied to scratch memory.
struct SideWork {
  CompressArgs c[2];
  int32_t n[2];
  // the step before the attention (query RMSNorm + RoPE and window insert) riding along with the
  // indexer: n_prep workgroups of four of its waves, prep_gx per sequence
  QNormArgs prep;
  int32_t n_prep;
  int32_t prep_gx;
};
hipError_t launch_swa_insert(const CompressArgs& a, hipStream_t s);

hipError_t launch_q_norm_kv_insert(const QNormArgs& a, hipStream_t s);
// n pages of page_bytes: dst + dst_page[j] * page_bytes <- src_dev + src_page[j] * page_bytes,
// skipping every j whose source page is outside [0, n_src) or destination page outside [0, n_dst)
hipError_t launch_gather_pages(const void* src_dev, int32_t n_src, void* dst, int32_t n_dst,
                               const int32_t* src_page, const int32_t* dst_page, int32_t n,
                               int64_t page_bytes, hipStream_t s);

// ---- indexer scores -------------------------------------------------------------------------
struct ScoreArgs {
  const void* q;
  int32_t q_dtype;
  const float* w;
  QueryDev qd;
  int32_t n_q;
  int32_t n_heads;
  int32_t max_pos;
  int32_t window;
  PoolDev pool;
  float* scores;
  int64_t ld;
  // Optional, for the selector that follows (the hand-off): per part of kScorePartKeys keys, the
  // cumulative histogram of the top kTopBits bits of the order keys, [n_q][part_ld][kTopBins]
  // uint16 (entry b = the part's keys whose top bits are >= b); `scores` then holds, per row of
  // ld uint32 words, each part's (order key, index) pairs bucketed by those bits, highest first,
  // as uint2 at kScorePartKeys * part.
  uint16_t* part_hist;
  int32_t part_ld;
  // Optional, with part_hist: per-query bin counts of the top kTopBits key bits over the whole row,
  // uint32 [n_q][kTopBins], zero before the call; the hand-off adds each part's counts (the
  // selector reads the row's first-pass bin from it and zeroes it again).
  uint32_t* row_hist;
};
hipError_t launch_index_score(const ScoreArgs& a, hipStream_t s, const SideWork* side = nullptr);
constexpr int kTopBits = 10;                  // the selector's first radix pass (then 11 + 11)
constexpr int kTopBins = 1 << kTopBits;
constexpr int kScorePartKeys = 1024;          // keys per partial histogram (one indexer workgroup)
constexpr int kMaxTopK = 2048;                // largest k of a top-k selection (HYB_KMAX)
constexpr int kTopkMaxParts = 4096;           // parts per row the hand-off selector takes
constexpr int kRowHistRows = 256;             // queries of one call with a per-row histogram
constexpr size_t kRowHistBytes = (size_t)kRowHistRows * kTopBins * sizeof(uint32_t);
constexpr size_t kRowDoneBytes = (size_t)kRowHistRows * sizeof(uint32_t);   // per-row reader counts

// ---- top-k ----------------------------------------------------------------------------------
// Row lengths come from `lengths` or, if null, from n_visible(p_i, ratio, window) of the queries.
struct TopkArgs {
  const float* scores;
  int64_t ld;
  const int32_t* lengths;
  QueryDev qd;
  int32_t ratio;
  int32_t window;
  int32_t n_q;
  int32_t max_len;
  int32_t k;
  int32_t* out;
  // Optional (after the indexer, see ScoreArgs::part_hist): `scores` is the hand-off of (key,
  // index) pairs and these cumulative histograms give the first radix pass.
  const uint16_t* part_hist;
  int32_t part_ld;
  // Optional, with part_hist: the indexer's per-row bin counts (ScoreArgs::row_hist); the selector
  // zeroes each row after reading it.
  uint32_t* row_hist;
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// ---- attention ------------------------------------------------------------------------------
// The indexer's hand-off (see ScoreArgs) as a workgroup that selects one row's top k itself reads
// it: the attention kernel of a decode step that fuses the selection.
struct SelDev {
  const uint32_t* pairs;        // row i: (key, index) word pairs at pairs + i * ld, part p at 2048 p
  int64_t ld;                   // words per row (>= 2048 * part_ld)
  const uint16_t* part_hist;    // [n_q][part_ld][kTopBins] cumulative counts per part
  int32_t part_ld;
  uint32_t* row_hist;           // [n_q][kTopBins] bin counts per row; zero again after the call
  uint32_t* row_done;           // [n_q] workgroups done reading row_hist; zero again after the call
  int32_t* out;                 // optional [n_q][k] selected rows (logical indices)
  int32_t max_nv;               // host bound on any row's length
};

struct AttnArgs {
  const void* q;
  int32_t q_dtype;
  QueryDev qd;
  int32_t n_q;
  int32_t n_heads;
  int32_t dim;
  PoolDev swa;
  PoolDev comp;
  const int32_t* topk;
  int32_t k;
  int32_t window;
  float scale;
  int32_t rope_dim;
  double rope_base;
  void* out;
  int32_t out_dtype;
  float* out_scale;   // FP8 output: one scale per (query, head) row
  int32_t max_keys;   // host bound on keys per query (window + compressed)
  // split-K plan (filled by plan_attention)
  int32_t n_split;
  int32_t chunk;      // keys per split
  int32_t use_mfma;
  // Split partials: each split's output normalised by its own softmax sum, [n_q][n_split][n_heads]
  // [dim], fp32 from the generic kernel and bf16 from the MFMA kernel (whose probabilities are
  // bf16 already); m (natural-log units) and l per split and head in part_ml [n_q][n_split][2][n_heads].
  void* part_o;
  float* part_ml;
  // MFMA path: the RoPE(-p) table of every query, [n_q][64 pairs][cos, sin], written by the query's
  // first split for the combine (which otherwise forms it itself).
  float* rope_tab;
  // Balanced decode plan (MFMA path, set with qplan): the launch has n_slots workgroup slots and
  // every workgroup derives from the queries' lengths how their keys are cut into pieces of equal
  // size (at most n_split per query) and which piece is its own; the piece's partial goes to its
  // slot, and the query's first slot and piece count to qplan [n_q][2] for the combine. NULL: n_split
  // pieces of `chunk` keys per query, slot = query * n_split + piece.
  int32_t* qplan;
  int32_t n_slots;
  // Decode step with the selection fused (sel.pairs set): each workgroup of query i selects the
  // top k of row i from the hand-off itself instead of reading topk.
  SelDev sel;
};

// Split plan and workspace size for an attention call; identical for sizing and for launching.
struct AttnPlan {
  int32_t use_mfma;
  int32_t n_split;
  int32_t chunk;
  size_t o_bytes;    // part_o bytes, rounded up to 256; part_ml follows
  size_t rope_off;   // MFMA path: offset of rope_tab (after part_ml), else 0
  int32_t balanced;  // the balanced decode plan (n_slots slots, qplan at qplan_off)
  int32_t n_slots;
  size_t qplan_off;
  size_t ws_bytes;
};
// balanced: a decode launch, whose queries may differ in length (the plan then balances the key
// work over the workgroups on the device when the MFMA kernel runs with more than one split).
AttnPlan plan_attention(int32_t n_q, int32_t n_heads, int32_t dim, int32_t max_keys,
                        int32_t q_dtype, int32_t pool_dtype, bool balanced);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// Attention with the selection fused (a.sel set, the MFMA kernel) and up to two compressor calls
// riding along with its launch, then the combine.
hipError_t launch_attention_select(const AttnArgs& a, const SideWork* side, hipStream_t s);
bool attention_select_supported(const AttnArgs& a);
hipError_t launch_attention_compress(const AttnArgs& a, const CompressArgs& c, hipStream_t s);

// Offloaded C4 pool: device-side working-set admission and write-back (offload.hip).
constexpr int kMaxOffloadSlots = 16384;   // working-set slots at most (one workgroup assigns them)
struct OffloadArgs {
  const int32_t* topk;          // [batch][k] selected entries (< 0: none)
  int32_t batch, k;
  const int32_t* extra;         // [n_extra] page keys also needed
  int32_t n_extra;
  int32_t* dev_table;           // [batch][max_blocks] logical block -> slot, -1 absent
  const int32_t* mirror_table;  // [batch][max_blocks] logical block -> mirror page
  int32_t max_blocks, per_page; // entries per page
  int32_t* slot_owner;          // [n_slots] page key or -1
  uint32_t* slot_stamp;         // [n_slots] last step that needed the slot (0: never)
  int32_t n_slots;
  uint32_t step;
  uint8_t* mirror;              // device alias of the pinned host pages
  int32_t n_mirror_pages;
  uint8_t* pool;                // [n_slots][page_bytes]
  int64_t page_bytes;
  uint8_t* mirror_scale;        // device alias of the mirror's scale pages, or NULL
  uint8_t* pool_scale;
  int64_t scale_page_bytes;     // 0: no scales
  int32_t* result;              // [2] misses admitted, misses left out
};
size_t offload_ws_bytes(int32_t batch, int32_t max_blocks, int32_t n_slots);
hipError_t launch_offload_admit(const OffloadArgs& a, void* ws, hipStream_t s);
hipError_t launch_offload_write_back(const OffloadArgs& a, const int32_t* seq_lens, int ratio,
                                     int64_t entry_bytes, int64_t scale_bytes, hipStream_t s);

}  // namespace hyb
