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
};

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
hipError_t launch_swa_insert(const CompressArgs& a, hipStream_t s);

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
hipError_t launch_q_norm_kv_insert(const QNormArgs& a, hipStream_t s);
// n pages of page_bytes: dst + dst_page[j] * page_bytes <- src_dev + src_page[j] * page_bytes
hipError_t launch_gather_pages(const void* src_dev, void* dst, const int32_t* src_page,
                               const int32_t* dst_page, int32_t n, int64_t page_bytes,
                               hipStream_t s);

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
};
hipError_t launch_index_score(const ScoreArgs& a, hipStream_t s);
constexpr int kTopBits = 10;                  // the selector's first radix pass (then 11 + 11)
constexpr int kTopBins = 1 << kTopBits;
constexpr int kScorePartKeys = 1024;          // keys per partial histogram (one indexer workgroup)
constexpr int kTopkMaxParts = 4096;           // parts per row the hand-off selector takes

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
};
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// ---- attention ------------------------------------------------------------------------------
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
};

// Split plan and workspace size for an attention call; identical for sizing and for launching.
struct AttnPlan {
  int32_t use_mfma;
  int32_t n_split;
  int32_t chunk;
  size_t o_bytes;    // part_o bytes, rounded up to 256; part_ml follows
  size_t ws_bytes;
};
AttnPlan plan_attention(int32_t n_q, int32_t n_heads, int32_t dim, int32_t max_keys,
                        int32_t q_dtype, int32_t pool_dtype);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_compress(const AttnArgs& a, const CompressArgs& c, hipStream_t s);

}  // namespace hyb
