// Indexer scores over the visible compressed entries:
//   score[i][g] = sum_h w[i][h] * max(0, q_idx[i][h] . key_g).
// Method: vLLM DeepSeek-V4 day-0 post ("DeepSeek Sparse Attention over compressed tokens"; fp4
// indexer cache) and the SGLang DeepSeek-V4 day-0 blog ("Shadow Radix": C4 keeps the top-512 of
// the indexer's scores).
//
// Kernels:
//  * score_mfma_reg: 64 heads x 128 dims, bf16 query, bf16 or fp4 (E2M1 + E8M0 per 32) keys, one
//    query per work item. The step streams every visible key once (the step's dominant HBM
//    traffic). S = Q . K^T runs on v_mfma_f32_32x32x16_bf16 with the 64 heads as the M dimension
//    (two 32-row blocks) and 32 keys as N; each lane then owns one key column and 32 of its heads,
//    so the ReLU-weighted head sum is 32 in-lane FMAs plus one cross-half add.
//  * score_mfma_multi: the same contraction for prefill chunks, four queries sharing each tile.
//  * score_generic: any (heads x dim) <= 8192, fp32 / bf16 / fp4 - one thread per key.
// For the selector that follows, all can instead hand over each part of kScorePartKeys keys as a
// cumulative histogram of the top kTopBits bits of the scores' order keys plus the part's
// (order key, index) pairs bucketed by those bits (see finish_parts): the first radix pass of the
// top-k, and the gathering of its candidates, ride along with the score stream.
#include <type_traits>

#include "common.h"
#include "compress_dev.h"

namespace hyb {

constexpr int kScoreKeysPerBlock = 2 * kScorePartKeys;  // keys per workgroup (MFMA kernel)
constexpr int kScoreParts = kScoreKeysPerBlock / kScorePartKeys;
constexpr int kMfmaHeads = 64;
constexpr int kMfmaDim = 128;

__device__ __forceinline__ float canonical_zero(float v) { return v == 0.0f ? 0.0f : v; }
// A workgroup-uniform read of data no kernel writes while this one runs, through the constant
// address space: a scalar load, which the wait counters track apart from the vector loads, so
// that it holds up none of them.
__device__ __forceinline__ int32_t uniform_ld(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}
// max(x, 0) for finite x as one integer max on the bit pattern: negative values (and -0) have a
// negative pattern and become +0, non-negative ones stay.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Eight E2M1 nibbles (one 32-bit word, element 0 in the low nibble) times a power-of-two block
// scale -> eight bf16 values, exactly, with gfx950's scaled conversion (two elements of one byte
// per instruction, low nibble first; it matches the arithmetic conversion bit for bit for every
// code and scales from 2^-100 to 2^60).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float sc) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// Selector hand-off (part_hist set). For each part of kScorePartKeys keys a workgroup writes
//  * its cumulative histogram over the top kTopBits bits of the order keys: part_hist[b] = number
//    of the part's keys whose top bits are >= b (uint16, <= kScorePartKeys), and
//  * the part's (order key, row index) pairs bucketed by those bits, highest bin first (order
//    within a bin unspecified), as uint2 at pairs + kScorePartKeys * part,
// so that the selector, once it knows the bin b0 of the k-th largest key, reads only the leading
// part_hist[b0] pairs of every part. The workgroup's keys are in lkeys[0, P * kScorePartKeys)
// (index g - base) and its per-part counts in lhist[P][kTopBins], which become bucket cursors;
// each pair goes straight to its bucket slot in the output (slots from LDS atomics on the cursors;
// a direct global scatter measured faster than sorting in LDS and copying out). 256 threads.
template <int P, bool kPacked = false>
__device__ __forceinline__ void finish_parts(const ScoreArgs& a, int i, int part0, int base, int end,
                                             const uint32_t* lkeys, uint32_t* lhist,
                                             uint32_t* wtot) {
  static_assert(kTopBins == 4 * 256, "four bins per thread");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  __syncthreads();   // keys and counts complete
#pragma unroll
  for (int q = 0; q < P; ++q) {
    if (base + q * kScorePartKeys >= end) break;   // uniform
    uint32_t* h = lhist + q * (kPacked ? kTopBins / 2 : kTopBins);
    // thread t owns bins 1023 - 4t - e (e < 4), i.e. bins in descending order across threads
    // (packed: two 16-bit counts per word, bin b in half b % 2 of word b / 2)
    uint32_t c[4], tot = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int bin = kTopBins - 1 - 4 * t - e;
      c[e] = kPacked ? (h[bin >> 1] >> (16 * (bin & 1))) & 0xffffu : h[bin];
      tot += c[e];
      if (a.row_hist != nullptr && c[e] != 0u)   // the row's counts for the selector's first pass
        atomicAdd(a.row_hist + (int64_t)i * kTopBins + bin, c[e]);
    }
    const uint32_t incl = wave_inclusive_scan(tot);
    if (lane == 63) wtot[q * 4 + w] = incl;
    __syncthreads();
    uint32_t before = incl - tot;
    for (int v = 0; v < w; ++v) before += wtot[q * 4 + v];
    // cum[b] = keys with top bits >= b; bucket b starts at cum[b] - count[b]
    uint32_t run = before;
    uint32_t cum[4], cur[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cur[e] = run;   // cursor: start of the bucket
      run += c[e];
      cum[e] = run;
    }
    if constexpr (kPacked) {   // bins 1020 - 4t .. 1023 - 4t: words 510 - 2t, 511 - 2t
      h[kTopBins / 2 - 2 - 2 * t] = cur[3] | (cur[2] << 16);
      h[kTopBins / 2 - 1 - 2 * t] = cur[1] | (cur[0] << 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) h[kTopBins - 1 - 4 * t - e] = cur[e];
    }
    // bins 1020 - 4t .. 1023 - 4t, ascending in memory
    uint2 wv;
    wv.x = cum[3] | (cum[2] << 16);
    wv.y = cum[1] | (cum[0] << 16);
    *reinterpret_cast<uint2*>(a.part_hist + ((int64_t)i * a.part_ld + part0 + q) * kTopBins +
                              (kTopBins - 4 - 4 * t)) = wv;
  }
  __syncthreads();
  const int nk = min(P * kScorePartKeys, end - base);
  uint2* pairs = reinterpret_cast<uint2*>(a.scores) + (int64_t)i * (a.ld / 2) +
                 (int64_t)part0 * kScorePartKeys;
  for (int j = t; j < nk; j += 256) {
    const uint32_t key = lkeys[j];
    const int q = j / kScorePartKeys;
    const uint32_t bin = key >> (32 - kTopBits);
    uint32_t slot;
    if constexpr (kPacked) {
      const uint32_t sh = 16 * (bin & 1u);
      slot = (atomicAdd(&lhist[q * (kTopBins / 2) + (bin >> 1)], 1u << sh) >> sh) & 0xffffu;
    } else {
      slot = atomicAdd(&lhist[q * kTopBins + bin], 1u);
    }
    pairs[q * kScorePartKeys + slot] = make_uint2(key, (uint32_t)(base + j));   // straight to its bucket
  }
}

// The hand-off of one part for one query by one wave (no workgroup barrier): the wave's 16-bit
// packed histogram of the part's keys becomes the cumulative histogram (written out) and bucket
// cursors (written back), then every key is scattered to its bucket in the output pairs. Lane l
// owns bins 1023 - 16 l - e (e < 16), i.e. bins in descending order across lanes.
__device__ __forceinline__ void finish_part_wave(const ScoreArgs& a, int i, int part, int base,
                                                 int end, const uint32_t* lkeys, uint32_t* lhist,
                                                 int lane) {
  uint32_t c[16], tot = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int bin = kTopBins - 1 - 16 * lane - e;
    c[e] = (lhist[bin >> 1] >> (16 * (bin & 1))) & 0xffffu;
    tot += c[e];
  }
  const uint32_t incl = wave_inclusive_scan(tot);
  uint32_t run = incl - tot;
  uint32_t cur[16], cum[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    cur[e] = run;
    run += c[e];
    cum[e] = run;
  }
  // bins 1008 - 16l .. 1023 - 16l: ascending in memory, bin 1023 - 16l - e holds cum[e]
  u32x4 w0, w1;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    w0[m] = cum[15 - 2 * m] | (cum[14 - 2 * m] << 16);
    w1[m] = cum[7 - 2 * m] | (cum[6 - 2 * m] << 16);
  }
  uint16_t* ph = a.part_hist + ((int64_t)i * a.part_ld + part) * kTopBins + (kTopBins - 16 - 16 * lane);
  *reinterpret_cast<u32x4*>(ph) = w0;
  *reinterpret_cast<u32x4*>(ph + 8) = w1;
#pragma unroll
  for (int m = 0; m < 8; ++m)   // word 504 - 8l + m: bins 1008 - 16l + 2m (low), + 1 (high)
    lhist[kTopBins / 2 - 8 - 8 * lane + m] = cur[15 - 2 * m] | (cur[14 - 2 * m] << 16);
  __builtin_amdgcn_wave_barrier();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the cursors before any lane's atomics
  __builtin_amdgcn_wave_barrier();
  uint2* pairs = reinterpret_cast<uint2*>(a.scores) + (int64_t)i * (a.ld / 2) +
                 (int64_t)part * kScorePartKeys;
  const int nk = min(kScorePartKeys, end - base);
  for (int j = lane; j < nk; j += 64) {
    const uint32_t key = lkeys[j];
    const uint32_t bin = key >> (32 - kTopBits);
    const uint32_t sh = 16 * (bin & 1u);
    const uint32_t slot = (atomicAdd(&lhist[bin >> 1], 1u << sh) >> sh) & 0xffffu;
    pairs[slot] = make_uint2(key, (uint32_t)(base + j));
  }
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane i's bytes land
// at LDS byte address lds + 16i. Issued through inline asm: with the compiler builtin every LDS
// read waits for all outstanding loads (the compiler cannot tell which LDS bytes a load writes),
// which would serialise the prefetch; here the caller waits with wait_vmcnt for exactly the tiles
// it reads. Younger loads or stores issued by the compiler only make such a wait stricter.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Decode form (one query per workgroup item), bf16 or fp4 keys: the contraction of score_mfma
// with every key tile fetched by fully coalesced loads into registers and passed through the
// wave's own LDS stage to the MFMA operand layout. A plain streaming read of this GPU's memory
// reaches about 7.1 TB/s with such loads against 6.0-6.3 TB/s through direct global -> LDS loads.
// A tile is 32 keys:
//   bf16: 32 x 256 B; load instruction j (< 8) brings key 4j + lane/16, 16-byte chunk lane % 16,
//         stored in the stage at chunk c ^ (n % 16) of row n (conflict-free for the stores and
//         for the operand reads: 32 keys, one logical chunk);
//   fp4:  32 x 64 B of E2M1 pairs + 32 x 4 E8M0 bytes; instruction j (< 2) brings key
//         16j + lane/4, chunk lane % 4, stored at chunk c ^ ((n / 2) % 4) of row n (eight lanes
//         reading one logical chunk of eight keys then hit eight different bank groups); lanes
//         below 32 bring key `lane`'s four scale bytes. Operands are widened exactly to bf16.
// Each wave keeps its next kDepth tiles in flight in registers and reads only its own stage, so
// the tile loop has no workgroup barrier.
// Work: an item is one block of kScoreKeysPerBlock visible keys of one query. Every workgroup
// derives the list of non-empty items from the queries' positions itself (one load per query and a
// prefix sum in LDS; up to kItemQueries queries, else it walks every (query, block) pair and skips
// the empty ones), and workgroup w takes items w, w + G, ...: the grid is a fixed size, whatever the
// lengths, and short and long rows spread evenly.
// kTile: a 32-key tile always lies in one block (256 / ratio >= 32, the C4 case); kHand: hand-off
// to the selector instead of plain scores. The first n_c0 + n_c1 workgroups run the compressor
// calls c0, c1 riding along with this launch.
constexpr int kItemQueries = 1024;
constexpr int kIndexWorkgroups = 512;

template <bool kFp4>
struct KeyFormat {
  static constexpr int kLoads = 8;          // 16-byte loads per lane per tile
  static constexpr int kRowBytes = 256;
  static constexpr int kStageBytes = 8192;
  static constexpr int kDepth = 2;          // tiles in flight per wave
};
template <>
struct KeyFormat<true> {
  static constexpr int kLoads = 2;
  static constexpr int kRowBytes = 64;
  static constexpr int kStageBytes = 2048 + 128;
  static constexpr int kDepth = 4;
};

template <bool kTile, bool kHand, bool kFp4>
__global__ __launch_bounds__(256, 1) void score_mfma_reg(ScoreArgs a, CompressArgs c0, CompressArgs c1,
                                                          int n_c0, int n_c1, QNormArgs prep, int n_prep,
                                                          int prep_gx) {
  using KF = KeyFormat<kFp4>;
  constexpr int kLoads = KF::kLoads, kDepth = KF::kDepth;
  __shared__ __attribute__((aligned(1024))) uint8_t stage[4][8192];
  __shared__ uint32_t lhist[kScoreParts * kTopBins];
  __shared__ int32_t tbl[kScoreKeysPerBlock / 2 + 2];
  __shared__ uint32_t lkeys[kScoreKeysPerBlock];
  __shared__ uint32_t wtot[kScoreParts * 4];
  __shared__ int32_t istart[kItemQueries + 1];
  __shared__ int32_t nvq[kItemQueries];
  static_assert(sizeof(stage) >= kCompressFusedLds, "a compressor workgroup fits the stages");
  int bid = blockIdx.x;
  if (bid < n_c0) {
    compress_fused<4>(c0, bid, reinterpret_cast<float*>(&stage[0][0]));
    return;
  }
  if (bid < n_c0 + n_c1) {
    compress_fused<4>(c1, bid - n_c0, reinterpret_cast<float*>(&stage[0][0]));
    return;
  }
  bid -= n_c0 + n_c1;
  const int n_wg = gridDim.x - n_c0 - n_c1 - n_prep;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (bid >= n_wg) {   // the step before the attention, last in the grid: its workgroups take the
                       // compute units that the indexer's first finishers leave
    const int k = bid - n_wg;
    q_norm_kv_wave_any(prep, k / prep_gx, (k % prep_gx) * 4 + wave, lane);
    return;
  }
  const int col = lane & 31;
  const int hf = lane >> 5;
  const int max_nv = n_visible(a.max_pos, a.pool.ratio, a.window);
  const int gx = (max_nv + kScoreKeysPerBlock - 1) / kScoreKeysPerBlock;
  // positions: seq_lens - 1 (decode) or q_pos; one source and offset chosen once, so that the
  // loads carry no branch and go out together
  const int32_t* pos_src = a.qd.seq_lens ? a.qd.seq_lens : a.qd.q_pos;
  const int pos_adj = a.qd.seq_lens ? 1 : 0;
  auto nv_of = [&](int q) {   // q uniform
    return min(n_visible(uniform_ld(pos_src + q) - pos_adj, a.pool.ratio, a.window), max_nv);
  };

  const int per_block = a.pool.per_block;   // 256 / ratio: a power of two
  const int pb_shift = __builtin_ctz(per_block);
  const int nk = kFp4 ? lane >> 2 : lane >> 4;
  const int ck = kFp4 ? lane & 3 : lane & 15;
  // bytes per key row: the pool's entry size for 128 dimensions (bf16: 256; fp4: 64, scales apart)
  constexpr int kRow = KF::kRowBytes;
  const uint32_t lane_off = nk * kRow + 16 * ck;   // this lane's bytes of the first load
  // Operand reads: lane (key col, hf) reads logical chunk 8hf + s (bf16) or 2hf + s (fp4) of its
  // key, stored at that chunk XOR (col % 16) or XOR ((col / 2) % 4). As the logical chunk is a
  // disjoint OR of the hf and s bits, its stored offset is the s = 0 offset XOR 16 s: one offset
  // per lane, and an XOR per read instead of a register per K-step.
  const uint32_t roff0 = kFp4 ? col * 64 + 16 * ((2 * hf) ^ ((col >> 1) & 3))
                              : col * 256 + 16 * ((8 * hf) ^ (col & 15));

  uint8_t* st = &stage[wave][0];
  auto rd16 = [&](int s) -> u32x4 {   // 16 bytes of K-step s's operand chunk
    return *reinterpret_cast<const u32x4*>(st + (roff0 ^ (16u * s)));
  };

  // ---- one item's prologue: the block-table entries of its key range (into tbl), the query's
  // operands and its head weights (registers), as independent loads issued together. In decode
  // form the sequence is the query itself. Operands as in score_mfma: d = 64*hf + 8*s + e, i.e.
  // lane (key col, hf) takes logical chunk 8*hf + s of its key at K-step s.
  bf16x8 qa[2][8];
  float wv[2][16];
  int lb0 = 0;
  auto fetch = [&](int i, int base, int end) {
    const int seq = (a.qd.seq_lens || !a.qd.q_seq) ? i : uniform_ld(a.qd.q_seq + i);
    lb0 = base >> pb_shift;
    const int n_lb = ((end - 1) >> pb_shift) - lb0 + 1;
    const int32_t* bt = a.pool.block_table + (int64_t)seq * a.pool.max_blocks;
    auto raw = [&](int j) {   // in bounds of the row; checked by phys_of
      return bt[min(lb0 + j, a.pool.max_blocks - 1)];
    };
    auto phys_of = [&](int j, int v) {
      if (lb0 + j >= a.pool.max_blocks) return -1;
      note_bad_page(a.pool, v);
      return (v >= 0 && v < a.pool.num_blocks) ? v : -1;
    };
    const int v0 = raw(min(tid, n_lb - 1));   // first entries: the load goes out before q and w's
    __builtin_amdgcn_sched_barrier(0);
    const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)i * kMfmaHeads * kMfmaDim;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        qa[mb][s] = *reinterpret_cast<const bf16x8*>(q + (32 * mb + col) * kMfmaDim + 64 * hf + 8 * s);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        wv[mb][r] = a.w[(int64_t)i * kMfmaHeads + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3)];
    if (tid < n_lb) tbl[tid] = phys_of(tid, v0);
    for (int j = tid + 256; j < n_lb; j += 256) tbl[j] = phys_of(j, raw(j));   // ratio 128 only
  };

  // ---- the item list: istart[q] = items of the queries before q (exclusive prefix sum), and
  // each query's visible key count in nvq. The workgroup's first item is guessed in the order of
  // the walk over every (query, block) pair, which is the list's own order whenever every query
  // sees max_nv keys (the usual batch of equal lengths); its prologue loads go out together with
  // the lengths', so that the list costs no extra round trip to memory in that case.
  const bool compact = a.n_q <= kItemQueries;
  const int g_i = bid / gx, g_base = (bid - g_i * gx) * kScoreKeysPerBlock;
  const bool guessed = g_i < a.n_q;   // uniform
  int total;
  if (compact) {
    // Every wave builds the whole list itself, writing the same values to the same LDS words, and
    // reads only words it has written itself (or identical ones): no workgroup barrier. Query
    // q = 64 g + lane for group g < n_grp.
    constexpr int kGroups = kItemQueries / 64;
    const int n_grp = (a.n_q + 63) >> 6;
    int pq[kGroups];   // queries past n_q read the last one's (in bounds, unused); no branch
#pragma unroll
    for (int g = 0; g < kGroups; ++g) pq[g] = pos_src[min(64 * g + lane, a.n_q - 1)];
    __builtin_amdgcn_sched_barrier(0);   // the lengths' loads before the guess's
    if (guessed) fetch(g_i, g_base, min(max_nv, g_base + kScoreKeysPerBlock));
    uint32_t run = 0;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      if (g >= n_grp) break;   // uniform
      const int q = 64 * g + lane;
      const int nv = q < a.n_q ? min(n_visible(pq[g] - pos_adj, a.pool.ratio, a.window), max_nv) : 0;
      const uint32_t cnt = (uint32_t)((nv + kScoreKeysPerBlock - 1) / kScoreKeysPerBlock);
      const uint32_t incl = wave_inclusive_scan(cnt);
      if (q < a.n_q) {
        istart[q] = (int32_t)(run + incl - cnt);
        nvq[q] = nv;
      }
      run += __builtin_amdgcn_readlane(incl, 63);
    }
    if (lane == 0) istart[a.n_q] = (int32_t)run;
    total = (int)run;
  } else {
    if (guessed) fetch(g_i, g_base, min(max_nv, g_base + kScoreKeysPerBlock));
    total = a.n_q * gx;
  }

  for (int item = bid; item < total; item += n_wg) {
    int i, base, nv;
    if (compact) {
      int lo = 0, hi = a.n_q - 1;   // last query whose first item is <= item
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (istart[mid] <= item) lo = mid; else hi = mid - 1;
      }
      // uniform across the workgroup: scalar registers keep the tile loop's control and the
      // item's addresses out of the vector registers
      i = __builtin_amdgcn_readfirstlane(lo);
      base = __builtin_amdgcn_readfirstlane((item - istart[i]) * kScoreKeysPerBlock);
      nv = __builtin_amdgcn_readfirstlane(nvq[i]);
    } else {
      i = item / gx;
      base = (item - i * gx) * kScoreKeysPerBlock;
      nv = nv_of(i);
    }
    if (base >= nv) continue;   // only in the walk over every pair; uniform
    const int end = min(nv, base + kScoreKeysPerBlock);
    if (item != bid) __syncthreads();   // the previous item's readers of the LDS are done
    // The previous item's hand-off stores have been issued. Waiting for them here (vmcnt 0, the
    // other counters free) leaves only loads outstanding in the tile loop, whose waits then count
    // tiles; with stores still in flight the compiler cannot count and waits for every load.
    if constexpr (kHand) __builtin_amdgcn_s_waitcnt(0x0F70);
    // the guess's range [g_base, min(max_nv, g_base + block)) covers [base, end) when it holds
    if (!(item == bid && guessed && i == g_i && base == g_base)) fetch(i, base, end);
    if (kHand)
      for (int j = tid; j < kScoreParts * kTopBins; j += 256) lhist[j] = 0;
    __syncthreads();
    float* out = a.scores + (int64_t)i * a.ld;

    auto entry_of = [&](int g) -> int64_t {   // entry 0 when the block is absent (scored -inf)
      g = min(g, end - 1);
      const int phys = tbl[(g >> pb_shift) - lb0];
      return phys >= 0 ? ((int64_t)phys << pb_shift) + (g & (per_block - 1)) : 0;
    };
    // tile m of this wave: keys base + 32*wave + 128*m + [0, 32)
    const int first = base + 32 * wave;
    const int n_mine = first < end ? (end - first + 127) / 128 : 0;
    struct Regs {
      u32x4 v[kLoads];
      uint32_t sc;
    };
    auto load = [&](Regs& r, int m) {
      const int tb = first + 128 * m;   // wave-uniform
      if constexpr (kTile) {
        // the 32-key tile lies in one block; tiles past the end re-read the last tile's block
        // (in bounds, unused). The tile's base address is wave-uniform (scalar registers) and
        // each lane adds its fixed offset, so the loads need no per-lane address arithmetic.
        const int gb = min(tb, (end - 1) & ~31);
        const int phys = __builtin_amdgcn_readfirstlane(tbl[(gb >> pb_shift) - lb0]);
        const int64_t e0 = (phys >= 0 ? ((int64_t)phys << pb_shift) : 0) + (gb & (per_block - 1));
        const uint8_t* kb = a.pool.data + e0 * kRow;
        // every key is read once per query: nontemporal loads stream past the caches (a
        // row-gather probe measured them 11-15 % faster than plain loads)
#pragma unroll
        for (int j = 0; j < kLoads; ++j)
          r.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + lane_off + j * (kFp4 ? 16 : 4) * kRow));
        if constexpr (kFp4) r.sc = (reinterpret_cast<const uint32_t*>(a.pool.scale) + e0)[lane & 31];
      } else {
#pragma unroll
        for (int j = 0; j < kLoads; ++j) {
          const int n = (kFp4 ? 16 : 4) * j + nk;
          r.v[j] = __builtin_nontemporal_load(
              reinterpret_cast<const u32x4*>(a.pool.data + entry_of(tb + n) * kRow + 16 * ck));
        }
        if constexpr (kFp4) r.sc = reinterpret_cast<const uint32_t*>(a.pool.scale)[entry_of(tb + (lane & 31))];
      }
    };
    auto publish = [&](const Regs& r) {
#pragma unroll
      for (int j = 0; j < kLoads; ++j) {
        const int n = (kFp4 ? 16 : 4) * j + nk;
        const int c = kFp4 ? (ck ^ ((n >> 1) & 3)) : (ck ^ (n & 15));
        *reinterpret_cast<u32x4*>(st + n * KF::kRowBytes + 16 * c) = r.v[j];
      }
      if constexpr (kFp4) {
        if (lane < 32) *reinterpret_cast<uint32_t*>(st + 2048 + 4 * lane) = r.sc;
      }
    };
    auto score = [&](int m) {
      f32x16 acc0 = {}, acc1 = {};
      if constexpr (!kFp4) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 b = __builtin_bit_cast(bf16x8, rd16(s));
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], b, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], b, acc1, 0, 0, 0);
        }
      } else {
        const u32x4 w0 = rd16(0);
        const u32x4 w1 = rd16(1);
        const uint32_t scb = *reinterpret_cast<const uint32_t*>(st + 2048 + 4 * col) >> (16 * hf);
        const float s0 = e8m0_to_f32(scb & 0xffu), s1 = e8m0_to_f32((scb >> 8) & 0xffu);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 b = s < 4 ? fp4x8_to_bf16x8(w0[s], s0) : fp4x8_to_bf16x8(w1[s - 4], s1);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], b, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], b, acc1, 0, 0, 0);
        }
      }
      float part = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        part = fmaf(wv[0][r], relu(acc0[r]), part);
        part = fmaf(wv[1][r], relu(acc1[r]), part);
      }
      part += __shfl_xor(part, 32, 64);
      const int g = first + 128 * m + col;
      if (hf == 0 && g < end) {
        const bool valid = tbl[(g >> pb_shift) - lb0] >= 0;
        const float v = valid ? canonical_zero(part) : -INFINITY;
        if constexpr (kHand) {
          const uint32_t key = order_key(v);
          lkeys[g - base] = key;
          atomicAdd(&lhist[((g - base) / kScorePartKeys) * kTopBins + (key >> (32 - kTopBits))], 1u);
        } else {
          out[g] = v;
        }
      }
    };
    if (n_mine > 0) {
      // kDepth tiles in flight in registers while one is staged and multiplied (a count that is
      // not a multiple of kDepth runs tiles of clamped rows, whose keys score() drops)
      Regs r[kDepth];
#pragma unroll
      for (int d = 0; d < kDepth; ++d) {
        load(r[d], d);
        // keep the tiles' loads in tile order: loads return in order, so the tile loop's waits
        // count only the tiles behind the one it stages (reordered, it would wait for all)
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int m = 0; m < n_mine; m += kDepth) {
#pragma unroll
        for (int d = 0; d < kDepth; ++d) {
          publish(r[d]);
          load(r[d], m + d + kDepth);
          score(m + d);
        }
      }
    }
    if constexpr (kHand)
      finish_parts<kScoreParts>(a, i, base / kScorePartKeys, base, end, lkeys, lhist, wtot);
  }
}

// Prefill form, bf16 keys: four query tokens per workgroup, one per wave, share every key tile.
// Queries of one sequence see the same keys, so a tile streamed once into LDS serves all of them:
// the key traffic of a prefill chunk drops fourfold and the kernel becomes MFMA-bound. The waves'
// queries are grouped by sequence (consecutive queries of a chunk usually share one): each group
// streams the keys up to its longest visible range, the four waves loading a quarter of each
// tile (two direct loads of four keys each) into a ring of kMStages shared tiles; after a barrier
// every wave whose query is in the group scores the tile. Each query's keys and histograms then go
// through the same hand-off (or plain scores) as in the one-query kernels.
constexpr int kMQ = 4;                       // queries per workgroup (one per wave)
constexpr int kMKeys = kScorePartKeys;       // keys per workgroup: one hand-off part
constexpr int kMParts = kMKeys / kScorePartKeys;
constexpr int kMStages = 3;                  // shared 8 KB tiles in the ring (two in flight)
// LDS: ring 24 KB + per query 1024 keys (16 KB for four queries) and 1024 16-bit bin counts
// packed two to a word (8 KB) + block table: about 50 KB, so that three workgroups (three waves
// per SIMD) share a compute unit and one's barriers, operand reads and hand-off overlap the
// others' MFMA work.
// Launches with explicit sequence ids and at least this many queries take the shared-tile kernel.
// A workgroup whose four queries belong to different sequences streams each sequence's keys in
// turn, which is only cheap when most workgroups hold one sequence and the grid is large; a decode
// batch (one or a few queries per sequence) keeps the one-query kernel.
constexpr int kMultiMinQueries = 256;

__global__ __launch_bounds__(256, 3) void score_mfma_multi(ScoreArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage[kMStages][8192];
  __shared__ uint32_t lhist[kMQ][kMParts * kTopBins / 2];   // counts <= 1024: 16 bits each
  __shared__ uint32_t lkeys[kMQ][kMKeys];
  __shared__ int32_t tbl[kMKeys / 2 + 2];
  __shared__ uint32_t wtot[kMParts * 4];
  __shared__ int32_t gseq[kMQ], gnv[kMQ];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hf = lane >> 5;
  const int base = blockIdx.x * kMKeys;
  const int i = blockIdx.y * kMQ + wave;   // this wave's query
  const bool has_q = i < a.n_q;
  const int iq = min(i, a.n_q - 1);        // in-bounds row for the loads of an absent query
  const int seq = a.qd.q_seq ? a.qd.q_seq[iq] : iq;
  const int p = a.qd.q_pos[iq];
  const int nv = has_q ? min(n_visible(p, a.pool.ratio, a.window),
                             n_visible(a.max_pos, a.pool.ratio, a.window)) : 0;
  const int end_w = min(nv, base + kMKeys);   // this wave's keys: [base, end_w)
  if (lane == 0) {
    gseq[wave] = has_q ? seq : -1;
    gnv[wave] = nv;
  }
  if (a.part_hist)
    for (int j = tid; j < kMQ * kMParts * kTopBins / 2; j += 256) (&lhist[0][0])[j] = 0;

  // this wave's query and head weights (as in score_mfma_dma)
  bf16x8 qa[2][8];
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)iq * kMfmaHeads * kMfmaDim;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qa[mb][s] = *reinterpret_cast<const bf16x8*>(q + (32 * mb + col) * kMfmaDim + 64 * hf + 8 * s);
  float wv[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wv[mb][r] = a.w[(int64_t)iq * kMfmaHeads + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3)];
  __syncthreads();   // gseq / gnv / histograms ready

  const int per_block = a.pool.per_block;   // 256 / ratio: a power of two
  const int pb_shift = __builtin_ctz(per_block);
  const int lb0 = base >> pb_shift;
  const uint32_t st0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&stage[0][0]);
  uint32_t roff[8];   // operand read offsets within a tile: key col, chunk (8hf + s) ^ (col % 16)
#pragma unroll
  for (int s = 0; s < 8; ++s) roff[s] = col * 256 + 16 * ((8 * hf + s) ^ (col & 15));

  for (int w0 = 0; w0 < kMQ; ++w0) {
    const int sq = gseq[w0];
    bool lead = sq >= 0;   // w0 is the first wave of its sequence
    int nv_s = 0;
    for (int w1 = 0; w1 < kMQ; ++w1) {
      if (gseq[w1] != sq) continue;
      if (w1 < w0) lead = false;
      nv_s = max(nv_s, gnv[w1]);
    }
    const int end_s = min(nv_s, base + kMKeys);
    if (!lead || base >= end_s) continue;   // uniform
    const bool mine = has_q && seq == sq;   // uniform per wave
    __syncthreads();   // the previous group's readers of tbl and of the tiles are done
    const int n_lb = ((end_s - 1) >> pb_shift) - lb0 + 1;
    for (int j = tid; j < n_lb; j += 256) {
      const int lb = lb0 + j;
      const int phys = lb < a.pool.max_blocks ? a.pool.block_table[(int64_t)sq * a.pool.max_blocks + lb] : -1;
      note_bad_page(a.pool, phys);
      tbl[j] = (phys >= 0 && phys < a.pool.num_blocks) ? phys : -1;
    }
    __syncthreads();
    const int n_tiles = (end_s - base + 31) / 32;
    // tile t into stage t % kMStages: this wave moves keys 8 wave .. 8 wave + 7 (two loads of
    // four keys); keys past the group's range re-read its last key (in bounds, unused)
    auto issue = [&](int t) {
      const int tb = base + 32 * t;
      const uint32_t lds = st0 + (t % kMStages) * 8192;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = 8 * wave + 4 * j + (lane >> 4);
        const int g = min(tb + n, end_s - 1);
        const int phys = tbl[(g >> pb_shift) - lb0];
        const int64_t e = phys >= 0 ? ((int64_t)phys << pb_shift) + (g & (per_block - 1)) : 0;
        const int c = (lane & 15) ^ (n & 15);
        lds_dma16(a.pool.data + e * a.pool.entry_bytes + 16 * c, lds + 1024 * (2 * wave + j));
      }
    };
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // tbl reads of the address math above
#pragma unroll
    for (int t = 0; t < kMStages - 1; ++t) issue(t);
    for (int t = 0; t < n_tiles; ++t) {
      wait_vmcnt<2 * (kMStages - 2)>();   // this wave's loads of tile t are done
      __syncthreads();                    // everyone's are, and tile t - 1 has been read
      issue(t + kMStages - 1);
      if (mine) {
        const uint8_t* sb = &stage[t % kMStages][0];
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(sb + roff[s]);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], b, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], b, acc1, 0, 0, 0);
        }
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          part = fmaf(wv[0][r], relu(acc0[r]), part);
          part = fmaf(wv[1][r], relu(acc1[r]), part);
        }
        part += __shfl_xor(part, 32, 64);
        const int g = base + 32 * t + col;
        if (hf == 0 && g < end_w) {
          const bool valid = tbl[(g >> pb_shift) - lb0] >= 0;
          const float v = valid ? canonical_zero(part) : -INFINITY;
          if (a.part_hist) {
            const uint32_t key = order_key(v);
            lkeys[wave][g - base] = key;
            const uint32_t bin = key >> (32 - kTopBits);   // one part per workgroup
            atomicAdd(&lhist[wave][bin >> 1], 1u << (16 * (bin & 1u)));
          } else {
            a.scores[(int64_t)i * a.ld + g] = v;
          }
        }
      }
    }
    wait_vmcnt<0>();   // no load may still be writing a tile when the ring is reused
  }
  if (a.part_hist && has_q && base < end_w) {
    // each wave hands off its own query's part (its keys and counts are its own LDS writes)
    finish_part_wave(a, i, blockIdx.x, base, end_w, lkeys[wave], lhist[wave], lane);
  }
}

// One thread per key (workgroups of kScorePartKeys keys, four per thread); query rows and weights
// staged in LDS as float.
__global__ __launch_bounds__(256) void score_generic(ScoreArgs a) {
  extern __shared__ float sm[];
  __shared__ uint32_t lhist[kTopBins];
  __shared__ uint32_t lkeys[kScorePartKeys];
  __shared__ uint32_t wtot[4];
  const int i = blockIdx.y;
  int seq, p;
  query_at(a.qd, i, &seq, &p);
  const int nv = min(n_visible(p, a.pool.ratio, a.window), n_visible(a.max_pos, a.pool.ratio, a.window));
  const int base = blockIdx.x * kScorePartKeys;
  if (base >= nv) return;
  const int H = a.n_heads, Dk = a.pool.dim;
  float* qs = sm;
  float* ws = sm + H * Dk;
  for (int e = threadIdx.x; e < H * Dk; e += 256) {
    int64_t off = (int64_t)i * H * Dk + e;
    qs[e] = a.q_dtype == F32 ? reinterpret_cast<const float*>(a.q)[off]
                             : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[off]);
  }
  for (int h = threadIdx.x; h < H; h += 256) ws[h] = a.w[(int64_t)i * H + h];
  if (a.part_hist)
    for (int j = threadIdx.x; j < kTopBins; j += 256) lhist[j] = 0;
  __syncthreads();
  for (int r = 0; r < kScorePartKeys / 256; ++r) {
    const int g = base + threadIdx.x + 256 * r;
    if (g >= nv) break;
    const int64_t idx = entry_index(a.pool, seq, g);
    float v = -INFINITY;
    if (idx >= 0) {
      const uint8_t* row = a.pool.data + idx * a.pool.entry_bytes;
      float total = 0.f;
      for (int h = 0; h < H; ++h) {
        float dot = 0.f;
        for (int d = 0; d < Dk; ++d) {
          float kd;
          if (a.pool.dtype == F32) {
            kd = reinterpret_cast<const float*>(row)[d];
          } else if (a.pool.dtype == BF16) {
            kd = bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[d]);
          } else {
            uint32_t byte = row[d >> 1];
            uint32_t nib = (d & 1) ? (byte >> 4) : (byte & 0xfu);
            const uint8_t* scl = reinterpret_cast<const uint8_t*>(a.pool.scale) + idx * (Dk / 32);
            kd = fp4_to_f32(nib) * e8m0_to_f32(scl[d >> 5]);
          }
          dot = fmaf(qs[h * Dk + d], kd, dot);
        }
        total = fmaf(ws[h], fmaxf(dot, 0.f), total);
      }
      v = canonical_zero(total);
    }
    if (a.part_hist) {
      const uint32_t key = order_key(v);
      lkeys[g - base] = key;
      atomicAdd(&lhist[key >> (32 - kTopBits)], 1u);
    } else {
      a.scores[(int64_t)i * a.ld + g] = v;
    }
  }
  if (a.part_hist)
    finish_parts<1>(a, i, blockIdx.x, base, min(nv, base + kScorePartKeys), lkeys, lhist, wtot);
}

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t s, const SideWork* side) {
  const int max_nv = (a.max_pos - a.window + 1 > 0)
                         ? (a.max_pos - a.window + 1 + a.pool.ratio - 1) / a.pool.ratio
                         : 0;
  SideWork none{};
  const SideWork& sw = side ? *side : none;
  const int n_side = sw.n[0] + sw.n[1] + sw.n_prep;
  if (n_side > 0 && (max_nv == 0 || a.n_q == 0 || (a.pool.dtype != BF16 && a.pool.dtype != FP4) || a.n_heads != kMfmaHeads ||
                     a.pool.dim != kMfmaDim || a.q_dtype != BF16 || (a.qd.q_seq && a.n_q >= kMultiMinQueries)))
    return hipErrorInvalidValue;   // the caller offers side work only to the one-query bf16 kernel
  if (max_nv == 0 || a.n_q == 0) return hipSuccess;
  const bool mfma = a.n_heads == kMfmaHeads && a.pool.dim == kMfmaDim && a.q_dtype == BF16 &&
                    (a.pool.dtype == BF16 || a.pool.dtype == FP4);
  if (mfma) {
    dim3 grid((max_nv + kScoreKeysPerBlock - 1) / kScoreKeysPerBlock, a.n_q);
    if (a.pool.dtype == BF16 && a.qd.q_seq && a.n_q >= kMultiMinQueries) {
      // a prefill chunk: runs of queries of one sequence share the key stream, kMQ per workgroup
      grid.x = (max_nv + kMKeys - 1) / kMKeys;
      grid.y = (a.n_q + kMQ - 1) / kMQ;
      hipLaunchKernelGGL(score_mfma_multi, grid, dim3(256), 0, s, a);
    } else {
      // one-query kernel over the item list: two workgroups per compute unit (registers and LDS
      // allow two), fewer when the items fit
      const int items = grid.x * grid.y;
      const dim3 g1(n_side + (items < kIndexWorkgroups ? items : kIndexWorkgroups));
      const bool tile = a.pool.per_block >= 32, hand = a.part_hist != nullptr;
#define HYB_SCORE_REG(T, H, F) \
  hipLaunchKernelGGL((score_mfma_reg<T, H, F>), g1, dim3(256), 0, s, a, sw.c[0], sw.c[1], sw.n[0], sw.n[1], \
                     sw.prep, sw.n_prep, sw.prep_gx)
      if (a.pool.dtype == BF16) {
        if (tile && hand) HYB_SCORE_REG(true, true, false);
        else if (tile) HYB_SCORE_REG(true, false, false);
        else if (hand) HYB_SCORE_REG(false, true, false);
        else HYB_SCORE_REG(false, false, false);
      } else {
        if (tile && hand) HYB_SCORE_REG(true, true, true);
        else if (tile) HYB_SCORE_REG(true, false, true);
        else if (hand) HYB_SCORE_REG(false, true, true);
        else HYB_SCORE_REG(false, false, true);
      }
#undef HYB_SCORE_REG
    }
  } else {
    dim3 grid((max_nv + kScorePartKeys - 1) / kScorePartKeys, a.n_q);
    size_t lds = sizeof(float) * ((size_t)a.n_heads * a.pool.dim + a.n_heads);
    hipLaunchKernelGGL(score_generic, grid, dim3(256), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace hyb
