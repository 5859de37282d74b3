// Exact top-k per row: the first min(k, n) indices under (score descending, index ascending), with
// -0.0 equal to +0.0, written in ascending index order and padded with -1.
// Method: SGLang DeepSeek-V4 day-0 blog, section "Shadow Radix" (C4 layers keep the top-512
// compressed entries chosen by the indexer); vLLM day-0 post ("DeepSeek Sparse Attention over
// compressed tokens").
//
// One 1024-thread workgroup per row. Scores become order-preserving 32-bit keys held in
// registers (32 consecutive scores per thread). Three radix passes (10 + 11 + 11 bits, histograms
// in LDS) find the k-th largest key T and how many of the keys equal to T are taken (the
// lowest-indexed ones). The first pass either comes from the indexer (per-workgroup partial
// histograms written while it scored the row, which then holds order keys) or is counted here.
// Because every thread owns a contiguous index range, one workgroup scan of its "> T" and "== T"
// counts gives each chosen index its output slot directly - the output is ascending without a sort.
//
// Short list: after the first pass only keys whose top 10 bits are >= b0 (those of the k-th key)
// can be chosen. When they number at most kListCap (the common case: the keys above bin b0 plus
// those in it), they are compacted with their indices into LDS in index order and the other two
// passes and the final selection run over that list instead of over every key of the row.
#include "common.h"
#include "select_dev.h"

namespace hyb {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Exclusive scan of a 32-bit value over the workgroup (thread order); also returns the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot,
                                                         uint32_t* total_out) {
  return block_scan_excl<kTopkThreads>(v, wave_tot, total_out);
}

// Each thread owns kPer consecutive scores of a chunk of kChunk, held in registers as keys. A
// chunk is fetched with coalesced 16-byte loads and redistributed through LDS (row pitch padded
// to 36 words so the per-thread reads do not collide in banks); rows longer than one chunk are
// re-read chunk by chunk in every pass.
constexpr int kPer = 32;
constexpr int kChunk = kTopkThreads * kPer;
constexpr int kStagePitch = kPer + 4;  // words per thread's slice in the staging area

// Dynamic LDS: staging [kTopkThreads][kStagePitch] words (reused for the per-wave histograms of a
// counted first pass, kTopkWaves x kTopWords, and for the short list), then the histogram.
constexpr int kTopWords = kTopBins + kTopBins / 32;   // padded first-pass histogram
constexpr size_t kTopkLds = sizeof(uint32_t) * ((size_t)kTopkThreads * kStagePitch + kHistWords);
static_assert(kTopkWaves * kTopWords <= kTopkThreads * kStagePitch, "per-wave histograms fit");
static_assert(kTopBins == kTopkThreads, "the counted first pass merges one bin per thread");
constexpr int kListCap = 16384;   // short-list entries: keys then indices in the staging area
static_assert(2 * kListCap <= kTopkThreads * kStagePitch, "short list fits the staging area");

// Row length of query i.
__device__ __forceinline__ int topk_row_len(const TopkArgs& a, int i) {
  int n;
  if (a.lengths) {
    n = a.lengths[i];
  } else {
    int seq, p;
    query_at(a.qd, i, &seq, &p);
    n = n_visible(p, a.ratio, a.window);
  }
  return max(0, min(n, a.max_len));
}

// kMulti: rows may exceed one chunk (launched when max_len > kChunk); the single-chunk form keeps
// the row in registers from the start and needs far fewer registers.
template <bool kMulti>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t tk_lds[];
  uint32_t* stage = tk_lds;
  uint32_t* hist = tk_lds + kTopkThreads * kStagePitch;
  __shared__ uint32_t wave_tot[kTopkWaves];
  __shared__ uint32_t sel_res[2];

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = topk_row_len(a, i);
  const int k = a.k;
  int* out = a.out + (int64_t)i * k;
  if (n <= k) {
    for (int j = tid; j < k; j += kTopkThreads) out[j] = j < n ? j : -1;
    return;
  }
  const float* sc = a.scores + (int64_t)i * a.ld;
  const bool keys_in = a.part_hist != nullptr;   // the indexer stored order keys
  const bool aligned16 = ((reinterpret_cast<uintptr_t>(sc) & 15u) == 0);
  const int n_chunks = kMulti ? (n + kChunk - 1) / kChunk : 1;

  // First-pass histogram from the indexer's partials (kTopBins uint16 bins = 512 words each):
  // thread t reads word t % 512 (bins 2w, 2w+1) of partials t / 512 + 2j. The loads of the
  // first kPartsInFlight partials are issued before the row's own loads (clamped, not branched)
  // and consumed after them, so both are in flight together.
  constexpr int kPartWords = kTopBins / 2;
  constexpr int kPartGroups = kTopkThreads / kPartWords;            // 2
  constexpr int kPartsInFlight = kChunk / kScorePartKeys;            // 32
  constexpr int kPartLoads = kPartsInFlight / kPartGroups;           // 16 per thread
  const int nb = keys_in ? (n + kScorePartKeys - 1) / kScorePartKeys : 0;
  const int pwd = tid % kPartWords, pg = tid / kPartWords;
  const uint32_t* ph =
      keys_in ? reinterpret_cast<const uint32_t*>(a.part_hist + (int64_t)i * a.part_ld * kTopBins) + pwd
              : nullptr;
  uint32_t pw[kPartLoads];
  if (keys_in) {
#pragma unroll
    for (int q = 0; q < kPartLoads; ++q)
      pw[q] = ph[(int64_t)min(pg + kPartGroups * q, nb - 1) * kPartWords];
  }
  for (int j = tid; j < kHistWords; j += kTopkThreads) hist[j] = 0;   // before the first pass

  // Row loads never branch per lane (a branch between a load and its use makes the compiler wait
  // for every load in flight): 16-byte loads from addresses clamped into the row's ld, or, for
  // unaligned rows, 4-byte loads clamped into [0, n); elements past n are masked to key 0.
  const bool vec_ok = aligned16 && (a.ld & 3) == 0 && a.ld >= 4;
  const int vec_last = (int)min<int64_t>(a.ld - 4, INT32_MAX - 4);
  uint32_t u[kPer];
  auto load_chunk = [&](int c) {
    const int base = c * kChunk;
    __syncthreads();  // the staging area may still hold histograms or the previous chunk
    // coalesced: thread t moves elements base + 4*(t + 1024*q) .. +3 for q = 0..7
    u32x4 v[kPer / 4];
    if (vec_ok) {
#pragma unroll
      for (int q = 0; q < kPer / 4; ++q) {
        const int j = base + 4 * (tid + kTopkThreads * q);
        const f32x4 f = *reinterpret_cast<const f32x4*>(sc + min(j, vec_last));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t key = keys_in ? __float_as_uint(f[e]) : order_key(f[e]);
          v[q][e] = j + e < n ? key : 0u;
        }
      }
    } else {
#pragma unroll
      for (int q = 0; q < kPer / 4; ++q) {
        const int j = base + 4 * (tid + kTopkThreads * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float f = sc[min(j + e, n - 1)];
          const uint32_t key = keys_in ? __float_as_uint(f) : order_key(f);
          v[q][e] = j + e < n ? key : 0u;
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const int jj = 4 * (tid + kTopkThreads * q);  // owner thread jj / 32, slot jj % 32
      *reinterpret_cast<u32x4*>(stage + (jj / kPer) * kStagePitch + (jj % kPer)) = v[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + tid * kStagePitch + 4 * q);
      u[4 * q] = v[0];
      u[4 * q + 1] = v[1];
      u[4 * q + 2] = v[2];
      u[4 * q + 3] = v[3];
    }
  };
  // bit e set <=> element e of this thread's slice of chunk c lies inside the row
  auto valid_mask = [&](int c) {
    const int cnt = n - (c * kChunk + tid * kPer);
    return cnt >= kPer ? 0xffffffffu : (cnt <= 0 ? 0u : (1u << cnt) - 1u);
  };
  // bit e set <=> element e is inside the row and its key matches the prefix
  auto match_mask = [&](uint32_t valid, uint32_t pmask, uint32_t prefix) {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) m |= (uint32_t)((u[e] & pmask) == prefix) << e;
    return m & valid;
  };
  if (!kMulti || n_chunks == 1) load_chunk(0);

  // ---- first pass (top kTopBits bits)
  if (keys_in) {
    uint32_t h0 = 0, h1 = 0;
#pragma unroll
    for (int q = 0; q < kPartLoads; ++q) {
      const uint32_t on = pg + kPartGroups * q < nb ? 0xffffffffu : 0u;
      h0 += pw[q] & 0xffffu & on;
      h1 += (pw[q] >> 16) & on;
    }
    for (int b = pg + kPartsInFlight; b < nb; b += kPartGroups) {   // rows longer than one chunk
      const uint32_t w = ph[(int64_t)b * kPartWords];
      h0 += w & 0xffffu;
      h1 += w >> 16;
    }
    if (kMulti && n_chunks > 1) __syncthreads();   // no staging barrier since the clearing
    atomicAdd(&hist[hp(2 * pwd)], h0);
    atomicAdd(&hist[hp(2 * pwd + 1)], h1);
    __syncthreads();
  } else {
    // counted into per-wave histograms (the busiest bins would otherwise serialise atomics of all
    // waves) laid over the staging area, once its data is in registers
    const bool private_hist = n_chunks == 1;
    uint32_t* h = private_hist ? stage + wave * kTopWords : hist;
    __syncthreads();
    if (private_hist) {
      for (int j = lane; j < kTopWords; j += 64) h[j] = 0;
    }
    __syncthreads();
#pragma unroll 1
    for (int c = 0; c < n_chunks; ++c) {
      if (kMulti && n_chunks > 1) load_chunk(c);
      const uint32_t m = valid_mask(c);
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if ((m >> e) & 1u) atomicAdd(&h[hp(u[e] >> kShift0)], 1u);
    }
    __syncthreads();
    if (private_hist) {
      const int j = hp(tid);   // kTopBins == kTopkThreads: one bin per thread
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) t += stage[w * kTopWords + j];
      hist[j] = t;
      __syncthreads();
    }
  }
  uint32_t b0, above0;
  select_bin(hist, kTopBins, (uint32_t)k, sel_res, &b0, &above0);
  uint32_t prefix = b0 << kShift0, pmask = ~0u << kShift0;
  uint32_t remaining = (uint32_t)k - above0;   // still to take among keys matching the prefix

  // ---- short list (single chunk): keys whose top bits are >= b0, with their indices, into LDS
  if (!kMulti) {
    const uint32_t lo = prefix;
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) m |= (uint32_t)(u[e] >= lo) << e;
    m &= valid_mask(0);
    uint32_t total = 0;
    // (its barriers also order every staging read before the list overwrites the staging area)
    const uint32_t o = block_exclusive_scan(__builtin_popcount(m), wave_tot, &total);
    if (total <= (uint32_t)kListCap) {
      uint32_t* lkey = stage;
      int32_t* lidx = reinterpret_cast<int32_t*>(stage + kListCap);
      // element e goes to slot o + (number of kept elements before e): no data-dependent loop
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        if ((m >> e) & 1u) {
          const uint32_t slot = o + __builtin_popcount(m & ((1u << e) - 1u));
          lkey[slot] = u[e];
          lidx[slot] = tid * kPer + e;
        }
      }
#pragma unroll 1
      for (int shift = kBits12; shift >= 0; shift -= kBits12) {
        for (int j = tid; j < kHistWords; j += kTopkThreads) hist[j] = 0;
        __syncthreads();   // list written (first time), histogram cleared
        for (int j = tid; j < (int)total; j += kTopkThreads) {
          const uint32_t key = lkey[j];
          if ((key & pmask) == prefix) atomicAdd(&hist[hp((key >> shift) & 2047u)], 1u);
        }
        __syncthreads();
        uint32_t b, ab;
        select_bin(hist, 2048, remaining, sel_res, &b, &ab);
        prefix |= b << shift;
        pmask |= 2047u << shift;
        remaining -= ab;
      }
      const uint32_t T = prefix;   // the k-th largest key; `remaining` keys equal to it are taken
      // thread t owns list positions [j0, j1), in index order
      const int C = ((int)total + kTopkThreads - 1) / kTopkThreads;
      const int j0 = min((int)total, tid * C), j1 = min((int)total, j0 + C);
      uint32_t gt = 0, tie = 0;
      for (int j = j0; j < j1; ++j) {
        gt += lkey[j] > T;
        tie += lkey[j] == T;
      }
      // counts <= kListCap < 2^16: both fit 16 bits of one word
      const uint32_t pre = block_exclusive_scan((tie << 16) | gt, wave_tot, nullptr);
      // signed clamps (ties still to take when this thread's keys begin may be negative)
      const int32_t left = (int32_t)remaining - (int32_t)(pre >> 16);
      uint32_t pos = (pre & 0xffffu) + (uint32_t)((int32_t)remaining - max(left, 0));
      int32_t tseen = 0;
      for (int j = j0; j < j1; ++j) {
        const uint32_t key = lkey[j];
        bool take = key > T;
        if (key == T) {
          take = tseen < left;
          ++tseen;
        }
        if (take) {
          if (pos < (uint32_t)k) out[pos] = lidx[j];
          ++pos;
        }
      }
      return;
    }
  }

  // ---- general form: the other two passes over every key of the row
#pragma unroll 1
  for (int shift = kBits12; shift >= 0; shift -= kBits12) {
    for (int j = tid; j < kHistWords; j += kTopkThreads) hist[j] = 0;
    __syncthreads();
#pragma unroll 1
    for (int c = 0; c < n_chunks; ++c) {
      if (kMulti && n_chunks > 1) load_chunk(c);
      uint32_t m = match_mask(valid_mask(c), pmask, prefix);
      // later passes see few matching keys: visit only those
      while (m) {
        const int e = __builtin_ctz(m);
        m &= m - 1;
        uint32_t ue = 0;
#pragma unroll
        for (int q = 0; q < kPer; ++q) ue = q == e ? u[q] : ue;
        atomicAdd(&hist[hp((ue >> shift) & 2047u)], 1u);
      }
    }
    __syncthreads();
    uint32_t b, ab;
    select_bin(hist, 2048, remaining, sel_res, &b, &ab);
    prefix |= b << shift;
    pmask |= 2047u << shift;
    remaining -= ab;
  }
  const uint32_t T = prefix;  // key of the k-th largest score; `remaining` ties of it are taken

  uint32_t gt_base = 0, tie_base = 0;
#pragma unroll 1
  for (int c = 0; c < n_chunks; ++c) {
    if (kMulti && n_chunks > 1) load_chunk(c);
    const uint32_t valid = valid_mask(c);
    uint32_t gtm = 0, tiem = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      gtm |= (uint32_t)(u[e] > T) << e;
      tiem |= (uint32_t)(u[e] == T) << e;
    }
    gtm &= valid;
    tiem &= valid;
    const uint32_t gt = __builtin_popcount(gtm), tie = __builtin_popcount(tiem);
    // per-thread counts are <= 32, chunk totals <= 32768: both fit 16 bits of one word
    uint32_t tot = 0;
    const uint32_t pre = block_exclusive_scan((tie << 16) | gt, wave_tot, &tot);
    const uint32_t gt_pre = gt_base + (pre & 0xffffu);
    const uint32_t tie_pre = tie_base + (pre >> 16);
    // Ties are taken lowest index first: keep this thread's first `take` tie bits. `left` (ties
    // still to take when this thread's slice begins) may be negative, so it is signed, and both
    // clamps are explicit: written as `remaining > tie_pre ? min(remaining - tie_pre, tie) : 0`
    // with unsigned operands, the compiler hoisted the subtraction with a no-wrap flag and then
    // folded min(remaining, tie_pre) to tie_pre, shifting later slots when ties were left over.
    const int32_t left = (int32_t)remaining - (int32_t)tie_pre;
    const int32_t take = max(0, min(left, (int32_t)tie));
    uint32_t keep = 0, tm = tiem;
    for (int32_t t = 0; t < take; ++t) {
      keep |= tm & (0u - tm);
      tm &= tm - 1;
    }
    uint32_t sel = gtm | keep;
    // slot of this slice's first chosen key: keys > T before it plus min(remaining, tie_pre)
    uint32_t pos = gt_pre + (uint32_t)((int32_t)remaining - max(left, 0));
    const int base = c * kChunk + tid * kPer;
    while (sel) {
      const int e = __builtin_ctz(sel);
      sel &= sel - 1;
      if (pos < (uint32_t)k) out[pos] = base + e;
      ++pos;
    }
    gt_base += tot & 0xffffu;
    tie_base += tot >> 16;
  }
}

// ------------------------------------------------------------------------------------------
// Single-chunk rows (n <= kChunk): thread t owns the elements 4t + 4096q + e (q < 8, e < 4), i.e.
// the row is read with one coalesced 16-byte load per q and never redistributed. The row and the
// first-pass partials are requested before the row length is known (addresses are clamped into
// the row's ld and the partials' part_ld; the length only masks). The other two passes visit
// each thread's few elements that match the prefix so far. The output order comes from two
// 32768-bit maps (keys > T, keys == T): thread t takes word t of both, and one workgroup scan of
// the packed counts gives every chosen index its slot, lowest-index ties first.
// ------------------------------------------------------------------------------------------
constexpr int kShortUnion = kTopkWaves * kTopWords;   // per-wave first-pass histograms
constexpr int kMapWords = kChunk / 32;
constexpr size_t kShortLds = sizeof(uint32_t) * ((size_t)kShortUnion + kHistWords + 2 * kMapWords);

__global__ __launch_bounds__(kTopkThreads) void topk_short(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t ts_lds[];
  uint32_t* uni = ts_lds;                 // per-wave first-pass histograms
  uint32_t* hist = ts_lds + kShortUnion;
  uint32_t* gtmap = hist + kHistWords;
  uint32_t* tiemap = gtmap + kMapWords;
  __shared__ uint32_t wave_tot[kTopkWaves];
  __shared__ uint32_t sel_res[2];

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int k = a.k;
  const float* sc = a.scores + (int64_t)i * a.ld;
  const bool keys_in = a.part_hist != nullptr;
  const bool vec_ok = ((reinterpret_cast<uintptr_t>(sc) & 15u) == 0) && (a.ld & 3) == 0 && a.ld >= 4;
  const int64_t ld_last = a.ld - 1;

  // ---- loads, before the row length arrives
  f32x4 raw[kPer / 4];
  if (vec_ok) {
    const int vec_last = (int)min<int64_t>(a.ld - 4, INT32_MAX - 4);
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q)
      raw[q] = *reinterpret_cast<const f32x4*>(sc + min(4 * tid + kTopkThreads * 4 * q, vec_last));
  } else {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        raw[q][e] = sc[min<int64_t>(4 * tid + kTopkThreads * 4 * q + e, ld_last)];
  }
  constexpr int kPartWords = kTopBins / 2;
  constexpr int kPartGroups = kTopkThreads / kPartWords;            // 2
  constexpr int kPartLoads = (kChunk / kScorePartKeys) / kPartGroups;   // 16 per thread
  const int pwd = tid % kPartWords, pg = tid / kPartWords;
  uint32_t pw[kPartLoads];
  if (keys_in) {
    const uint32_t* ph = reinterpret_cast<const uint32_t*>(a.part_hist + (int64_t)i * a.part_ld * kTopBins) + pwd;
#pragma unroll
    for (int q = 0; q < kPartLoads; ++q)
      pw[q] = ph[(int64_t)min(pg + kPartGroups * q, a.part_ld - 1) * kPartWords];
  }
  for (int j = tid; j < kHistWords; j += kTopkThreads) hist[j] = 0;

  const int n = topk_row_len(a, i);
  int* out = a.out + (int64_t)i * k;
  if (n <= k) {   // uniform
    for (int j = tid; j < k; j += kTopkThreads) out[j] = j < n ? j : -1;
    return;
  }
  // element 4q + e of this thread is row index 4 tid + 4096 q + e
  uint32_t u[kPer];
  uint32_t valid = 0;
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = 4 * tid + kTopkThreads * 4 * q + e;
      const uint32_t key = keys_in ? __float_as_uint(raw[q][e]) : order_key(raw[q][e]);
      u[4 * q + e] = j < n ? key : 0u;
      valid |= (uint32_t)(j < n) << (4 * q + e);
    }
  auto index_of = [&](int e) { return 4 * tid + kTopkThreads * 4 * (e >> 2) + (e & 3); };

  // ---- first pass (top kTopBits bits)
  if (keys_in) {
    const int nb = (n + kScorePartKeys - 1) / kScorePartKeys;
    uint32_t h0 = 0, h1 = 0;
#pragma unroll
    for (int q = 0; q < kPartLoads; ++q) {
      const uint32_t on = pg + kPartGroups * q < nb ? 0xffffffffu : 0u;
      h0 += pw[q] & 0xffffu & on;
      h1 += (pw[q] >> 16) & on;
    }
    __syncthreads();   // histogram cleared
    atomicAdd(&hist[hp(2 * pwd)], h0);
    atomicAdd(&hist[hp(2 * pwd + 1)], h1);
    __syncthreads();
  } else {
    // per-wave histograms (the busiest bins would otherwise serialise the atomics of all waves)
    uint32_t* h = uni + wave * kTopWords;
    for (int j = lane; j < kTopWords; j += 64) h[j] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      if ((valid >> e) & 1u) atomicAdd(&h[hp(u[e] >> kShift0)], 1u);
    __syncthreads();
    const int j = hp(tid);   // kTopBins == kTopkThreads: one bin per thread
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) t += uni[w * kTopWords + j];
    hist[j] = t;
    __syncthreads();   // also: every read of the per-wave histograms precedes the short list
  }
  uint32_t b0, above0;
  select_bin(hist, kTopBins, (uint32_t)k, sel_res, &b0, &above0);
  uint32_t prefix = b0 << kShift0, pmask = ~0u << kShift0;
  uint32_t remaining = (uint32_t)k - above0;

  // ---- second and third passes (11 bits each) over the keys matching the prefix; after the
  // first pass they are few, so each thread visits only its matching elements
#pragma unroll 1
  for (int shift = kBits12; shift >= 0; shift -= kBits12) {
    for (int j = tid; j < kHistWords; j += kTopkThreads) hist[j] = 0;
    __syncthreads();
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) m |= (uint32_t)((u[e] & pmask) == prefix) << e;
    m &= valid;
    while (m) {
      const int e = __builtin_ctz(m);
      m &= m - 1;
      uint32_t ue = 0;
#pragma unroll
      for (int q = 0; q < kPer; ++q) ue = q == e ? u[q] : ue;
      atomicAdd(&hist[hp((ue >> shift) & 2047u)], 1u);
    }
    __syncthreads();
    uint32_t b, ab;
    select_bin(hist, 2048, remaining, sel_res, &b, &ab);
    prefix |= b << shift;
    pmask |= 2047u << shift;
    remaining -= ab;
  }
  const uint32_t T = prefix;   // the k-th largest key; `remaining` keys equal to it are taken

  // ---- index maps of the keys > T and == T. Element 4q + e of thread t is index
  // 4t + 4096q + e: map word t/8 + 128q, bits 4(t%8) + e. The eight threads of a word (consecutive
  // lanes) OR their nibbles together with row shifts, and the first of them stores the word.
  {
    uint32_t gtm = 0, tiem = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      gtm |= (uint32_t)(u[e] > T) << e;
      tiem |= (uint32_t)(u[e] == T) << e;
    }
    gtm &= valid;
    tiem &= valid;
    const int sh = 4 * (tid & 7);
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      uint32_t g = ((gtm >> (4 * q)) & 15u) << sh;
      uint32_t t = ((tiem >> (4 * q)) & 15u) << sh;
      // OR over lanes l..l+7 into lane l (l % 8 == 0): row_shl 1, 2, 4 (lanes past the row end
      // contribute 0; only the group's first lane is used)
      g |= __builtin_amdgcn_update_dpp(0u, g, 0x101, 0xf, 0xf, false);
      t |= __builtin_amdgcn_update_dpp(0u, t, 0x101, 0xf, 0xf, false);
      g |= __builtin_amdgcn_update_dpp(0u, g, 0x102, 0xf, 0xf, false);
      t |= __builtin_amdgcn_update_dpp(0u, t, 0x102, 0xf, 0xf, false);
      g |= __builtin_amdgcn_update_dpp(0u, g, 0x104, 0xf, 0xf, false);
      t |= __builtin_amdgcn_update_dpp(0u, t, 0x104, 0xf, 0xf, false);
      if ((tid & 7) == 0) {
        gtmap[(tid >> 3) + 128 * q] = g;
        tiemap[(tid >> 3) + 128 * q] = t;
      }
    }
  }
  __syncthreads();
  const uint32_t gtw = gtmap[tid], tiew = tiemap[tid];
  const uint32_t gt = __builtin_popcount(gtw), tie = __builtin_popcount(tiew);
  // counts <= 32768 in total: both fit 16 bits of one word
  const uint32_t pre = block_exclusive_scan((tie << 16) | gt, wave_tot, nullptr);
  // signed clamps (ties still to take when this word begins may be negative)
  const int32_t left = (int32_t)remaining - (int32_t)(pre >> 16);
  const int32_t take = max(0, min(left, (int32_t)tie));
  uint32_t keep = 0, tm = tiew;
  for (int32_t t = 0; t < take; ++t) {
    keep |= tm & (0u - tm);
    tm &= tm - 1;
  }
  uint32_t sel = gtw | keep;
  uint32_t pos = (pre & 0xffffu) + (uint32_t)((int32_t)remaining - max(left, 0));
  while (sel) {
    const int b = __builtin_ctz(sel);
    sel &= sel - 1;
    if (pos < (uint32_t)k) out[pos] = 32 * tid + b;
    ++pos;
  }
}

// ------------------------------------------------------------------------------------------
// Selection from the indexer's hand-off (TopkArgs::part_hist set): per part of kScorePartKeys
// keys, a cumulative histogram of the top kTopBits key bits (cum_p[b] = keys with top bits >= b)
// and the part's (key, index) pairs bucketed by those bits, highest bin first. One workgroup per
// row:
//   1. C[b] = sum_p cum_p[b]; the first-pass bin b0 is the one with C[b0] >= k > C[b0 + 1].
//   2. The candidates are the keys with top bits >= b0: the leading cum_p[b0] pairs of every
//      part. They are gathered into LDS (a few per thread); the first 64 pairs of the first 32
//      parts are requested together with the counts, before b0 is known, so the usual row costs
//      one global round trip.
//   3. Two 11-bit passes over the candidates whose top bits equal b0 find the k-th largest key T
//      and how many keys equal to T are taken (the lowest-indexed ones).
//   4. Output in ascending index order, 32768 indices at a time: bit maps of the chosen keys > T
//      and of the keys == T (word w = indices 32w..32w+31, one word per thread), one workgroup
//      scan of the packed counts, ties taken lowest index first.
// When the candidates exceed the LDS list (degenerate score distributions) they are read from
// the hand-off buffer in every step instead.
// ------------------------------------------------------------------------------------------
constexpr int kPairCap = 8192;         // candidates held in LDS
constexpr int kPairMaxParts = kTopkMaxParts;   // parts per row (rows of up to 4M entries)
constexpr int kPairLdsWords = kTopBins + kHistWords + 2 * (kPairMaxParts + 1) + 2 * kPairCap +
                              2 * kMapWords;
constexpr size_t kPairLds = sizeof(uint32_t) * (size_t)kPairLdsWords;

__global__ __launch_bounds__(kTopkThreads) void topk_pairs(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t tp_lds[];
  uint32_t* C = tp_lds;                         // [kTopBins] global cumulative counts
  uint32_t* hist = C + kTopBins;                // [kHistWords] padded 2048-bin histogram
  uint32_t* cnt = hist + kHistWords;            // [kPairMaxParts + 1] candidates per part
  uint32_t* off = cnt + kPairMaxParts + 1;      // [kPairMaxParts + 1] their offsets
  uint32_t* lkey = off + kPairMaxParts + 1;     // [kPairCap]
  uint32_t* lidx = lkey + kPairCap;             // [kPairCap]
  uint32_t* gtmap = lidx + kPairCap;            // [kMapWords]
  uint32_t* tiemap = gtmap + kMapWords;         // [kMapWords]
  __shared__ uint32_t wave_tot[kTopkWaves];
  __shared__ uint32_t sel_res[2];

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int k = a.k;
  const bool rowh = a.row_hist != nullptr;   // uniform
  // first 32 parts' cumulative counts, before the row length is known (clamped to part_ld) - or,
  // with the indexer's per-row counts, this thread's bin of the row
  constexpr int kPartWords = kTopBins / 2;
  constexpr int kPartGroups = kTopkThreads / kPartWords;            // 2
  constexpr int kPartLoads = 16;                                     // parts pg + 2q, q < 16
  const int pwd = tid % kPartWords, pg = tid / kPartWords;
  const uint32_t* ph = reinterpret_cast<const uint32_t*>(a.part_hist + (int64_t)i * a.part_ld * kTopBins);
  uint32_t pw[kPartLoads];
  uint32_t rcount = 0;
  if (rowh) {
    rcount = a.row_hist[(int64_t)i * kTopBins + (kTopBins - 1 - tid)];   // bin 1023 - tid
  } else {
#pragma unroll
    for (int q = 0; q < kPartLoads; ++q)
      pw[q] = ph[(int64_t)min(pg + kPartGroups * q, a.part_ld - 1) * kPartWords + pwd];
  }
  const uint2* pairs = reinterpret_cast<const uint2*>(a.scores) + (int64_t)i * (a.ld / 2);
  // (ext-vector pairs: a register array of HIP's union-based uint2 would stay in scratch)
  const int ep = tid >> 5, el = tid & 31;   // early part, lane: pairs el and el + 32
  u32x2 pre[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    pre[j] = *reinterpret_cast<const u32x2*>(pairs + (int64_t)min(ep, a.part_ld - 1) * kScorePartKeys + el + 32 * j);
  C[tid] = 0;
  const int n = topk_row_len(a, i);
  int* out = a.out + (int64_t)i * k;
  if (rowh) a.row_hist[(int64_t)i * kTopBins + (kTopBins - 1 - tid)] = 0u;   // zero for the next call
  if (n <= k) {   // uniform
    for (int j = tid; j < k; j += kTopkThreads) out[j] = j < n ? j : -1;
    return;
  }
  const int nb = (n + kScorePartKeys - 1) / kScorePartKeys;   // <= kPairMaxParts (host check)

  // ---- 1. global cumulative histogram and b0
  if (rowh) {
    // C[b] = the row's keys with top bits >= b: thread t holds bin 1023 - t, so the inclusive
    // scan over threads is C of its bin
    __syncthreads();   // C cleared
    const uint32_t incl = block_exclusive_scan(rcount, wave_tot, nullptr) + rcount;
    C[kTopBins - 1 - tid] = incl;
    __syncthreads();
  } else {
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int q = 0; q < kPartLoads; ++q) {
      const uint32_t on = pg + kPartGroups * q < nb ? 0xffffffffu : 0u;
      c0 += pw[q] & 0xffffu & on;
      c1 += (pw[q] >> 16) & on;
    }
    for (int p = pg + kPartGroups * kPartLoads; p < nb; p += kPartGroups) {   // rows past 32 parts
      const uint32_t w = ph[(int64_t)p * kPartWords + pwd];
      c0 += w & 0xffffu;
      c1 += w >> 16;
    }
    __syncthreads();   // C cleared
    atomicAdd(&C[2 * pwd], c0);
    atomicAdd(&C[2 * pwd + 1], c1);
    __syncthreads();
  }
  {
    // C is non-increasing in b and C[0] = n > k: exactly one bin satisfies this
    const uint32_t here = C[tid], next = tid + 1 < kTopBins ? C[tid + 1] : 0u;
    if (here >= (uint32_t)k && next < (uint32_t)k) {
      sel_res[0] = (uint32_t)tid;
      sel_res[1] = next;
    }
  }
  __syncthreads();
  const uint32_t b0 = sel_res[0], above0 = sel_res[1];

  // ---- 2. candidates per part: cum_p[b0]
  if (rowh) {
    for (int p = tid; p < nb; p += kTopkThreads)
      cnt[p] = a.part_hist[((int64_t)i * a.part_ld + p) * kTopBins + b0];
  } else {
    if (pwd == (int)(b0 >> 1)) {
#pragma unroll
      for (int q = 0; q < kPartLoads; ++q) {
        const int p = pg + kPartGroups * q;
        if (p < nb) cnt[p] = (b0 & 1u) ? (pw[q] >> 16) : (pw[q] & 0xffffu);
      }
    }
    for (int p = kPartGroups * kPartLoads + tid; p < nb; p += kTopkThreads)
      cnt[p] = a.part_hist[((int64_t)i * a.part_ld + p) * kTopBins + b0];
  }
  for (int j = tid; j < 2 * kMapWords; j += kTopkThreads) gtmap[j] = 0;
  __syncthreads();
  // exclusive scan of the counts over parts (four parts per thread)
  {
    uint32_t v[4], s = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 4 * tid + e;
      v[e] = p < nb ? cnt[p] : 0u;
      s += v[e];
    }
    uint32_t total = 0;
    uint32_t run = block_exclusive_scan(s, wave_tot, &total);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 4 * tid + e;
      if (p < nb) off[p] = run;
      run += v[e];
    }
    if (tid == 0) off[nb] = total;
  }
  __syncthreads();
  const uint32_t M = off[nb];
  const bool in_lds = M <= (uint32_t)kPairCap;   // uniform
  // candidate m: part p with off[p] <= m < off[p + 1], position m - off[p]
  auto fetch = [&](uint32_t m) -> uint2 {
    int lo = 0, hi = nb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= m) lo = mid; else hi = mid - 1;
    }
    return pairs[(int64_t)lo * kScorePartKeys + (m - off[lo])];
  };
  if (in_lds) {
    if (ep < nb) {
      const uint32_t cp = cnt[ep], op = off[ep];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t pos = el + 32 * j;
        if (pos < cp) {
          lkey[op + pos] = pre[j][0];
          lidx[op + pos] = pre[j][1];
        }
      }
      for (uint32_t pos = 64 + el; pos < cp; pos += 32) {   // long early parts
        const uint2 pr = pairs[(int64_t)ep * kScorePartKeys + pos];
        lkey[op + pos] = pr.x;
        lidx[op + pos] = pr.y;
      }
    }
    if (nb > 32) {
      for (uint32_t m = off[32] + tid; m < M; m += kTopkThreads) {
        const uint2 pr = fetch(m);
        lkey[m] = pr.x;
        lidx[m] = pr.y;
      }
    }
    __syncthreads();
  }
  auto cand = [&](uint32_t m) -> uint2 { return in_lds ? make_uint2(lkey[m], lidx[m]) : fetch(m); };

  // ---- 3. passes over the candidates of bin b0
  uint32_t prefix = b0 << kShift0, pmask = ~0u << kShift0;
  uint32_t remaining = (uint32_t)k - above0;
#pragma unroll 1
  for (int shift = kBits12; shift >= 0; shift -= kBits12) {
    for (int j = tid; j < kHistWords; j += kTopkThreads) hist[j] = 0;
    __syncthreads();
    for (uint32_t m = tid; m < M; m += kTopkThreads) {
      const uint32_t key = cand(m).x;
      if ((key & pmask) == prefix) atomicAdd(&hist[hp((key >> shift) & 2047u)], 1u);
    }
    __syncthreads();
    uint32_t b, ab;
    select_bin(hist, 2048, remaining, sel_res, &b, &ab);
    prefix |= b << shift;
    pmask |= 2047u << shift;
    remaining -= ab;
  }
  const uint32_t T = prefix;   // the k-th largest key; `remaining` keys equal to it are taken

  // ---- 4. output, 32768 indices at a time
  uint32_t gt_base = 0, tie_base = 0;
  const int n_chunks = (n + kChunk - 1) / kChunk;
#pragma unroll 1
  for (int c = 0; c < n_chunks; ++c) {
    const uint32_t lo = (uint32_t)c * kChunk;
    if (c > 0) {
      __syncthreads();   // the previous chunk's maps are read
      for (int j = tid; j < 2 * kMapWords; j += kTopkThreads) gtmap[j] = 0;
      __syncthreads();
    }
    for (uint32_t m = tid; m < M; m += kTopkThreads) {
      const uint2 pr = cand(m);
      const uint32_t j = pr.y - lo;
      if (j < (uint32_t)kChunk) {
        if (pr.x > T) atomicOr(&gtmap[j >> 5], 1u << (j & 31));
        else if (pr.x == T) atomicOr(&tiemap[j >> 5], 1u << (j & 31));
      }
    }
    __syncthreads();
    const uint32_t gtw = gtmap[tid], tiew = tiemap[tid];
    const uint32_t gt = __builtin_popcount(gtw), tie = __builtin_popcount(tiew);
    uint32_t tot = 0;
    // per-chunk counts <= 32768: both fit 16 bits of one word
    const uint32_t pre = block_exclusive_scan((tie << 16) | gt, wave_tot, &tot);
    const uint32_t gt_pre = gt_base + (pre & 0xffffu);
    const uint32_t tie_pre = tie_base + (pre >> 16);
    // signed clamps (ties still to take when this word begins may be negative)
    const int32_t left = (int32_t)remaining - (int32_t)tie_pre;
    const int32_t take = max(0, min(left, (int32_t)tie));
    uint32_t keep = 0, tm = tiew;
    for (int32_t t = 0; t < take; ++t) {
      keep |= tm & (0u - tm);
      tm &= tm - 1;
    }
    uint32_t sel = gtw | keep;
    uint32_t pos = gt_pre + (uint32_t)((int32_t)remaining - max(left, 0));
    while (sel) {
      const int b = __builtin_ctz(sel);
      sel &= sel - 1;
      if (pos < (uint32_t)k) out[pos] = (int)(lo + 32 * tid + b);
      ++pos;
    }
    gt_base += tot & 0xffffu;
    tie_base += tot >> 16;
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  static bool attr_set = false;   // the dynamic LDS above 64 KiB must be enabled once per kernel
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_kernel<true>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTopkLds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_short),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kShortLds);
    if (e == hipSuccess)
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(topk_pairs),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)kPairLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  if (a.part_hist)
    hipLaunchKernelGGL(topk_pairs, dim3(a.n_q), dim3(kTopkThreads), kPairLds, s, a);
  else if (a.max_len <= kChunk)
    hipLaunchKernelGGL(topk_short, dim3(a.n_q), dim3(kTopkThreads), kShortLds, s, a);
  else
    hipLaunchKernelGGL(topk_kernel<true>, dim3(a.n_q), dim3(kTopkThreads), kTopkLds, s, a);
  return hipGetLastError();
}

}  // namespace hyb
