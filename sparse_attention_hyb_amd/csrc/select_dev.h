// Exact top-k selection device code shared by the selector kernels (topk.hip) and by the
// attention kernel that selects its own compressed entries from the indexer's hand-off.
// Selection rule: the first min(k, n) indices under (key descending, index ascending), written in
// ascending index order and padded with -1.
// Method: SGLang DeepSeek-V4 day-0 blog, section "Shadow Radix" (C4 layers keep the top-512
// compressed entries chosen by the indexer); vLLM day-0 post ("DeepSeek Sparse Attention over
// compressed tokens").
#pragma once

#include "common.h"

namespace hyb {

// Histograms live in LDS with one padding word after every 32 bins: bin b at hp(b). A lane that
// reads 32 consecutive bins then starts 33 words after its neighbour, so the 64 lanes of a wave
// hit 64 different banks.
__device__ __forceinline__ int hp(uint32_t b) { return (int)(b + (b >> 5)); }
constexpr int kHistWords = 2048 + 2048 / 32;   // padded 2048-bin histogram
constexpr int kShift0 = 32 - kTopBits;         // 22: first pass = key bits 22..31
constexpr int kBits12 = kShift0 / 2;           // 11: second pass bits 11..21, third 0..10

// Exclusive scan of a 32-bit value over an NT-thread workgroup (thread order); also returns the
// total. Two barriers.
template <int NT>
__device__ __forceinline__ uint32_t block_scan_excl(uint32_t v, uint32_t* wave_tot, uint32_t* total_out) {
  constexpr int W = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const uint32_t t = wave_tot[w];
    before += w < wave ? t : 0u;
    total += t;
  }
  __syncthreads();
  if (total_out) *total_out = total;
  return before + incl - v;
}

// Bin holding the `remaining`-th largest key of an nbins-bin histogram (nbins = 1024 or 2048,
// bins in ascending key order) and the number of keys in the bins above it. Wave 0 searches:
// lane l sums the 32-bin group [nbins - 32(l+1), nbins - 32l), one wave scan finds the group
// that holds the bin, a second scan over that group's 32 bins (one per lane, descending) finds
// the bin. The result reaches every thread through LDS (one barrier). The histogram must hold at
// least `remaining` keys.
__device__ __forceinline__ void select_bin(const uint32_t* hist, int nbins, uint32_t remaining,
                                           uint32_t* res, uint32_t* bin, uint32_t* above) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int groups = nbins >> 5;
    uint32_t sum = 0;
    if (lane < groups) {
      const uint32_t* g = hist + 33 * (groups - 1 - lane);
#pragma unroll
      for (int m = 0; m < 32; ++m) sum += g[m];
    }
    const uint32_t incl = wave_inclusive_scan(sum);
    const uint32_t excl = incl - sum;
    const uint64_t own = __ballot(excl < remaining && incl >= remaining);
    const int grp = own ? __builtin_ctzll(own) : 0;
    const uint32_t grp_above = (uint32_t)__builtin_amdgcn_readlane((int)excl, grp);
    const int top = nbins - 1 - 32 * grp;
    const uint32_t c = lane < 32 ? hist[hp(top - lane)] : 0u;
    const uint32_t incl2 = wave_inclusive_scan(c) + grp_above;
    const uint32_t excl2 = incl2 - c;
    const uint64_t hit = __ballot(lane < 32 && excl2 < remaining && incl2 >= remaining);
    const int j = hit ? __builtin_ctzll(hit) : 0;
    if (lane == j) {
      res[0] = (uint32_t)(top - j);
      res[1] = excl2;
    }
  }
  __syncthreads();
  *bin = res[0];
  *above = res[1];
}

// ------------------------------------------------------------------------------------------
// Selection of one row from the indexer's hand-off by one workgroup of kSelThreads threads.
// The hand-off (see the indexer): per part of kScorePartKeys keys the (order key, index) pairs
// bucketed by the top kTopBits key bits, highest bin first, with the part's cumulative bin counts,
// and the row's bin counts (row_hist). Steps:
//   1. (with the loads of the first step of the caller) the row's bin counts, two bins per thread,
//      and the leading pairs of every part: 8 per thread, kSelPrefetch / parts per part (a power
//      of two), requested before the row length is known;
//   2. one workgroup scan of the counts gives C[b] = keys with top bits >= b and the first-pass
//      bin b0: C[b0] >= k > C[b0 + 1];
//   3. the candidates are the keys with top bits >= b0, the leading pairs of every part. When
//      every part's candidates lie within its prefetched pairs (its last prefetched pair is below
//      b0, or the part is fetched whole) they come from registers; otherwise each part's count
//      comes from its cumulative counts at b0 and the pairs from memory;
//   4. two 11-bit passes over the candidates whose top bits equal b0 find the k-th largest key T
//      and how many keys equal to T are taken (the lowest-indexed ones);
//   5. output in ascending index order, 32768 indices at a time: bit maps of the chosen keys > T
//      and == T, one workgroup scan of the packed counts (two map words per thread).
// When the candidates exceed the LDS list they are read from the hand-off in every step instead.
// ------------------------------------------------------------------------------------------
constexpr int kSelThreads = 512;
constexpr int kSelPrefetch = 4096;            // pairs requested in step 1 (8 per thread)
constexpr int kSelPer = kSelPrefetch / kSelThreads;
constexpr int kSelMaxParts = 1024;            // rows of up to 1024 x 1024 entries
constexpr int kSelCap = 4096;                 // candidates held in LDS
constexpr int kSelMapWords = 1024;            // one output chunk of 32768 indices
constexpr int kSelChunk = 32 * kSelMapWords;
// LDS words of select_finish: two histograms | two maps | wave totals + results | (slow path)
// counts | offsets | keys | indices
constexpr int kSelLdsWords = 2 * kHistWords + 2 * kSelMapWords + 16 + 2 * (kSelMaxParts + 1) + 2 * kSelCap;

// Registers of step 1: bins 1022 - 2t (x) and 1023 - 2t (y) of the row, and kSelPer prefetched
// pairs: slot s = t + kSelThreads e holds pair s mod P of part s / P, P = 2^lp.
struct SelRegs {
  u32x2 rh;
  u32x2 pre[kSelPer];
};

__device__ __forceinline__ int sel_prefetch_log2(int parts) {   // P = 2^lp pairs per part
  int lp = 31 - __builtin_clz((uint32_t)(kSelPrefetch / max(parts, 1)) | 1u);
  return min(lp, 10);
}

// Step 1 for row i (every load in bounds of the row; no wait here).
__device__ __forceinline__ void select_issue(const SelDev& s, int i, SelRegs& R) {
  const int t = threadIdx.x;
  R.rh = *reinterpret_cast<const u32x2*>(s.row_hist + (int64_t)i * kTopBins + (kTopBins - 2 - 2 * t));
  const int nb_max = (s.max_nv + kScorePartKeys - 1) / kScorePartKeys;
  const int lp = sel_prefetch_log2(nb_max);
  const uint32_t* row = s.pairs + (int64_t)i * s.ld;
#pragma unroll
  for (int e = 0; e < kSelPer; ++e) {
    const int slot = t + kSelThreads * e;
    const int p = min(slot >> lp, s.part_ld - 1), pos = slot & ((1 << lp) - 1);
    R.pre[e] = *reinterpret_cast<const u32x2*>(row + 2 * ((int64_t)p * kScorePartKeys + pos));
  }
}

// Output of a selection, 32768 indices at a time: the chosen keys > T and the first `remaining`
// keys == T (lowest index first), in ascending index order, into lsel and (write_out) gout.
// for_each(f) calls f(key, index) for every candidate; maps: two zeroed kSelMapWords-word maps.
// Thread t owns map words 2t and 2t + 1.
template <typename ForEach>
__device__ __forceinline__ void select_output(int n, int k, uint32_t T, uint32_t remaining,
                                              uint32_t* gtmap, uint32_t* tiemap, uint32_t* wt,
                                              int32_t* lsel, int32_t* gout, bool write_out,
                                              ForEach for_each) {
  constexpr int NT = kSelThreads;
  const int t = threadIdx.x;
  uint32_t gt_base = 0, tie_base = 0;
  const int n_chunks = (n + kSelChunk - 1) / kSelChunk;
#pragma unroll 1
  for (int c = 0; c < n_chunks; ++c) {
    const uint32_t lo = (uint32_t)c * kSelChunk;
    if (c > 0) {
      __syncthreads();   // the previous chunk's maps are read
      for (int j = t; j < 2 * kSelMapWords; j += NT) gtmap[j] = 0u;   // both maps
      __syncthreads();
    }
    for_each([&](uint32_t key, uint32_t idx) {
      const uint32_t j = idx - lo;
      if (j < (uint32_t)kSelChunk) {
        if (key > T) atomicOr(&gtmap[j >> 5], 1u << (j & 31));
        else if (key == T) atomicOr(&tiemap[j >> 5], 1u << (j & 31));
      }
    });
    __syncthreads();
    const uint32_t g0 = gtmap[2 * t], g1 = gtmap[2 * t + 1];
    const uint32_t e0 = tiemap[2 * t], e1 = tiemap[2 * t + 1];
    const uint32_t gc0 = __builtin_popcount(g0), gc1 = __builtin_popcount(g1);
    const uint32_t tc0 = __builtin_popcount(e0), tc1 = __builtin_popcount(e1);
    uint32_t tot = 0;
    // per-chunk counts <= 32768: both fit 16 bits of one word
    const uint32_t pre = block_scan_excl<NT>(((tc0 + tc1) << 16) | (gc0 + gc1), wt, &tot);
    const uint32_t gt_pre = gt_base + (pre & 0xffffu);
    const uint32_t tie_pre = tie_base + (pre >> 16);
    // word w takes all its keys > T and, lowest index first, the ties still owed when it begins
    auto emit = [&](uint32_t gm, uint32_t tm, uint32_t tc, uint32_t gt_before, uint32_t tie_before, int w) {
      const int32_t left = (int32_t)remaining - (int32_t)tie_before;
      const int32_t take = max(0, min(left, (int32_t)tc));
      uint32_t keep = 0;
      for (int32_t q = 0; q < take; ++q) {
        keep |= tm & (0u - tm);
        tm &= tm - 1;
      }
      uint32_t sel = gm | keep;
      uint32_t pos = gt_before + (uint32_t)((int32_t)remaining - max(left, 0));
      while (sel) {
        const int b = __builtin_ctz(sel);
        sel &= sel - 1;
        if (pos < (uint32_t)k) {
          const int32_t idx = (int32_t)(lo + 32 * w + b);
          lsel[pos] = idx;
          if (write_out) gout[pos] = idx;
        }
        ++pos;
      }
    };
    emit(g0, e0, tc0, gt_pre, tie_pre, 2 * t);
    emit(g1, e1, tc1, gt_pre + gc0, tie_pre + tc0, 2 * t + 1);
    gt_base += tot & 0xffffu;
    tie_base += tot >> 16;
  }
  __syncthreads();   // lsel complete
}

// Steps 2-5 for row i of length n (n <= kSelMaxParts * kScorePartKeys): the k chosen indices
// (ascending, -1 padded) into lsel (LDS, k ints), and into s.out when write_out. lds:
// kSelLdsWords words of scratch. Every thread of the workgroup calls it (barriers inside).
// Fast path (every part's candidates among the prefetched pairs): each thread keeps its eight
// pairs in registers throughout - the passes and the output read no candidate list - and the
// first refining pass is counted while the pairs are classified.
__device__ inline void select_finish(const SelDev& s, int i, int n, int k, uint32_t* lds, int32_t* lsel,
                                     bool write_out, const SelRegs& R) {
  constexpr int NT = kSelThreads;
  const int t = threadIdx.x;
  int32_t* gout = s.out + (int64_t)i * k;
  n = min(n, s.max_nv);   // as the indexer scored it
  if (n <= k) {   // uniform: every entry, in order
    for (int j = t; j < k; j += NT) {
      const int v = j < n ? j : -1;
      lsel[j] = v;
      if (write_out) gout[j] = v;
    }
    __syncthreads();
    return;
  }
  uint32_t* hist1 = lds;                        // [kHistWords] second-pass histogram
  uint32_t* hist2 = hist1 + kHistWords;         // [kHistWords] third-pass histogram
  uint32_t* gtmap = hist2 + kHistWords;         // [kSelMapWords]
  uint32_t* tiemap = gtmap + kSelMapWords;      // [kSelMapWords]
  uint32_t* wt = tiemap + kSelMapWords;         // [8] wave totals
  uint32_t* res = wt + 8;                       // [0] bin, [1] above, [2] incomplete flag, [3] C[b0]
  const int nb = (n + kScorePartKeys - 1) / kScorePartKeys;
  const int nb_max = (s.max_nv + kScorePartKeys - 1) / kScorePartKeys;
  const int lp = sel_prefetch_log2(nb_max);
  const int P = 1 << lp;

  // ---- 2. C[b] over the row and b0 (thread t holds bins 1023 - 2t and 1022 - 2t); the
  // histograms and maps are cleared meanwhile
  for (int j = t; j < 2 * kHistWords + 2 * kSelMapWords; j += NT) hist1[j] = 0u;
  if (t == 0) res[2] = 0u;
  const uint32_t c_hi = R.rh[1], c_lo = R.rh[0];
  const uint32_t excl = block_scan_excl<NT>(c_hi + c_lo, wt, nullptr);
  const uint32_t C_hi = excl + c_hi, C_lo = C_hi + c_lo;
  if (C_hi >= (uint32_t)k && excl < (uint32_t)k) {
    res[0] = (uint32_t)(kTopBins - 1 - 2 * t);
    res[1] = excl;
    res[3] = C_hi;
  }
  if (C_lo >= (uint32_t)k && C_hi < (uint32_t)k) {
    res[0] = (uint32_t)(kTopBins - 2 - 2 * t);
    res[1] = C_hi;
    res[3] = C_lo;
  }
  __syncthreads();
  const uint32_t b0 = res[0], above0 = res[1], M0 = res[3];

  // ---- 3. classify the prefetched pairs: candidate (top bits >= b0) or not; a part whose last
  // prefetched pair is still a candidate may hold more (slow path). The second pass (bits 11..21
  // of the keys in bin b0) is counted here already.
  uint32_t candm = 0;   // bit e: pair e is a candidate
#pragma unroll
  for (int e = 0; e < kSelPer; ++e) {
    const int slot = t + NT * e;
    const int p = slot >> lp, pos = slot & (P - 1);
    const int size_p = min(kScorePartKeys, n - p * kScorePartKeys);
    const uint32_t key = R.pre[e][0];
    const uint32_t bin = key >> kShift0;
    if (p < nb && pos < size_p && bin >= b0) {
      candm |= 1u << e;
      if (pos == P - 1 && P < size_p) res[2] = 1u;
      if (bin == b0) atomicAdd(&hist1[hp((key >> kBits12) & 2047u)], 1u);
    }
  }
  __syncthreads();
  uint32_t remaining = (uint32_t)k - above0;
  if (res[2] == 0u) {   // uniform: fast path
    uint32_t b1, ab1, b2, ab2;
    select_bin(hist1, 2048, remaining, res, &b1, &ab1);
    remaining -= ab1;
    const uint32_t pre1 = (b0 << kBits12) | b1;   // key bits 11..31 of T
#pragma unroll
    for (int e = 0; e < kSelPer; ++e) {
      const uint32_t key = R.pre[e][0];
      if (((candm >> e) & 1u) && (key >> kBits12) == pre1) atomicAdd(&hist2[hp(key & 2047u)], 1u);
    }
    __syncthreads();
    select_bin(hist2, 2048, remaining, res, &b2, &ab2);
    remaining -= ab2;
    const uint32_t T = (pre1 << kBits12) | b2;
    (void)M0;
    select_output(n, k, T, remaining, gtmap, tiemap, wt, lsel, gout, write_out, [&](auto f) {
#pragma unroll
      for (int e = 0; e < kSelPer; ++e)
        if ((candm >> e) & 1u) f(R.pre[e][0], R.pre[e][1]);
    });
    return;
  }

  // ---- slow path: each part's candidates from its cumulative counts at b0, the pairs from the
  // hand-off (into LDS when they fit, else re-read in every step)
  uint32_t* cnt = res + 8;                      // [kSelMaxParts + 1]
  uint32_t* off = cnt + kSelMaxParts + 1;       // [kSelMaxParts + 1]
  uint32_t* lkey = off + kSelMaxParts + 1;      // [kSelCap]
  uint32_t* lidx = lkey + kSelCap;              // [kSelCap]
  const uint32_t* row = s.pairs + (int64_t)i * s.ld;
  for (int p = t; p < nb; p += NT) cnt[p] = s.part_hist[((int64_t)i * s.part_ld + p) * kTopBins + b0];
  __syncthreads();
  {
    // exclusive scan of the counts over parts (two parts per thread)
    const uint32_t v0 = 2 * t < nb ? cnt[2 * t] : 0u, v1 = 2 * t + 1 < nb ? cnt[2 * t + 1] : 0u;
    uint32_t total = 0;
    const uint32_t run = block_scan_excl<NT>(v0 + v1, wt, &total);
    if (2 * t < nb) off[2 * t] = run;
    if (2 * t + 1 < nb) off[2 * t + 1] = run + v0;
    if (t == 0) off[nb] = total;
  }
  __syncthreads();
  const uint32_t M = off[nb];
  const bool in_lds = M <= (uint32_t)kSelCap;   // uniform
  auto fetch = [&](uint32_t m) -> u32x2 {       // candidate m from the hand-off
    int lo = 0, hi = nb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= m) lo = mid; else hi = mid - 1;
    }
    const uint32_t pos = min(m - off[lo], (uint32_t)kScorePartKeys - 1u);
    return *reinterpret_cast<const u32x2*>(row + 2 * ((int64_t)lo * kScorePartKeys + pos));
  };
  if (in_lds) {
    for (uint32_t m = t; m < M; m += NT) {
      const u32x2 pr = fetch(m);
      lkey[m] = pr[0];
      lidx[m] = pr[1];
    }
  }
  __syncthreads();
  auto cand = [&](uint32_t m) -> u32x2 {
    if (in_lds) return u32x2{lkey[m], lidx[m]};
    return fetch(m);
  };
  uint32_t prefix = b0 << kShift0, pmask = ~0u << kShift0;
#pragma unroll 1
  for (int shift = kBits12; shift >= 0; shift -= kBits12) {
    for (int j = t; j < kHistWords; j += NT) hist1[j] = 0u;
    __syncthreads();
    for (uint32_t m = t; m < M; m += NT) {
      const uint32_t key = cand(m)[0];
      if ((key & pmask) == prefix) atomicAdd(&hist1[hp((key >> shift) & 2047u)], 1u);
    }
    __syncthreads();
    uint32_t b, ab;
    select_bin(hist1, 2048, remaining, res, &b, &ab);
    prefix |= b << shift;
    pmask |= 2047u << shift;
    remaining -= ab;
  }
  select_output(n, k, prefix, remaining, gtmap, tiemap, wt, lsel, gout, write_out, [&](auto f) {
    for (uint32_t m = t; m < M; m += NT) {
      const u32x2 pr = cand(m);
      f(pr[0], pr[1]);
    }
  });
}

}  // namespace hyb
