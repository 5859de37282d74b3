// Exact top-k per row: the first min(k, n) indices under (score descending, index ascending), with
// -0.0 equal to +0.0, written in ascending index order and padded with -1.
// Method: SGLang DeepSeek-V4 day-0 blog, section "Shadow Radix" (C4 layers keep the top-512
// compressed entries chosen by the indexer); vLLM day-0 post ("DeepSeek Sparse Attention over
// compressed tokens").
//
// One 1024-thread workgroup per row. Scores become order-preserving 32-bit keys held in
// registers (32 consecutive scores per thread); three radix passes (11 + 11 + 10 bits,
// histograms in LDS) find the k-th largest key T and how many of the keys equal to T are taken
// (the lowest-indexed ones). Because every thread owns a contiguous index range, one workgroup
// scan of its "> T" and "== T" counts gives each chosen index its output slot directly - the
// output is ascending without a sort.
#include "common.h"

namespace hyb {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Exclusive scan of a 32-bit value over the workgroup (thread order); also returns the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot,
                                                         uint32_t* total_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t t = wave_tot[w];
    before += w < wave ? t : 0u;
    total += t;
  }
  __syncthreads();
  if (total_out) *total_out = total;
  return before + incl - v;
}

// Each thread owns kPer consecutive scores of a chunk of kChunk, held in registers as keys. A
// chunk is fetched with coalesced 16-byte loads and redistributed through LDS (row pitch padded
// to 36 words so the per-thread reads do not collide in banks); rows longer than one chunk are
// re-read chunk by chunk in every pass.
constexpr int kPer = 32;
constexpr int kChunk = kTopkThreads * kPer;
constexpr int kStagePitch = kPer + 4;  // words per thread's slice in the staging area

// Dynamic LDS: staging [kTopkThreads][kStagePitch] words (also reused for the per-wave
// histograms of the first pass: kTopkWaves x 2048 words), then hist[2048].
constexpr size_t kTopkLds = sizeof(uint32_t) * ((size_t)kTopkThreads * kStagePitch + kHistBins);

// kMulti: rows may exceed one chunk (launched when max_len > kChunk); the single-chunk form keeps
// the row in registers from the start and needs far fewer registers.
template <bool kMulti>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t tk_lds[];
  uint32_t* stage = tk_lds;
  uint32_t* hist = tk_lds + kTopkThreads * kStagePitch;
  __shared__ uint32_t wave_tot[kTopkWaves];
  __shared__ uint32_t s_bin, s_above;

  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  int n;
  if (a.lengths) {
    n = a.lengths[i];
  } else {
    int seq, p;
    query_at(a.qd, i, &seq, &p);
    n = n_visible(p, a.ratio, a.window);
  }
  n = max(0, min(n, a.max_len));
  const int k = a.k;
  int* out = a.out + (int64_t)i * k;
  if (n <= k) {
    for (int j = tid; j < k; j += kTopkThreads) out[j] = j < n ? j : -1;
    return;
  }
  const float* sc = a.scores + (int64_t)i * a.ld;
  const bool aligned16 = ((reinterpret_cast<uintptr_t>(sc) & 15u) == 0);
  const int n_chunks = kMulti ? (n + kChunk - 1) / kChunk : 1;

  uint32_t u[kPer];
  auto load_chunk = [&](int c) {
    const int base = c * kChunk;
    __syncthreads();  // the staging area may still hold histograms or the previous chunk
    // coalesced: thread t moves elements base + 4*(t + 1024*q) .. +3 for q = 0..7
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const int j = base + 4 * (tid + kTopkThreads * q);
      u32x4 v;
      if (aligned16 && j + 3 < n) {
        const f32x4 f = *reinterpret_cast<const f32x4*>(sc + j);
        v[0] = order_key(f[0]);
        v[1] = order_key(f[1]);
        v[2] = order_key(f[2]);
        v[3] = order_key(f[3]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = j + e < n ? order_key(sc[j + e]) : 0u;
      }
      const int jj = j - base;  // element within the chunk: owner thread jj / 32, slot jj % 32
      *reinterpret_cast<u32x4*>(stage + (jj / kPer) * kStagePitch + (jj % kPer)) = v;
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

  uint32_t prefix = 0, pmask = 0;
  uint32_t remaining = (uint32_t)k;  // how many still to take among keys matching the prefix
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t bmask = pass == 2 ? 1023u : 2047u;
    if (pass == 0 && a.hist) {
      // the indexer already counted the top 11 bits of every score of this row
      __syncthreads();
      const uint32_t* g = a.hist + (int64_t)i * kHistBins;
      for (int j = tid; j < kHistBins; j += kTopkThreads) hist[j] = g[j];
      __syncthreads();
    } else {
      // the first pass counts into per-wave histograms (the busiest bins would otherwise
      // serialise atomics of all waves) laid over the staging area, once its data is in registers
      const bool private_hist = pass == 0 && n_chunks == 1;
      uint32_t* h = private_hist ? stage + wave * kHistBins : hist;
      __syncthreads();
      if (private_hist) {
        for (int j = lane; j < kHistBins; j += 64) h[j] = 0;
      } else {
        for (int j = tid; j < kHistBins; j += kTopkThreads) hist[j] = 0;
      }
      __syncthreads();
#pragma unroll 1
      for (int c = 0; c < n_chunks; ++c) {
        if (kMulti && n_chunks > 1) load_chunk(c);
        uint32_t m = match_mask(valid_mask(c), pmask, prefix);
        if (pass == 0) {
#pragma unroll
          for (int e = 0; e < kPer; ++e)
            if ((m >> e) & 1u) atomicAdd(&h[u[e] >> shift], 1u);
        } else {
          // later passes see few matching keys: visit only those
          while (m) {
            const int e = __builtin_ctz(m);
            m &= m - 1;
            uint32_t ue = 0;
#pragma unroll
            for (int q = 0; q < kPer; ++q) ue = q == e ? u[q] : ue;
            atomicAdd(&h[(ue >> shift) & bmask], 1u);
          }
        }
      }
      __syncthreads();
      if (private_hist) {
        for (int j = tid; j < kHistBins; j += kTopkThreads) {
          uint32_t t = 0;
#pragma unroll
          for (int w = 0; w < kTopkWaves; ++w) t += stage[w * kHistBins + j];
          hist[j] = t;
        }
        __syncthreads();
      }
    }
    // Wave 0 finds the bin holding the remaining-th largest key: lane l sums 32 bins (in
    // descending order), one wave scan, then the owning lane walks its 32 bins in registers.
    if (wave == 0) {
      uint32_t hb[32];
      const u32x4* hv = reinterpret_cast<const u32x4*>(hist + kHistBins - 32 * (lane + 1));
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const u32x4 v = hv[q];
        hb[31 - 4 * q] = v[0];
        hb[30 - 4 * q] = v[1];
        hb[29 - 4 * q] = v[2];
        hb[28 - 4 * q] = v[3];
      }
      uint32_t sum = 0;
#pragma unroll
      for (int e = 0; e < 32; ++e) sum += hb[e];
      const uint32_t incl = wave_inclusive_scan(sum);
      const uint32_t excl = incl - sum;
      if (excl < remaining && incl >= remaining) {
        uint32_t above = excl;
        int found = 31;
        uint32_t found_above = 0;
        bool done = false;
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const bool hit = !done && above + hb[e] >= remaining;
          found = hit ? e : found;
          found_above = hit ? above : found_above;
          done = done || hit;
          above += hb[e];
        }
        s_bin = (uint32_t)(kHistBins - 1 - 32 * lane - found);
        s_above = found_above;
      }
    }
    __syncthreads();
    prefix |= s_bin << shift;
    pmask |= bmask << shift;
    remaining -= s_above;
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

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  static bool attr_set = false;   // the dynamic LDS above 64 KiB must be enabled once per kernel
  if (!attr_set) {
    for (const void* f : {reinterpret_cast<const void*>(topk_kernel<false>),
                          reinterpret_cast<const void*>(topk_kernel<true>)}) {
      hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kTopkLds);
      if (e != hipSuccess) return e;
    }
    attr_set = true;
  }
  if (a.max_len <= kChunk)
    hipLaunchKernelGGL(topk_kernel<false>, dim3(a.n_q), dim3(kTopkThreads), kTopkLds, s, a);
  else
    hipLaunchKernelGGL(topk_kernel<true>, dim3(a.n_q), dim3(kTopkThreads), kTopkLds, s, a);
  return hipGetLastError();
}

}  // namespace hyb
