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

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of a 64-bit value over the workgroup (thread order).
__device__ __forceinline__ uint64_t block_exclusive_scan(uint64_t v, uint64_t* wave_tot,
                                                         uint64_t* total_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint64_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint64_t n = __shfl_up(incl, o, 64);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint64_t before = 0, total = 0;
  for (int w = 0; w < kTopkWaves; ++w) {
    uint64_t t = wave_tot[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  if (total_out) *total_out = total;
  return before + incl - v;
}

// Each thread owns kPer consecutive scores of a 32768-score chunk, held in registers as keys:
// one row of up to 32768 scores is read from memory once, with all loads of a thread in flight
// together; longer rows are re-read chunk by chunk in every pass.
constexpr int kPer = 32;
constexpr int kChunk = kTopkThreads * kPer;

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
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
  const int n_chunks = (n + kChunk - 1) / kChunk;

  __shared__ uint32_t hist[2048];
  __shared__ uint64_t wave_tot[kTopkWaves];
  __shared__ uint32_t s_bin, s_above;

  uint32_t u[kPer];
  auto load_chunk = [&](int c) {
    const int base = c * kChunk + tid * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int j = base + e;
      u[e] = j < n ? order_key(sc[j]) : 0u;
    }
  };
  auto count_in = [&](int c) { return max(0, min(kPer, n - (c * kChunk + tid * kPer))); };
  if (n_chunks == 1) load_chunk(0);

  uint32_t prefix = 0, pmask = 0;
  uint32_t remaining = (uint32_t)k;  // how many still to take among keys matching the prefix
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t bmask = pass == 2 ? 1023u : 2047u;
    for (int j = tid; j < 2048; j += kTopkThreads) hist[j] = 0;
    __syncthreads();
#pragma unroll 1
    for (int c = 0; c < n_chunks; ++c) {
      if (n_chunks > 1) load_chunk(c);
      const int cnt = count_in(c);
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        if (e < cnt && (u[e] & pmask) == prefix) atomicAdd(&hist[(u[e] >> shift) & bmask], 1u);
    }
    __syncthreads();
    // bins in descending order: thread t owns bins 2047-2t and 2046-2t
    const uint32_t bh = 2047u - 2u * tid, bl = bh - 1u;
    const uint32_t ch = hist[bh], cl = hist[bl];
    uint64_t above = block_exclusive_scan((uint64_t)(ch + cl), wave_tot, nullptr);
    if (above < remaining && above + ch >= remaining) {
      s_bin = bh;
      s_above = (uint32_t)above;
    } else if (above + ch < remaining && above + ch + cl >= remaining) {
      s_bin = bl;
      s_above = (uint32_t)(above + ch);
    }
    __syncthreads();
    prefix |= s_bin << shift;
    pmask |= bmask << shift;
    remaining -= s_above;
    __syncthreads();
  }
  const uint32_t T = prefix;  // key of the k-th largest score; `remaining` ties of it are taken

  uint32_t gt_base = 0, tie_base = 0;
#pragma unroll 1
  for (int c = 0; c < n_chunks; ++c) {
    if (n_chunks > 1) load_chunk(c);
    const int cnt = count_in(c);
    uint32_t gt = 0, tie = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      gt += (e < cnt) & (u[e] > T);
      tie += (e < cnt) & (u[e] == T);
    }
    uint64_t tot = 0;
    uint64_t pre = block_exclusive_scan(((uint64_t)tie << 32) | gt, wave_tot, &tot);
    const uint32_t gt_pre = gt_base + (uint32_t)pre;
    const uint32_t tie_pre = tie_base + (uint32_t)(pre >> 32);
    uint32_t pos = gt_pre + min(remaining, tie_pre);
    uint32_t tseen = tie_pre;
    const int base = c * kChunk + tid * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      if (e < cnt) {
        if (u[e] > T) {
          if (pos < (uint32_t)k) out[pos] = base + e;
          ++pos;
        } else if (u[e] == T) {
          if (tseen < remaining) {
            if (pos < (uint32_t)k) out[pos] = base + e;
            ++pos;
          }
          ++tseen;
        }
      }
    }
    gt_base += (uint32_t)tot;
    tie_base += (uint32_t)(tot >> 32);
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(a.n_q), dim3(kTopkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hyb
