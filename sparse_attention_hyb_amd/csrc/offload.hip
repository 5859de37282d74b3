// Offloaded C4 pool (SGLang DeepSeek-V4 day-0 blog, section "HiSparse"): the whole compressed
// cache lives in a pinned host mirror, the device keeps a working set of pages, and every step
// brings in the pages its top-k selection misses, evicting the least recently used ones the step
// does not need; new entries are backed up to the mirror. Here every part of that runs on the
// device, in the step's stream: no top-k row is read back to the host.
//
// A page is one logical block (256 positions, `per_page` entries); its key is
// sequence * max_blocks + logical block. Kernels of one admission:
//   offload_mark    one thread per selected entry (and per extra page key): a resident page gets
//                   the step's stamp; a missing one is claimed once (per-page claim word = step)
//                   and appended to the miss list;
//   offload_assign  one workgroup: sorts the misses by key, picks as many victims among the slots
//                   the step does not need (smallest stamp first, lowest slot first), pairs the
//                   i-th miss with the i-th victim in slot order, updates the tables and writes the
//                   copy list;
//   offload_copy    one workgroup per listed page: mirror page -> slot (through the mirror's
//                   device alias), and its scale page.
// offload_write_back copies the entry each sequence completed at its position back to the mirror.
#include "common.h"
#include "hyb_internal.h"

namespace hyb {

namespace {

constexpr int kAssignThreads = 1024;
constexpr int kPerThread = kMaxOffloadSlots / kAssignThreads;   // 16 slots per thread

// Workspace: claim words, then a 256-byte header (miss count), the miss list and the copy list.
struct OffloadWs {
  uint32_t* claim;      // [batch * max_blocks]
  uint32_t* n_miss;     // [1]
  int32_t* miss;        // [n_slots]
  int32_t* copy;        // [1 + 2 n_slots]: count, (mirror page, slot) pairs
};

__global__ __launch_bounds__(256) void offload_mark(OffloadArgs a, OffloadWs w) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n_sel = (int64_t)a.batch * a.k;
  int64_t key = -1;
  if (t < n_sel) {
    const int e = a.topk[t];
    const int b = (int)(t / a.k);
    if (e >= 0 && e / a.per_page < a.max_blocks) key = (int64_t)b * a.max_blocks + e / a.per_page;
  } else if (t - n_sel < a.n_extra) {
    const int32_t x = a.extra[t - n_sel];
    if (x >= 0 && x < a.batch * a.max_blocks) key = x;
  }
  if (key < 0) return;
  const int slot = a.dev_table[key];
  if (slot >= 0 && slot < a.n_slots) {
    a.slot_stamp[slot] = a.step;   // needed this step (every writer stores the same value)
  } else if (atomicExch(w.claim + key, a.step) != a.step) {
    const uint32_t m = atomicAdd(w.n_miss, 1u);
    if (m < (uint32_t)a.n_slots) w.miss[m] = (int32_t)key;
  }
}

// Sum of v over the workgroup (every thread gets it); red: 2 words of LDS, zero on entry is not
// needed. Two barriers.
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* red) {
  const int lane = threadIdx.x & 63;
  const uint32_t ws = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(v), 63);
  if (threadIdx.x == 0) red[0] = 0u;
  __syncthreads();
  if (lane == 0) atomicAdd(red, ws);
  __syncthreads();
  const uint32_t s = red[0];
  __syncthreads();   // red is reused by the next call
  return s;
}

// Exclusive scan over the workgroup in thread order; total to *tot. wt: 16 words of LDS.
__device__ __forceinline__ uint32_t block_excl(uint32_t v, uint32_t* wt, uint32_t* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_scan(v);
  if (lane == 63) wt[wave] = incl;
  __syncthreads();
  uint32_t before = 0, total = 0;
#pragma unroll
  for (int x = 0; x < kAssignThreads / 64; ++x) {
    const uint32_t s = wt[x];
    before += x < wave ? s : 0u;
    total += s;
  }
  __syncthreads();
  *tot = total;
  return before + incl - v;
}

__global__ __launch_bounds__(kAssignThreads) void offload_assign(OffloadArgs a, OffloadWs w) {
  __shared__ int32_t keys[kMaxOffloadSlots];
  __shared__ uint32_t wt[16], red[2];
  const int tid = threadIdx.x;
  const uint32_t m_all = *w.n_miss;
  const int m = (int)min(m_all, (uint32_t)a.n_slots);
  // ---- the misses, ascending by key (bitonic sort of the next power of two, padded high)
  int P = 1;
  while (P < m) P <<= 1;
  for (int j = tid; j < P; j += kAssignThreads) keys[j] = j < m ? w.miss[j] : 0x7fffffff;
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int j = tid; j < P; j += kAssignThreads) {
        const int o = j ^ stride;
        if (o > j) {
          const bool up = (j & size) == 0;
          const int x = keys[j], y = keys[o];
          if ((x > y) == up) {
            keys[j] = y;
            keys[o] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  // ---- candidate slots (not needed this step): slots 16 tid .. 16 tid + 15
  uint32_t st[kPerThread];
  uint32_t cand = 0;   // bit e: slot 16 tid + e is a candidate
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const int v = kPerThread * tid + e;
    st[e] = v < a.n_slots ? a.slot_stamp[v] : a.step;
    if (v < a.n_slots && st[e] < a.step) cand |= 1u << e;
  }
  const uint32_t n_cand = block_sum(__builtin_popcount(cand), red);
  const int mm = (int)min((uint32_t)m, n_cand);   // misses admitted
  if (mm > 0) {
    // smallest T with #{candidates with stamp <= T} >= mm (binary search over [0, step - 1])
    uint32_t lo = 0, hi = a.step - 1;
    while (lo < hi) {   // uniform
      const uint32_t mid = lo + (hi - lo) / 2;
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < kPerThread; ++e) c += ((cand >> e) & 1u) && st[e] <= mid;
      if ((int)block_sum(c, red) >= mm) hi = mid; else lo = mid + 1;
    }
    const uint32_t T = lo;
    uint32_t below = 0, eq = 0;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      below += ((cand >> e) & 1u) && st[e] < T;
      eq += ((cand >> e) & 1u) && st[e] == T;
    }
    const int n_below = (int)block_sum(below, red);
    uint32_t eq_tot = 0;
    const uint32_t eq_before = block_excl(eq, wt, &eq_tot);
    const int take_eq = mm - n_below;   // lowest slots with stamp T
    // victims in slot order and their ranks
    uint32_t vic = 0, r = eq_before;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (!((cand >> e) & 1u)) continue;
      if (st[e] < T) vic |= 1u << e;
      else if (st[e] == T) {
        if ((int)r < take_eq) vic |= 1u << e;
        ++r;
      }
    }
    uint32_t vtot = 0;
    uint32_t rank = block_excl(__builtin_popcount(vic), wt, &vtot);
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (!((vic >> e) & 1u)) continue;
      const int v = kPerThread * tid + e;
      const int key = keys[rank];
      const int old = a.slot_owner[v];
      if (old >= 0 && old < a.batch * a.max_blocks) a.dev_table[old] = -1;
      a.slot_owner[v] = key;
      a.slot_stamp[v] = a.step;
      a.dev_table[key] = v;
      w.copy[1 + 2 * rank] = a.mirror_table[key];
      w.copy[2 + 2 * rank] = v;
      ++rank;
    }
  }
  if (tid == 0) {
    w.copy[0] = mm;
    *w.n_miss = 0u;   // for the next call
    a.result[0] = mm;
    a.result[1] = (int32_t)(m_all - (uint32_t)mm);
  }
}

// Workgroup j copies listed page j (mirror page -> slot), 16 bytes per thread and load, every
// load of a thread issued before its stores; then the page's scales.
__device__ __forceinline__ void copy_page(const uint8_t* src, uint8_t* dst, int64_t bytes) {
  const u32x4* s = reinterpret_cast<const u32x4*>(src);
  u32x4* d = reinterpret_cast<u32x4*>(dst);
  const int64_t n16 = bytes / 16;
  constexpr int kU = 8;
  for (int64_t o = threadIdx.x; o < n16; o += 256 * kU) {
    u32x4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (o + 256 * u < n16) v[u] = s[o + 256 * u];
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (o + 256 * u < n16) d[o + 256 * u] = v[u];
  }
}

__global__ __launch_bounds__(256) void offload_copy(OffloadArgs a, OffloadWs w) {
  const int j = blockIdx.x;
  if (j >= w.copy[0]) return;
  const int sp = w.copy[1 + 2 * j], dp = w.copy[2 + 2 * j];
  if (sp < 0 || sp >= a.n_mirror_pages || dp < 0 || dp >= a.n_slots) return;
  copy_page(a.mirror + (int64_t)sp * a.page_bytes, a.pool + (int64_t)dp * a.page_bytes, a.page_bytes);
  if (a.scale_page_bytes > 0)
    copy_page(a.mirror_scale + (int64_t)sp * a.scale_page_bytes,
              a.pool_scale + (int64_t)dp * a.scale_page_bytes, a.scale_page_bytes);
}

// One thread per sequence: the entry completed at its position p = seq_lens[b] - 1 (when
// (p + 1) % ratio == 0) goes from its slot back to its mirror page; copies of 16 bytes.
__global__ __launch_bounds__(64) void offload_write_back(OffloadArgs a, const int32_t* seq_lens,
                                                         int ratio, int64_t entry_bytes,
                                                         int64_t scale_bytes) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= a.batch) return;
  const int p = seq_lens[b] - 1;
  if (p < 0 || (p + 1) % ratio != 0) return;
  const int g = (p + 1) / ratio - 1;
  const int lb = g / a.per_page, row = g % a.per_page;
  if (lb >= a.max_blocks) return;
  const int64_t key = (int64_t)b * a.max_blocks + lb;
  const int slot = a.dev_table[key], mp = a.mirror_table[key];
  if (slot < 0 || slot >= a.n_slots || mp < 0 || mp >= a.n_mirror_pages) return;
  const u32x4* s = reinterpret_cast<const u32x4*>(a.pool + (int64_t)slot * a.page_bytes + row * entry_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(a.mirror + (int64_t)mp * a.page_bytes + row * entry_bytes);
  for (int64_t o = 0; o < entry_bytes / 16; ++o) d[o] = s[o];
  if (scale_bytes > 0) {
    const uint8_t* ss = a.pool_scale + (int64_t)slot * a.scale_page_bytes + row * scale_bytes;
    uint8_t* ds = a.mirror_scale + (int64_t)mp * a.scale_page_bytes + row * scale_bytes;
    for (int64_t o = 0; o < scale_bytes; ++o) ds[o] = ss[o];
  }
}

OffloadWs carve(void* ws, int32_t batch, int32_t max_blocks, int32_t n_slots) {
  char* p = static_cast<char*>(ws);
  OffloadWs w{};
  w.claim = reinterpret_cast<uint32_t*>(p);
  p += ((size_t)batch * max_blocks * sizeof(uint32_t) + 255) / 256 * 256;
  w.n_miss = reinterpret_cast<uint32_t*>(p);
  p += 256;
  w.miss = reinterpret_cast<int32_t*>(p);
  p += ((size_t)n_slots * sizeof(int32_t) + 255) / 256 * 256;
  w.copy = reinterpret_cast<int32_t*>(p);
  return w;
}

}  // namespace

size_t offload_ws_bytes(int32_t batch, int32_t max_blocks, int32_t n_slots) {
  return ((size_t)batch * max_blocks * sizeof(uint32_t) + 255) / 256 * 256 + 256 +
         ((size_t)n_slots * sizeof(int32_t) + 255) / 256 * 256 + (1 + 2 * (size_t)n_slots) * sizeof(int32_t);
}

hipError_t launch_offload_admit(const OffloadArgs& a, void* ws, hipStream_t s) {
  const OffloadWs w = carve(ws, a.batch, a.max_blocks, a.n_slots);
  const int64_t n = (int64_t)a.batch * a.k + a.n_extra;
  if (n > 0) hipLaunchKernelGGL(offload_mark, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, w);
  hipLaunchKernelGGL(offload_assign, dim3(1), dim3(kAssignThreads), 0, s, a, w);
  hipLaunchKernelGGL(offload_copy, dim3(a.n_slots), dim3(256), 0, s, a, w);
  return hipGetLastError();
}

hipError_t launch_offload_write_back(const OffloadArgs& a, const int32_t* seq_lens, int ratio,
                                     int64_t entry_bytes, int64_t scale_bytes, hipStream_t s) {
  hipLaunchKernelGGL(offload_write_back, dim3((a.batch + 63) / 64), dim3(64), 0, s, a, seq_lens,
                     ratio, entry_bytes, scale_bytes);
  return hipGetLastError();
}

}  // namespace hyb
