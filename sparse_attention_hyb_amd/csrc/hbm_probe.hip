// HBM bandwidth probe: the achievable read (and copy) rate of this GPU's memory, measured with
// plain streaming kernels, so that a kernel's bytes per second can be set against what the memory
// actually delivers as well as against the published peak. Not part of the attention step.
//
// Kernels (256 threads per workgroup, 16-byte vector accesses):
//   read        workgroup w reads its contiguous share of the buffer, U loads per thread in flight
//   read_dyn    workgroups take chunks of the buffer from an atomic counter until it is exhausted
//               (evens out compute units or dies that stream at different rates)
//   read_lds    as read, but through direct global -> LDS loads, four 4 KB stages per wave
//   read_pages  pages of page_bytes in the order of a page list, pages split evenly over the grid
//               (the access pattern of a paged pool with a shuffled block table)
//   copy        dst <- src, contiguous share per workgroup
// Each workgroup may record (XCC id, start tick, end tick, bytes) into `trace` (the 100 MHz
// real-time counter), which shows how the work spreads over the dies.
#include "common.h"
#include "hyb_probe_internal.h"

namespace hyb {

namespace {

constexpr int kProbeThreads = 256;

__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 0xfu;
}

__device__ __forceinline__ void trace_begin(uint64_t* t0) {
  *t0 = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ void trace_end(const ProbeArgs& a, uint64_t t0, uint64_t bytes) {
  __syncthreads();
  if (a.trace != nullptr && threadIdx.x == 0) {
    uint64_t* r = a.trace + 4 * (uint64_t)blockIdx.x;
    r[0] = xcc_id();
    r[1] = t0;
    r[2] = __builtin_amdgcn_s_memrealtime();
    r[3] = bytes;
  }
}

// Keeps the loads alive: the sink is written only when the folded value hits a constant the data
// never produces in practice.
__device__ __forceinline__ void sink(const ProbeArgs& a, uint32_t acc) {
  if (acc == 0x9e3779b9u && a.sink != nullptr) a.sink[blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

template <int U>
__global__ __launch_bounds__(kProbeThreads) void probe_read(ProbeArgs a) {
  uint64_t t0;
  trace_begin(&t0);
  constexpr uint64_t kTile = (uint64_t)kProbeThreads * 16 * U;
  const uint64_t tiles = a.bytes / kTile;
  const uint64_t t_lo = tiles * blockIdx.x / gridDim.x, t_hi = tiles * (blockIdx.x + 1) / gridDim.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.src);
  uint32_t acc = 0;
  for (uint64_t t = t_lo; t < t_hi; ++t) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + (t * U + u) * kProbeThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink(a, acc);
  trace_end(a, t0, (t_hi - t_lo) * kTile);
}

template <int U>
__global__ __launch_bounds__(kProbeThreads) void probe_read_dyn(ProbeArgs a) {
  uint64_t t0;
  trace_begin(&t0);
  constexpr uint64_t kTile = (uint64_t)kProbeThreads * 16 * U;
  const uint64_t tiles = a.bytes / kTile;
  const uint32_t per_grab = (uint32_t)(a.chunk_bytes / kTile) > 0 ? (uint32_t)(a.chunk_bytes / kTile) : 1u;
  const uint64_t n_grabs = (tiles + per_grab - 1) / per_grab;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.src);
  __shared__ uint32_t next;
  uint32_t acc = 0;
  uint64_t done = 0;
  for (;;) {
    __syncthreads();
    if (threadIdx.x == 0) next = atomicAdd(a.counter, 1u);
    __syncthreads();
    const uint64_t g = next;
    if (g >= n_grabs) break;
    const uint64_t t_hi = (g + 1) * per_grab < tiles ? (g + 1) * per_grab : tiles;
    for (uint64_t t = g * per_grab; t < t_hi; ++t) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + (t * U + u) * kProbeThreads + threadIdx.x);
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    done += (t_hi - g * per_grab) * kTile;
  }
  sink(a, acc);
  trace_end(a, t0, done);
}

// Direct global -> LDS load of 16 bytes per lane (lane i's bytes land at lds + 16 i); the caller
// waits for it with s_waitcnt vmcnt before reading the LDS bytes.
__device__ __forceinline__ void probe_lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}

// Each wave streams its share in 4 KB stages (four 1 KB load instructions), three stages in flight.
__global__ __launch_bounds__(kProbeThreads) void probe_read_lds(ProbeArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage[4][4][4096];
  uint64_t t0;
  trace_begin(&t0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr uint64_t kTile = 4096;   // one stage
  const uint64_t tiles = a.bytes / kTile;
  const uint64_t n_w = (uint64_t)gridDim.x * 4, w = (uint64_t)blockIdx.x * 4 + wave;
  const uint64_t t_lo = tiles * w / n_w, t_hi = tiles * (w + 1) / n_w;
  const uint32_t st0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&stage[wave][0][0]);
  auto issue = [&](int s, uint64_t t) {
    const uint64_t tc = t < t_hi ? t : t_lo;   // past the end: re-read the first tile (unused)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int j = 0; j < 4; ++j)
      probe_lds_dma16(a.src + tc * kTile + 1024 * j + 16 * lane, st0 + s * 4096 + 1024 * j);
  };
  uint32_t acc = 0;
  if (t_lo < t_hi) {
    issue(0, t_lo);
    issue(1, t_lo + 1);
    issue(2, t_lo + 2);
    int s = 0;
    for (uint64_t t = t_lo; t < t_hi; ++t) {
      issue((s + 3) & 3, t + 3);
      asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
      const uint32_t* p = reinterpret_cast<const uint32_t*>(&stage[wave][s][0]);
      acc ^= p[lane] ^ p[256 + lane] ^ p[512 + lane] ^ p[768 + lane];
      s = (s + 1) & 3;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  sink(a, acc);
  trace_end(a, t0, (t_hi - t_lo) * kTile);
}

template <int U>
__global__ __launch_bounds__(kProbeThreads) void probe_read_pages(ProbeArgs a) {
  uint64_t t0;
  trace_begin(&t0);
  constexpr uint64_t kTile = (uint64_t)kProbeThreads * 16 * U;
  const uint64_t tiles_per_page = (uint64_t)a.chunk_bytes / kTile;
  const uint64_t tiles = (uint64_t)a.n_pages * tiles_per_page;
  const uint64_t t_lo = tiles * blockIdx.x / gridDim.x, t_hi = tiles * (blockIdx.x + 1) / gridDim.x;
  uint32_t acc = 0;
  for (uint64_t t = t_lo; t < t_hi; ++t) {
    const uint64_t pg = (uint64_t)a.pages[t / tiles_per_page];
    const u32x4* src = reinterpret_cast<const u32x4*>(a.src + pg * (uint64_t)a.chunk_bytes +
                                                      (t % tiles_per_page) * kTile);
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + u * kProbeThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  sink(a, acc);
  trace_end(a, t0, (t_hi - t_lo) * kTile);
}

template <int U>
__global__ __launch_bounds__(kProbeThreads) void probe_copy(ProbeArgs a) {
  uint64_t t0;
  trace_begin(&t0);
  constexpr uint64_t kTile = (uint64_t)kProbeThreads * 16 * U;
  const uint64_t tiles = a.bytes / kTile;
  const uint64_t t_lo = tiles * blockIdx.x / gridDim.x, t_hi = tiles * (blockIdx.x + 1) / gridDim.x;
  const u32x4* src = reinterpret_cast<const u32x4*>(a.src);
  u32x4* dst = reinterpret_cast<u32x4*>(a.dst);
  for (uint64_t t = t_lo; t < t_hi; ++t) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + (t * U + u) * kProbeThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + (t * U + u) * kProbeThreads + threadIdx.x);
  }
  trace_end(a, t0, 2 * (t_hi - t_lo) * kTile);
}

}  // namespace

// Granule (bytes) the buffer of each variant must be a multiple of.
uint64_t probe_granule(int variant, int unroll) {
  if (variant == kProbeReadLds) return 4096;
  return (uint64_t)kProbeThreads * 16 * (uint64_t)unroll;
}

hipError_t launch_probe(int variant, int unroll, int n_wg, const ProbeArgs& a, hipStream_t s) {
  const dim3 grid(n_wg), block(kProbeThreads);
#define HYB_PROBE_UNROLL(K)                                              \
  switch (unroll) {                                                      \
    case 4: hipLaunchKernelGGL(K<4>, grid, block, 0, s, a); break;       \
    case 8: hipLaunchKernelGGL(K<8>, grid, block, 0, s, a); break;       \
    case 16: hipLaunchKernelGGL(K<16>, grid, block, 0, s, a); break;     \
    default: return hipErrorInvalidValue;                                \
  }
  switch (variant) {
    case kProbeRead: HYB_PROBE_UNROLL(probe_read) break;
    case kProbeReadDyn: HYB_PROBE_UNROLL(probe_read_dyn) break;
    case kProbeReadLds: hipLaunchKernelGGL(probe_read_lds, grid, block, 0, s, a); break;
    case kProbeReadPages: HYB_PROBE_UNROLL(probe_read_pages) break;
    case kProbeCopy: HYB_PROBE_UNROLL(probe_copy) break;
    default: return hipErrorInvalidValue;
  }
#undef HYB_PROBE_UNROLL
  return hipGetLastError();
}

}  // namespace hyb
