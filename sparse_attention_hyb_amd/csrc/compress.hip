// KV compressor kernel and the raw sliding-window insert (RoPE only).
//
// Method: vLLM DeepSeek-V4 day-0 post, "four moves" (c4a / c128a KV compression) and "vLLM side"
// (fused compressor + RMSNorm + RoPE + cache insert; fused KV RoPE + K insert); SGLang DeepSeek-V4
// day-0 blog, section "Shadow Radix" (in-progress compression state in a state pool). The
// compressor's device code is in compress_dev.h.
#include <algorithm>

#include "compress_dev.h"

namespace hyb {

template <typename T, int kVec, int kJ, int kRB, bool kQuant>
__global__ __launch_bounds__(1024) void compress_kernel(CompressArgs a) {
  extern __shared__ float lds[];   // [nw - 1][D] partials, then cs pairs
  compress_group<T, kVec, kJ, kRB, 1, kQuant>(a, blockIdx.x, blockIdx.y, lds);
}

// Raw window entries: s_t = RoPE(x_t, t), stored at position t of the ratio-1 pool.
constexpr int kInsertTokens = 8;

template <typename T>
__global__ __launch_bounds__(256) void swa_insert_kernel(CompressArgs a) {
  const int b = blockIdx.y;
  const int c0 = a.cu_seqlens[b];
  const int n_new = a.cu_seqlens[b + 1] - c0;
  const int s0 = a.start_pos[b];
  const int D = a.out.dim;
  const int npairs = D / 2;
  const int rope_lo = D - a.rope_dim;
  const T* x = reinterpret_cast<const T*>(a.x);
  for (int i = blockIdx.x * kInsertTokens; i < (blockIdx.x + 1) * kInsertTokens && i < n_new; ++i) {
    const int t = s0 + i;
    const int64_t idx = entry_index(a.out, b, t);
    if (idx < 0) continue;
    const T* row = x + (int64_t)(c0 + i) * D;
    for (int pi = threadIdx.x; pi < npairs; pi += blockDim.x) {
      float2 v = load_pair<T>(row, 2 * pi);
      int d = 2 * pi;
      if (d >= rope_lo) {
        float c, s;
        rope_cs_theta((double)t, a.theta[(d - rope_lo) >> 1], &c, &s);
        float z0 = v.x * c - v.y * s;
        float z1 = v.x * s + v.y * c;
        v.x = z0;
        v.y = z1;
      }
      store_pair(a.out, idx, d, v.x, v.y);
    }
  }
}

// Window entries into an FP8_E4M3 pool (quantise-on-insert): one wave per token (dim <= 2048:
// up to 16 element pairs per lane), the rotated row quantised with one scale per entry.
constexpr int kInsertWaves = 4;

template <typename T>
__global__ __launch_bounds__(64 * kInsertWaves) void swa_insert_fp8_kernel(CompressArgs a) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * kInsertWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int c0 = a.cu_seqlens[b];
  if (i >= a.cu_seqlens[b + 1] - c0) return;   // whole waves
  const int t = a.start_pos[b] + i;
  const int64_t idx = entry_index(a.out, b, t);
  if (idx < 0) return;
  const int D = a.out.dim;
  const int npairs = D / 2;
  const int rope_lo = D - a.rope_dim;
  const T* row = reinterpret_cast<const T*>(a.x) + (int64_t)(c0 + i) * D;
  float y[16][2];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int pi = lane + 64 * j;
    float2 v = make_float2(0.f, 0.f);
    if (pi < npairs) {
      v = load_pair<T>(row, 2 * pi);
      const int d = 2 * pi;
      if (d >= rope_lo) {
        float c, s;
        rope_cs_theta((double)t, a.theta[(d - rope_lo) >> 1], &c, &s);
        const float z0 = v.x * c - v.y * s;
        const float z1 = v.x * s + v.y * c;
        v.x = z0;
        v.y = z1;
      }
    }
    y[j][0] = v.x;
    y[j][1] = v.y;
  }
  store_quantized<2, 16>(a.out, idx, lane, npairs, y);
}

// Fused step before the attention for new tokens (q_norm_kv_wave in compress_dev.h): kInsertWaves
// of its waves per workgroup, workgroup row b = sequence b.
template <typename TQ, typename TK>
__global__ __launch_bounds__(64 * kInsertWaves) void q_norm_kv_insert_kernel(QNormArgs a) {
  q_norm_kv_wave<TQ, TK>(a, blockIdx.y, blockIdx.x * kInsertWaves + (threadIdx.x >> 6), threadIdx.x & 63);
}

namespace {
template <typename T, int kVec, int kJ>
hipError_t launch_compress_t(const CompressArgs& a, int rows_per_wave, dim3 grid, dim3 block,
                             size_t lds, hipStream_t s) {
  // rows per batch and virtual wave: up to 64 words of loads in flight per lane and 8 rows for
  // rows of up to 8 words, fewer for wider rows (whose accumulators take registers too)
  constexpr int kWords = kJ * chunk_words<T, kVec>();
  constexpr int kRB = kWords >= 32 ? 1 : (kWords >= 16 ? 2 : (64 / kWords > 8 ? 8 : 64 / kWords));
  const bool quant = a.out.dtype == FP8 || a.out.dtype == FP4;
  if (quant) {
    if (rows_per_wave % kRB == 0)
      hipLaunchKernelGGL((compress_kernel<T, kVec, kJ, kRB, true>), grid, block, lds, s, a);
    else
      hipLaunchKernelGGL((compress_kernel<T, kVec, kJ, 1, true>), grid, block, lds, s, a);
  } else if (rows_per_wave % kRB == 0) {
    hipLaunchKernelGGL((compress_kernel<T, kVec, kJ, kRB, false>), grid, block, lds, s, a);
  } else {
    hipLaunchKernelGGL((compress_kernel<T, kVec, kJ, 1, false>), grid, block, lds, s, a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_compress_x(const CompressArgs& a, bool wide, int rows_per_wave, dim3 grid,
                             dim3 block, size_t lds, hipStream_t s) {
  constexpr int kWide = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  const bool small = a.out.dim <= 512;
  if (wide) return small ? launch_compress_t<T, kWide, 512 / kWide / 64>(a, rows_per_wave, grid, block, lds, s)
                         : launch_compress_t<T, kWide, 2048 / kWide / 64>(a, rows_per_wave, grid, block, lds, s);
  return small ? launch_compress_t<T, 2, 4>(a, rows_per_wave, grid, block, lds, s)
               : launch_compress_t<T, 2, 16>(a, rows_per_wave, grid, block, lds, s);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
}  // namespace

// dim <= 2048, ratio 4 or 128. One wave per virtual wave of the group (min(ratio, 16), 8 above
// dim 1024, so the partials fit in 60 KB of LDS). 16-byte chunks (four floats or eight bf16)
// when x, the state ring and the pool are 16-byte aligned and a row is a whole number of
// chunks, else element pairs.
hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  const int r = a.out.ratio;
  const int D = a.out.dim;
  const int nw = pooled_waves(r, D);
  const bool wide = D % (a.x_dtype == F32 ? 4 : 8) == 0 && aligned16(a.x) && aligned16(a.state) &&
                    aligned16(a.out.data);
  const dim3 grid((a.max_new_tokens + r - 1) / r + 1, a.batch);
  const dim3 block(64 * nw);
  const size_t lds = ((size_t)(nw - 1) * D + 128) * sizeof(float);
  return a.x_dtype == F32 ? launch_compress_x<float>(a, wide, r / nw, grid, block, lds, s)
                          : launch_compress_x<uint16_t>(a, wide, r / nw, grid, block, lds, s);
}

hipError_t launch_swa_insert(const CompressArgs& a, hipStream_t s) {
  if (a.out.dtype == FP8) {
    dim3 grid((a.max_new_tokens + kInsertWaves - 1) / kInsertWaves, a.batch);
    if (a.x_dtype == F32)
      hipLaunchKernelGGL(swa_insert_fp8_kernel<float>, grid, dim3(64 * kInsertWaves), 0, s, a);
    else
      hipLaunchKernelGGL(swa_insert_fp8_kernel<uint16_t>, grid, dim3(64 * kInsertWaves), 0, s, a);
    return hipGetLastError();
  }
  dim3 grid((a.max_new_tokens + kInsertTokens - 1) / kInsertTokens, a.batch);
  if (a.x_dtype == F32)
    hipLaunchKernelGGL(swa_insert_kernel<float>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(swa_insert_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_q_norm_kv_insert(const QNormArgs& a, hipStream_t s) {
  const int64_t waves = (int64_t)a.kv.max_new_tokens * (a.n_heads + 1);
  const dim3 grid((unsigned)((waves + kInsertWaves - 1) / kInsertWaves), a.kv.batch);
  const dim3 block(64 * kInsertWaves);
  const bool qf = a.q_dtype == F32, kf = a.kv.x_dtype == F32;
  if (qf && kf)
    hipLaunchKernelGGL((q_norm_kv_insert_kernel<float, float>), grid, block, 0, s, a);
  else if (qf)
    hipLaunchKernelGGL((q_norm_kv_insert_kernel<float, uint16_t>), grid, block, 0, s, a);
  else if (kf)
    hipLaunchKernelGGL((q_norm_kv_insert_kernel<uint16_t, float>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((q_norm_kv_insert_kernel<uint16_t, uint16_t>), grid, block, 0, s, a);
  return hipGetLastError();
}

// Working-set fill of an offloaded pool: workgroup j copies page src_page[j] of the host mirror
// (through its device alias) to page dst_page[j] of the device pool, 16 bytes per thread and
// load, every load of a thread issued before its stores.
__global__ __launch_bounds__(256) void gather_pages_kernel(const uint8_t* src, int32_t n_src,
                                                           uint8_t* dst, int32_t n_dst,
                                                           const int32_t* src_page,
                                                           const int32_t* dst_page,
                                                           int64_t page_bytes) {
  const int j = blockIdx.x;
  const int sp = src_page[j], dp = dst_page[j];
  if (sp < 0 || sp >= n_src || dp < 0 || dp >= n_dst) return;   // out of range: skipped
  const u32x4* s = reinterpret_cast<const u32x4*>(src + (int64_t)sp * page_bytes);
  u32x4* d = reinterpret_cast<u32x4*>(dst + (int64_t)dp * page_bytes);
  const int64_t n16 = page_bytes / 16;
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

hipError_t launch_gather_pages(const void* src_dev, int32_t n_src, void* dst, int32_t n_dst,
                               const int32_t* src_page, const int32_t* dst_page, int32_t n,
                               int64_t page_bytes, hipStream_t s) {
  hipLaunchKernelGGL(gather_pages_kernel, dim3(n), dim3(256), 0, s,
                     static_cast<const uint8_t*>(src_dev), n_src, static_cast<uint8_t*>(dst), n_dst,
                     src_page, dst_page, page_bytes);
  return hipGetLastError();
}

}  // namespace hyb
