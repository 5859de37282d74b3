// KV compressor (pool -> RMSNorm -> RoPE -> paged insert, with an in-progress state ring) and the
// raw sliding-window insert (RoPE only).
//
// Method: vLLM DeepSeek-V4 day-0 post, "four moves" (c4a / c128a KV compression) and "vLLM side"
// (fused compressor + RMSNorm + RoPE + cache insert; fused KV RoPE + K insert); SGLang DeepSeek-V4
// day-0 blog, section "Shadow Radix" (each compression layer keeps its in-progress compression
// state in a state pool).
//
// Layout of the work: one workgroup per (group touched, sequence). A group's r raw tokens are
// read once, row by row (each row is read by the whole workgroup: coalesced), pooled in float32
// registers, normalised with a workgroup reduction, rotated and stored once. Only the workgroup of
// the first group touched reads the state ring (it is the only group that can hold positions
// from earlier calls), and the same workgroup writes the trailing incomplete group into the ring
// after its reads, so no two workgroups touch the ring.
#include "common.h"

namespace hyb {

constexpr int kCompressThreads = 1024;
constexpr int kRowGroups = 4;                                  // token rows split 4 ways
constexpr int kPairThreads = kCompressThreads / kRowGroups;    // 256 threads per row group
constexpr int kMaxPairsPerThread = 4;                          // dim <= 2048

template <typename T>
__device__ __forceinline__ float2 load_pair(const T* row, int d);

template <>
__device__ __forceinline__ float2 load_pair<float>(const float* row, int d) {
  return *reinterpret_cast<const float2*>(row + d);
}

template <>
__device__ __forceinline__ float2 load_pair<uint16_t>(const uint16_t* row, int d) {
  uint32_t v = *reinterpret_cast<const uint32_t*>(row + d);
  return make_float2(bf16_to_f32(v & 0xffffu), bf16_to_f32(v >> 16));
}

__device__ __forceinline__ void store_pair(const PoolDev& p, int64_t idx, int d, float a,
                                           float b) {
  if (p.dtype == F32) {
    float* dst = reinterpret_cast<float*>(p.data + idx * p.entry_bytes);
    *reinterpret_cast<float2*>(dst + d) = make_float2(a, b);
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(p.data + idx * p.entry_bytes);
    *reinterpret_cast<uint32_t*>(dst + d) = pack_bf16x2(a, b);
  }
}

template <typename T>
__global__ __launch_bounds__(kCompressThreads) void compress_kernel(CompressArgs a) {
  const int b = blockIdx.y;
  const int gi = blockIdx.x;
  const int tid = threadIdx.x;
  const int pt = tid % kPairThreads;   // which dim pairs
  const int rg = tid / kPairThreads;   // which token rows (t = rg mod 4)
  const int r = a.out.ratio;
  const int D = a.out.dim;
  const int npairs = D / 2;
  const int c0 = a.cu_seqlens[b];
  const int n_new = a.cu_seqlens[b + 1] - c0;
  if (n_new <= 0) return;
  const int s0 = a.start_pos[b];
  const int t_end = s0 + n_new;
  const int g0 = s0 / r;
  const int g_last = (t_end - 1) / r;
  const int g = g0 + gi;
  if (g > g_last) return;
  const int gstart = g * r;
  const T* x = reinterpret_cast<const T*>(a.x);

  __shared__ float wts[128];
  __shared__ float red[kPairThreads / 64];
  __shared__ float2 part[kRowGroups - 1][kMaxPairsPerThread * kPairThreads];

  if (gstart + r <= t_end) {  // group complete: emit entry g
    if (tid < 64) {
      // pooling weights: 1/r for the mean, softmax of the logits for the gate
      float l0 = -INFINITY, l1 = -INFINITY;
      if (a.mode == 1) {
        int t = gstart + tid;
        if (tid < r) l0 = t < s0 ? a.state_logits[(int64_t)b * r + tid] : a.gate[c0 + t - s0];
        t = gstart + tid + 64;
        if (tid + 64 < r) l1 = t < s0 ? a.state_logits[(int64_t)b * r + tid + 64] : a.gate[c0 + t - s0];
        float m = wave_max(fmaxf(l0, l1));
        float e0 = tid < r ? expf(l0 - m) : 0.f;
        float e1 = tid + 64 < r ? expf(l1 - m) : 0.f;
        float inv = 1.0f / wave_sum(e0 + e1);
        if (tid < r) wts[tid] = e0 * inv;
        if (tid + 64 < r) wts[tid + 64] = e1 * inv;
      } else {
        if (tid < r) wts[tid] = 1.0f;
        if (tid + 64 < r) wts[tid + 64] = 1.0f;
      }
    }
    __syncthreads();

    float acc[kMaxPairsPerThread][2];
#pragma unroll
    for (int j = 0; j < kMaxPairsPerThread; ++j) acc[j][0] = acc[j][1] = 0.f;
    // Row group rg sums the group's tokens t = rg, rg + 4, ... in ascending order: those that
    // arrived in earlier calls from the state ring, the rest from x. The split depends only on
    // t, so a chunked compression adds exactly the same numbers in the same order as a one-shot
    // one. Loops are unrolled so each thread keeps several row loads in flight.
    const int n_state = max(0, min(s0, gstart + r) - gstart);
#pragma unroll 8
    for (int t = rg; t < n_state; t += kRowGroups) {
      const float wt = wts[t];
      const float* row = a.state + ((int64_t)b * r + t) * D;
#pragma unroll
      for (int j = 0; j < kMaxPairsPerThread; ++j) {
        int pi = pt + j * kPairThreads;
        if (pi < npairs) {
          float2 v = load_pair<float>(row, 2 * pi);
          acc[j][0] = fmaf(wt, v.x, acc[j][0]);
          acc[j][1] = fmaf(wt, v.y, acc[j][1]);
        }
      }
    }
    const int t_x0 = n_state + ((rg - n_state) % kRowGroups + kRowGroups) % kRowGroups;
#pragma unroll 8
    for (int t = t_x0; t < r; t += kRowGroups) {
      const float wt = wts[t];
      const T* row = x + (int64_t)(c0 + gstart + t - s0) * D;
#pragma unroll
      for (int j = 0; j < kMaxPairsPerThread; ++j) {
        int pi = pt + j * kPairThreads;
        if (pi < npairs) {
          float2 v = load_pair<T>(row, 2 * pi);
          acc[j][0] = fmaf(wt, v.x, acc[j][0]);
          acc[j][1] = fmaf(wt, v.y, acc[j][1]);
        }
      }
    }
    if (rg > 0) {
#pragma unroll
      for (int j = 0; j < kMaxPairsPerThread; ++j)
        part[rg - 1][pt + j * kPairThreads] = make_float2(acc[j][0], acc[j][1]);
    }
    __syncthreads();
    const float post = a.mode == 1 ? 1.0f : 1.0f / (float)r;
    float ss = 0.f;
    if (rg == 0) {
#pragma unroll
      for (int j = 0; j < kMaxPairsPerThread; ++j) {
#pragma unroll
        for (int q = 0; q < kRowGroups - 1; ++q) {
          const float2 v = part[q][pt + j * kPairThreads];
          acc[j][0] += v.x;
          acc[j][1] += v.y;
        }
        acc[j][0] *= post;
        acc[j][1] *= post;
        ss = fmaf(acc[j][0], acc[j][0], fmaf(acc[j][1], acc[j][1], ss));
      }
      ss = wave_sum(ss);
      if ((tid & 63) == 0) red[tid >> 6] = ss;
    }
    __syncthreads();
    if (rg == 0) {
      float tot = 0.f;
#pragma unroll
      for (int w = 0; w < kPairThreads / 64; ++w) tot += red[w];
      const float inv = 1.0f / sqrtf(tot / (float)D + a.eps);
      const int64_t idx = entry_index(a.out, b, g);
      const int rope_lo = D - a.rope_dim;
      const double pos = (double)(gstart + r - 1);
#pragma unroll
      for (int j = 0; j < kMaxPairsPerThread; ++j) {
        int pi = pt + j * kPairThreads;
        if (pi < npairs && idx >= 0) {
          float y0 = acc[j][0] * inv, y1 = acc[j][1] * inv;
          int d = 2 * pi;
          if (d >= rope_lo) {
            float c, s;
            rope_cs(pos, (d - rope_lo) >> 1, a.rope_dim, a.rope_base, &c, &s);
            float z0 = y0 * c - y1 * s;
            float z1 = y0 * s + y1 * c;
            y0 = z0;
            y1 = z1;
          }
          store_pair(a.out, idx, d, y0, y1);
        }
      }
    }
  }

  if (gi == 0) {
    // trailing incomplete group -> state ring (this workgroup's ring reads are finished)
    const int tail_start = g_last * r;
    if (tail_start + r > t_end) {
      __syncthreads();
      const int lo = tail_start > s0 ? tail_start : s0;
      for (int t = lo + rg; t < t_end; t += kRowGroups) {
        const int slot = t - tail_start;
        const T* row = x + (int64_t)(c0 + t - s0) * D;
        float* dst = a.state + ((int64_t)b * r + slot) * D;
        for (int pi = pt; pi < npairs; pi += kPairThreads) {
          float2 v = load_pair<T>(row, 2 * pi);
          *reinterpret_cast<float2*>(dst + 2 * pi) = v;
        }
        if (a.mode == 1 && pt == 0) a.state_logits[(int64_t)b * r + slot] = a.gate[c0 + t - s0];
      }
    }
  }
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
        rope_cs((double)t, (d - rope_lo) >> 1, a.rope_dim, a.rope_base, &c, &s);
        float z0 = v.x * c - v.y * s;
        float z1 = v.x * s + v.y * c;
        v.x = z0;
        v.y = z1;
      }
      store_pair(a.out, idx, d, v.x, v.y);
    }
  }
}

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  const int r = a.out.ratio;
  dim3 grid((a.max_new_tokens + r - 1) / r + 1, a.batch);
  if (a.x_dtype == F32)
    hipLaunchKernelGGL(compress_kernel<float>, grid, dim3(kCompressThreads), 0, s, a);
  else
    hipLaunchKernelGGL(compress_kernel<uint16_t>, grid, dim3(kCompressThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_swa_insert(const CompressArgs& a, hipStream_t s) {
  dim3 grid((a.max_new_tokens + kInsertTokens - 1) / kInsertTokens, a.batch);
  if (a.x_dtype == F32)
    hipLaunchKernelGGL(swa_insert_kernel<float>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(swa_insert_kernel<uint16_t>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hyb
