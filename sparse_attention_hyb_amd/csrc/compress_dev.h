// Device side of the KV compressor (pool -> RMSNorm -> RoPE -> paged insert, with an in-progress
// state ring), shared by the compressor's own kernel and the kernel that runs it beside the
// attention combine.
//
// Method: vLLM DeepSeek-V4 day-0 post, "four moves" (c4a / c128a KV compression) and "vLLM side"
// (fused compressor + RMSNorm + RoPE + cache insert); SGLang DeepSeek-V4 day-0 blog, section
// "Shadow Radix" (each compression layer keeps its in-progress compression state in a state pool).
//
// Layout of the work: one workgroup per (group touched, sequence). A group's r raw tokens are
// read once (each row by one wave: coalesced), pooled in float32 registers, normalised, rotated
// and stored once. The state ring holds the raw tokens of the group in progress in x's own
// storage type (they are copies of x). Only the workgroup of the first group touched reads the
// ring (it is the only group that can hold positions from earlier calls), and the same workgroup
// writes the trailing incomplete group into the ring after its reads, so no two workgroups touch
// the ring.
#pragma once

#include <type_traits>

#include "common.h"
#include "quant_dev.h"

namespace hyb {

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

// A chunk of kVec consecutive elements of a row of T, as raw 32-bit words: 16 bytes in the
// four-word form (four floats or eight bf16), else two or one words (element pairs).
template <typename T, int kVec>
constexpr int chunk_words() {
  return kVec * (int)sizeof(T) / 4;
}

template <typename T, int kVec>
__device__ __forceinline__ void load_words(const T* row, int d,
                                           uint32_t (&w)[chunk_words<T, kVec>()]) {
  constexpr int kW = chunk_words<T, kVec>();
  if constexpr (kW == 4) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(row + d);
    w[0] = q[0]; w[1] = q[1]; w[2] = q[2]; w[3] = q[3];
  } else if constexpr (kW == 2) {
    const u32x2 q = *reinterpret_cast<const u32x2*>(row + d);
    w[0] = q[0]; w[1] = q[1];
  } else {
    w[0] = *reinterpret_cast<const uint32_t*>(row + d);
  }
}

template <typename T, int kVec>
__device__ __forceinline__ void store_words(T* row, int d,
                                            const uint32_t (&w)[chunk_words<T, kVec>()]) {
  constexpr int kW = chunk_words<T, kVec>();
  if constexpr (kW == 4)
    *reinterpret_cast<u32x4*>(row + d) = u32x4{w[0], w[1], w[2], w[3]};
  else if constexpr (kW == 2)
    *reinterpret_cast<u32x2*>(row + d) = u32x2{w[0], w[1]};
  else
    *reinterpret_cast<uint32_t*>(row + d) = w[0];
}

// element e of a chunk held as raw words
template <typename T>
__device__ __forceinline__ float word_elem(const uint32_t* w, int e) {
  if constexpr (sizeof(T) == 4) return __uint_as_float(w[e]);
  else return bf16_to_f32((e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xffffu));
}

// kVec floats at d (LDS partials)
template <int kVec>
__device__ __forceinline__ void store_f32_vec(float* row, int d, const float (&v)[kVec]) {
#pragma unroll
  for (int e = 0; e < kVec; e += (kVec >= 4 ? 4 : 2)) {
    if constexpr (kVec >= 4)
      *reinterpret_cast<f32x4*>(row + d + e) = f32x4{v[e], v[e + 1], v[e + 2], v[e + 3]};
    else
      *reinterpret_cast<float2*>(row + d + e) = make_float2(v[e], v[e + 1]);
  }
}

template <int kVec>
__device__ __forceinline__ void load_f32_vec(const float* row, int d, float (&v)[kVec]) {
#pragma unroll
  for (int e = 0; e < kVec; e += (kVec >= 4 ? 4 : 2)) {
    if constexpr (kVec >= 4) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(row + d + e);
      v[e] = q[0]; v[e + 1] = q[1]; v[e + 2] = q[2]; v[e + 3] = q[3];
    } else {
      const float2 q = *reinterpret_cast<const float2*>(row + d + e);
      v[e] = q.x; v[e + 1] = q.y;
    }
  }
}

// kVec outputs at dim d of pool entry idx
template <int kVec>
__device__ __forceinline__ void store_vec(const PoolDev& p, int64_t idx, int d,
                                          const float (&y)[kVec]) {
  if (p.dtype == F32) {
    store_f32_vec<kVec>(reinterpret_cast<float*>(p.data + idx * p.entry_bytes), d, y);
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(p.data + idx * p.entry_bytes) + d;
    if constexpr (kVec == 8)
      *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                             pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
    else if constexpr (kVec == 4)
      *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    else
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(y[0], y[1]);
  }
}

// Virtual waves pooling one group: min(ratio, 16), 8 above dim 1024. The rows and the order in
// which they are added depend only on this count, not on how many waves run them.
__host__ __device__ inline int pooled_waves(int ratio, int dim) {
  const int v = dim <= 1024 ? 16 : 8;
  return ratio < v ? ratio : v;
}

// One group, pooled by V = pooled_waves(ratio, dim) virtual waves: virtual wave v adds the
// group's tokens t = v, v + V, ... in ascending order, each lane holding kJ chunks of kVec dims of
// the row (chunk c = lane + 64 j, so every row load is a coalesced sweep). The calling
// workgroup's nw = blockDim.x / 64 waves run kV = V / nw virtual waves each (v = w + nw u). Rows
// of the ring and of x have the same storage type and take the same load; all row loads of a
// batch are issued before the first is used. The partial sums p_v are then added as
// ((q_0 + q_1) + q_2) + q_3 with q_k = ((p_k + p_{k+4}) + p_{k+8}) + ...: a fixed order whatever
// nw is (with kV > 1, nw = 4 and wave w forms q_w itself). They meet in LDS behind the one
// barrier of the group, after which wave 0 normalises with a wave-only reduction, rotates and
// stores. The RoPE cos / sin of the entry's position (one pair per lane of the last wave) are
// formed while the row loads are in flight.
// The group is group gi (counted from the first group the call touches) of sequence b; the rows
// per virtual wave, ratio / V, are a multiple of kRB, the rows per virtual wave and batch (the
// launches see to it); lds holds (nw - 1) * dim + 128 floats. kQuant: the pool is FP8_E4M3 or
// FP4_E2M1 and the entry is quantised as it is stored (float32 pools and bf16 pools otherwise).
// kNW > 0: only the first kNW waves of the workgroup pool (nw = kNW); the others take part in
// the group's barrier and nothing else (for workgroups larger than the pooling needs).
template <typename T, int kVec, int kJ, int kRB, int kV, bool kQuant = false, int kNW = 0>
__device__ __forceinline__ void compress_group(const CompressArgs& a, int gi, int b, float* lds) {
  constexpr int kW = chunk_words<T, kVec>();
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = kNW > 0 ? kNW : (blockDim.x >> 6);
  const int V = nw * kV;
  const int r = a.out.ratio;
  const int D = a.out.dim;
  const int nchunks = D / kVec;
  const int c0 = a.cu_seqlens[b];
  const int c1 = a.cu_seqlens[b + 1];
  const int s0 = a.start_pos[b];   // loaded with the offsets: one round trip, not two
  const int n_new = c1 - c0;
  if (n_new <= 0) return;
  const int t_end = s0 + n_new;
  const int g0 = s0 / r;
  const int g_last = (t_end - 1) / r;
  const int g = g0 + gi;
  if (g > g_last) return;
  const int gstart = g * r;
  if (kNW > 0 && w >= kNW) {   // not a pooling wave: only the complete group's barrier
    if (gstart + r <= t_end) __syncthreads();
    return;
  }
  const T* x = reinterpret_cast<const T*>(a.x);
  T* ring = reinterpret_cast<T*>(a.state) + (int64_t)b * r * D;
  float2* cs = reinterpret_cast<float2*>(lds + (nw - 1) * D);

  if (gstart + r <= t_end) {  // group complete: emit entry g
    // block-table entry of the output, loaded now and checked after the barrier
    const int lb = g / a.out.per_block;
    const int phys = lb < a.out.max_blocks ? a.out.block_table[(int64_t)b * a.out.max_blocks + lb] : -1;
    // pooling weights: 1 for the mean (scaled by 1/r at the end), softmax of the logits for the
    // gate; every wave forms the softmax itself (r <= 128: two logits per lane), behind its first
    // batch of row loads
    float e0 = 1.f, e1 = 1.f;
    float l0 = -INFINITY, l1 = -INFINITY;
    if (a.mode == 1) {
      int t = gstart + lane;
      if (lane < r) l0 = t < s0 ? a.state_logits[(int64_t)b * r + lane] : a.gate[c0 + t - s0];
      t += 64;
      if (lane + 64 < r) l1 = t < s0 ? a.state_logits[(int64_t)b * r + lane + 64] : a.gate[c0 + t - s0];
    }

    float acc[kV][kJ][kVec];
#pragma unroll
    for (int u = 0; u < kV; ++u)
#pragma unroll
      for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[u][j][e] = 0.f;
    // Tokens before s0 come from the state ring, the rest from x. Which virtual wave adds which
    // token, and in what order, depends only on t, so a chunked compression adds the same numbers
    // in the same order as a one-shot one.
    const int n_state = max(0, min(s0, gstart + r) - gstart);
    // chunk offsets of this lane; lanes past the row's end load its last chunk again (so no load
    // is predicated) and drop it at the end
    int coff[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) coff[j] = min(lane + 64 * j, nchunks - 1) * kVec;
    const T* xs = x + (int64_t)(c0 - s0 + gstart) * D;   // row of token t of the group: xs + t * D
    // the RoPE frequency of this lane's pair (last wave), read before the rows
    const double theta = a.theta[min(lane, 63)];
    // batch: rows i0 .. i0 + kRB - 1 of each of this wave's virtual waves (row i of virtual wave
    // v is token v + V i), all loaded before any is added
    const int rows = r / V;
    for (int i0 = 0; i0 < rows; i0 += kRB) {
      uint32_t rv[kV][kRB][kJ][kW];
#pragma unroll
      for (int u = 0; u < kV; ++u)
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
          const int t = w + nw * u + V * (i0 + i);
          const T* row = (t < n_state ? ring : xs) + (int64_t)t * D;
#pragma unroll
          for (int j = 0; j < kJ; ++j) load_words<T, kVec>(row, coff[j], rv[u][i][j]);
        }
      if (i0 == 0 && a.mode == 1) {
        float m0 = l0, m1 = l1;
        asm volatile("" : "+v"(m0), "+v"(m1));   // keeps the softmax (and its wait) here
        const float m = wave_max(fmaxf(m0, m1));
        e0 = lane < r ? expf(m0 - m) : 0.f;
        e1 = lane + 64 < r ? expf(m1 - m) : 0.f;
        const float inv = 1.0f / wave_sum(e0 + e1);
        e0 *= inv;
        e1 *= inv;
      }
      if (i0 == 0 && w == nw - 1 && lane < (a.rope_dim >> 1)) {
        // here, behind the batch's loads (the empty asm keeps the compiler from hoisting the
        // math, and the wait for theta, in front of them)
        double th = theta;
        asm volatile("" : "+v"(th));
        float c, s;
        rope_cs_theta((double)(gstart + r - 1), th, &c, &s);
        cs[lane] = make_float2(c, s);
      }
#pragma unroll
      for (int u = 0; u < kV; ++u)
#pragma unroll
        for (int i = 0; i < kRB; ++i) {
          const int t = w + nw * u + V * (i0 + i);
          // weight of token t: lane t mod 64 holds it (t is the same on every lane)
          const float wt = __int_as_float(t < 64 ? __builtin_amdgcn_readlane(__float_as_int(e0), t & 63)
                                                 : __builtin_amdgcn_readlane(__float_as_int(e1), t & 63));
#pragma unroll
          for (int j = 0; j < kJ; ++j)
#pragma unroll
            for (int e = 0; e < kVec; ++e)
              acc[u][j][e] = fmaf(wt, word_elem<T>(rv[u][i][j], e), acc[u][j][e]);
        }
    }
    // with several virtual waves per wave (nw = 4), wave w holds p_w, p_{w+4}, ...: its q_w
#pragma unroll
    for (int u = 1; u < kV; ++u)
#pragma unroll
      for (int j = 0; j < kJ; ++j)
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[0][j][e] += acc[u][j][e];
    if (w > 0) {
      float* part = lds + (w - 1) * D;
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const int c = lane + 64 * j;
        if (c < nchunks) store_f32_vec<kVec>(part, c * kVec, acc[0][j]);
      }
    }
    __syncthreads();
    if (w == 0) {
      const float post = a.mode == 1 ? 1.0f : 1.0f / (float)r;
      float ss = 0.f;
      float (&tot)[kJ][kVec] = acc[0];
#pragma unroll
      for (int j = 0; j < kJ; ++j) {
        const int c = lane + 64 * j;
        if (c < nchunks) {
          // q_k = p_k + p_{k+4} + ... (slot v - 1 holds p_v; with kV > 1 slot k - 1 holds q_k)
          float qk[4][kVec];
          const int per = kV > 1 ? 1 : V / 4;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
#pragma unroll
            for (int e = 0; e < kVec; ++e) qk[k][e] = 0.f;
            for (int m = 0; m < per; ++m) {
              const int v = k + 4 * m;
              float p[kVec];
              if (v == 0) {
#pragma unroll
                for (int e = 0; e < kVec; ++e) p[e] = tot[j][e];
              } else {
                load_f32_vec<kVec>(lds + (v - 1) * D, c * kVec, p);
              }
#pragma unroll
              for (int e = 0; e < kVec; ++e) qk[k][e] = m == 0 ? p[e] : qk[k][e] + p[e];
            }
          }
#pragma unroll
          for (int e = 0; e < kVec; ++e) {
            tot[j][e] = ((qk[0][e] + qk[1][e]) + qk[2][e]) + qk[3][e];
            tot[j][e] *= post;
            ss = fmaf(tot[j][e], tot[j][e], ss);
          }
        }
      }
      ss = wave_sum(ss);
      const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
      note_bad_page(a.out, phys);
      if (phys >= 0 && phys < a.out.num_blocks) {
        const int64_t idx = (int64_t)phys * a.out.per_block + (g - lb * a.out.per_block);
        const int rope_lo = D - a.rope_dim;
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
          const int c = lane + 64 * j;
          if (c < nchunks) {
            float y[kVec];
#pragma unroll
            for (int e = 0; e < kVec; e += 2) {
              float y0 = tot[j][e] * inv, y1 = tot[j][e + 1] * inv;
              const int d = c * kVec + e;
              if (d >= rope_lo) {
                const float2 q = cs[(d - rope_lo) >> 1];
                const float z0 = y0 * q.x - y1 * q.y;
                const float z1 = y0 * q.y + y1 * q.x;
                y0 = z0;
                y1 = z1;
              }
              y[e] = y0;
              y[e + 1] = y1;
            }
            if constexpr (kQuant) {
#pragma unroll
              for (int e = 0; e < kVec; ++e) tot[j][e] = y[e];
            } else {
              store_vec<kVec>(a.out, idx, c * kVec, y);
            }
          }
        }
        if constexpr (kQuant) store_quantized<kVec, kJ>(a.out, idx, lane, nchunks, tot);
      }
    }
  }

  if (gi == 0) {
    // trailing incomplete group -> state ring (raw copies of x's rows)
    const int tail_start = g_last * r;
    if (tail_start + r > t_end) {
      const int lo = tail_start > s0 ? tail_start : s0;
      for (int t = lo + w; t < t_end; t += nw) {
        const int slot = t - tail_start;
        const T* row = x + (int64_t)(c0 + t - s0) * D;
        T* dst = ring + (int64_t)slot * D;
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
          const int c = lane + 64 * j;
          if (c < nchunks) {
            uint32_t v[kW];
            load_words<T, kVec>(row, c * kVec, v);
            store_words<T, kVec>(dst, c * kVec, v);
          }
        }
        if (a.mode == 1 && lane == 0) a.state_logits[(int64_t)b * r + slot] = a.gate[c0 + t - s0];
      }
    }
  }
}

}  // namespace hyb

namespace hyb {

// Fused step before the attention for new tokens ([vLLM] "vLLM side": fused Q-norm + KV RoPE +
// K insert): per token, n_heads waves RMS-normalise and rotate one query head each, and one more
// wave rotates the token's K=V row into the window pool (quantised for an FP8_E4M3 pool). A wave
// holds its whole row (dim <= 2048: up to 16 element pairs per lane) before it writes, so q_out
// may be q.
template <typename T>
__device__ __forceinline__ void store_pair_t(T* row, int d, float x0, float x1) {
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<float2*>(row + d) = make_float2(x0, x1);
  } else {
    *reinterpret_cast<uint32_t*>(row + d) = pack_bf16x2(x0, x1);
  }
}

// Wave wv of sequence b's share (wave-uniform arguments; lane = the wave's lane): token
// i = wv / (n_heads + 1) of the sequence, role wv % (n_heads + 1) = a query head, or n_heads = the
// window entry. Waves past the sequence's tokens return.
template <typename TQ, typename TK>
__device__ __forceinline__ void q_norm_kv_wave(const QNormArgs& a, int b, int wv, int lane) {
  const CompressArgs& c = a.kv;
  const int roles = a.n_heads + 1;
  const int i = wv / roles, role = wv % roles;
  const int c0 = c.cu_seqlens[b];
  if (i >= c.cu_seqlens[b + 1] - c0) return;   // whole waves
  const int t = c.start_pos[b] + i;
  const int64_t tok = c0 + i;
  const int D = c.out.dim;
  const int npairs = D / 2;
  const int rope_lo = D - c.rope_dim;
  float y[16][2];
  if (role < a.n_heads) {
    const TQ* row = reinterpret_cast<const TQ*>(a.q) + (tok * a.n_heads + role) * D;
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int pi = lane + 64 * j;
      float2 v = make_float2(0.f, 0.f);
      if (pi < npairs) v = load_pair<TQ>(row, 2 * pi);
      y[j][0] = v.x;
      y[j][1] = v.y;
      ss = fmaf(v.x, v.x, fmaf(v.y, v.y, ss));
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + a.eps);
    TQ* orow = reinterpret_cast<TQ*>(a.q_out) + (tok * a.n_heads + role) * D;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int pi = lane + 64 * j;
      if (pi < npairs) {
        float y0 = y[j][0] * inv, y1 = y[j][1] * inv;
        const int d = 2 * pi;
        if (d >= rope_lo) {
          float cs, sn;
          rope_cs_theta((double)t, c.theta[(d - rope_lo) >> 1], &cs, &sn);
          const float z0 = y0 * cs - y1 * sn;
          const float z1 = y0 * sn + y1 * cs;
          y0 = z0;
          y1 = z1;
        }
        store_pair_t<TQ>(orow, d, y0, y1);
      }
    }
  } else {
    const int64_t idx = entry_index(c.out, b, t);
    if (idx < 0) return;
    const TK* row = reinterpret_cast<const TK*>(c.x) + tok * D;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int pi = lane + 64 * j;
      float2 v = make_float2(0.f, 0.f);
      if (pi < npairs) {
        v = load_pair<TK>(row, 2 * pi);
        const int d = 2 * pi;
        if (d >= rope_lo) {
          float cs, sn;
          rope_cs_theta((double)t, c.theta[(d - rope_lo) >> 1], &cs, &sn);
          const float z0 = v.x * cs - v.y * sn;
          const float z1 = v.x * sn + v.y * cs;
          v.x = z0;
          v.y = z1;
        }
        if (c.out.dtype != FP8) store_pair(c.out, idx, d, v.x, v.y);
      }
      y[j][0] = v.x;
      y[j][1] = v.y;
    }
    if (c.out.dtype == FP8) store_quantized<2, 16>(c.out, idx, lane, npairs, y);
  }
}

// q_norm_kv_wave for the dtypes of a (F32 or BF16 query and K=V rows).
__device__ __forceinline__ void q_norm_kv_wave_any(const QNormArgs& a, int b, int wv, int lane) {
  const bool qf = a.q_dtype == F32, kf = a.kv.x_dtype == F32;
  if (qf && kf) q_norm_kv_wave<float, float>(a, b, wv, lane);
  else if (qf) q_norm_kv_wave<float, uint16_t>(a, b, wv, lane);
  else if (kf) q_norm_kv_wave<uint16_t, float>(a, b, wv, lane);
  else q_norm_kv_wave<uint16_t, uint16_t>(a, b, wv, lane);
}

// A compressor call that can run as extra workgroups of another launch: four waves pool each
// group in 16-byte chunks (dim <= 512, a whole number of chunks; x, the ring and the pool 16-byte
// aligned), ratio 4 or 128. Host side: the launchers decide with this.
inline bool compress_fusable(const CompressArgs& c) {
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  const int r = c.out.ratio, D = c.out.dim;
  return c.batch > 0 && c.max_new_tokens > 0 && D <= 512 && D % (c.x_dtype == F32 ? 4 : 8) == 0 &&
         al16(c.x) && al16(c.state) && al16(c.out.data) && (r == 4 || r == 128) &&
         (c.out.dtype != FP4 || D % 32 == 0);
}

// Workgroups one fusable call takes: one per (group touched, sequence).
inline int compress_fused_groups(const CompressArgs& c) {
  return ((c.max_new_tokens + c.out.ratio - 1) / c.out.ratio + 1) * c.batch;
}

// LDS (bytes) of one fused compressor workgroup: three waves' partial sums and the RoPE table.
constexpr size_t kCompressFusedLds = (3 * 512 + 128) * sizeof(float);

// Workgroup k of a fusable call, run by the first four waves of the calling workgroup (any other
// waves only take part in the barrier); lds: kCompressFusedLds bytes.
template <int kNW>
__device__ __forceinline__ void compress_fused(const CompressArgs& c, int k, float* lds) {
  const int gx = (c.max_new_tokens + c.out.ratio - 1) / c.out.ratio + 1;
  const int gi = k % gx, b = k / gx;
  const bool quant = c.out.dtype == FP8 || c.out.dtype == FP4;
  if (c.x_dtype == F32) {
    if (c.out.ratio == 4) {
      if (quant) compress_group<float, 4, 2, 1, 1, true, kNW>(c, gi, b, lds);
      else compress_group<float, 4, 2, 1, 1, false, kNW>(c, gi, b, lds);
    } else {
      if (quant) compress_group<float, 4, 2, 2, 4, true, kNW>(c, gi, b, lds);
      else compress_group<float, 4, 2, 2, 4, false, kNW>(c, gi, b, lds);
    }
  } else {
    if (c.out.ratio == 4) {
      if (quant) compress_group<uint16_t, 8, 1, 1, 1, true, kNW>(c, gi, b, lds);
      else compress_group<uint16_t, 8, 1, 1, 1, false, kNW>(c, gi, b, lds);
    } else {
      if (quant) compress_group<uint16_t, 8, 1, 4, 4, true, kNW>(c, gi, b, lds);
      else compress_group<uint16_t, 8, 1, 4, 4, false, kNW>(c, gi, b, lds);
    }
  }
}

}  // namespace hyb
