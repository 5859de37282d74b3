// Hybrid attention (decode and prefill): each query attends, with one shared K=V head, to its raw
// sliding window plus either its selected compressed entries (C4, sparse) or every visible
// compressed entry (C128, dense); the output gets the inverse RoPE of the query position.
// Method: vLLM DeepSeek-V4 day-0 post, "four moves" ("Shared K/V + inverse RoPE", "DeepSeek
// Sparse Attention over compressed tokens", "short sliding window"); SGLang DeepSeek-V4 day-0
// blog, section "Shadow Radix" (SWA over the newest 128 raw tokens + C4 top-512 or C128 dense).
//
// A query's keys form one list: window entries (ascending positions) then compressed entries.
// Split-K: workgroup (split, query) folds keys [split*chunk, (split+1)*chunk) into an online
// softmax state (m, l, o) per head and writes it as a partial; attn_combine merges the partials
// with their log-sum-exp weights, applies RoPE(-p) and casts.
//
// attn_mfma (64 heads x 512 dims, bf16 query, bf16 or fp8 pools): 4 waves as a 2 x 2 grid
// (head half hh, dim half dh). Per 32-key tile:
//   QK   S^T[key][h] = sum_d K[key][d] Q[h][d] on v_mfma_f32_32x32x16_bf16, each wave over its
//        256 dims with its 32 heads; K rows go straight from HBM into operand registers.
//        The two dim halves are summed through LDS (both waves add the same two fp32 values,
//        so they hold identical sums).
//   soft each lane owns one head and 16 keys of the tile: row max / sum need one cross-half
//        shuffle; the probabilities are already laid out as the PV B operand (no data movement).
//   PV   O^T[d][h] += sum_key K^T[d][key] P^T[key][h], each wave for its 256 dims x 32 heads. The
//        K tile (the same bytes as the values) is staged once in LDS by the four waves and read
//        back transposed.
// fp8 pools: codes are widened to bf16 exactly; the per-entry scale multiplies the score before
// the softmax and the probability before PV (so no rounding of scaled values).
#include "common.h"

namespace hyb {

constexpr int kMH = 64;         // heads in the MFMA kernel
constexpr int kMD = 512;        // dims in the MFMA kernel
constexpr int kKT = 32;         // keys per tile in the MFMA kernel
constexpr int kKRow = kMD + 8;  // LDS row pitch of the K tile (bf16 elements)
constexpr int kGenTile = 64;    // keys per tile in the generic kernel
constexpr int kMaxSplit = 64;
constexpr float kLog2e = 1.4426950408889634f;

// Where key j of a query lives: a pool and the flattened entry index (-1 = masked).
struct KeyRef {
  int64_t idx;
  int comp;
};

__device__ __forceinline__ KeyRef resolve_key(const AttnArgs& a, int i, int seq, int ws, int n_win,
                                              int nv, int j) {
  KeyRef r{-1, 0};
  if (j < n_win) {
    r.idx = entry_index(a.swa, seq, ws + j);
  } else {
    int c = j - n_win;
    int g = a.topk ? a.topk[(int64_t)i * a.k + c] : c;
    r.comp = 1;
    if (g >= 0 && g < nv) r.idx = entry_index(a.comp, seq, g);
  }
  return r;
}

struct QueryKeys {
  int seq, p, ws, n_win, nv, n_keys;
};

__device__ __forceinline__ QueryKeys query_keys(const AttnArgs& a, int i) {
  QueryKeys k;
  query_at(a.qd, i, &k.seq, &k.p);
  k.ws = window_start(k.p, a.window);
  k.n_win = k.p - k.ws + 1;
  k.nv = n_visible(k.p, a.comp.ratio, a.window);
  k.n_keys = k.n_win + (a.topk ? a.k : k.nv);
  return k;
}

__device__ __forceinline__ float pool_elem(const PoolDev& P, int64_t idx, int d) {
  const uint8_t* row = P.data + idx * P.entry_bytes;
  if (P.dtype == F32) return reinterpret_cast<const float*>(row)[d];
  if (P.dtype == BF16) return bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[d]);
  return fp8_to_f32(row[d]) * reinterpret_cast<const float*>(P.scale)[idx];
}

// ------------------------------------------------------------------------------------------
// Generic kernel: any heads x dims <= 4096, fp32 or bf16 query, fp32 / bf16 / fp8 pools.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_generic(AttnArgs a) {
  extern __shared__ float sm[];
  const int i = blockIdx.y, sp = blockIdx.x;
  const QueryKeys qk = query_keys(a, i);
  const int H = a.n_heads, D = a.dim;
  const int j_begin = sp * a.chunk, j_end = min(qk.n_keys, j_begin + a.chunk);
  float* qs = sm;                    // [H][D]
  float* os = qs + H * D;            // [H][D]
  float* sc = os + H * D;            // [H][kGenTile]
  float* mrow = sc + H * kGenTile;   // [H]
  float* lrow = mrow + H;            // [H]
  float* alph = lrow + H;            // [H]
  __shared__ int64_t kidx[kGenTile];
  __shared__ int kcomp[kGenTile];
  for (int e = threadIdx.x; e < H * D; e += 256) {
    int64_t off = (int64_t)i * H * D + e;
    qs[e] = a.q_dtype == F32 ? reinterpret_cast<const float*>(a.q)[off]
                             : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[off]);
    os[e] = 0.f;
  }
  for (int h = threadIdx.x; h < H; h += 256) {
    mrow[h] = -INFINITY;
    lrow[h] = 0.f;
  }
  __syncthreads();
  for (int j0 = j_begin; j0 < j_end; j0 += kGenTile) {
    const int nt = min(kGenTile, j_end - j0);
    if (threadIdx.x < nt) {
      KeyRef r = resolve_key(a, i, qk.seq, qk.ws, qk.n_win, qk.nv, j0 + threadIdx.x);
      kidx[threadIdx.x] = r.idx;
      kcomp[threadIdx.x] = r.comp;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < H * nt; e += 256) {
      const int h = e / nt, j = e % nt;
      float s = -INFINITY;
      if (kidx[j] >= 0) {
        const PoolDev& P = kcomp[j] ? a.comp : a.swa;
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[h * D + d], pool_elem(P, kidx[j], d), dot);
        s = dot * a.scale;
      }
      sc[h * kGenTile + j] = s;
    }
    __syncthreads();
    for (int h = threadIdx.x; h < H; h += 256) {
      float mx = mrow[h];
      for (int j = 0; j < nt; ++j) mx = fmaxf(mx, sc[h * kGenTile + j]);
      const float ref = mx == -INFINITY ? 0.f : mx;
      const float al = expf(mrow[h] - ref);
      float sum = 0.f;
      for (int j = 0; j < nt; ++j) {
        float pj = expf(sc[h * kGenTile + j] - ref);
        sc[h * kGenTile + j] = pj;
        sum += pj;
      }
      lrow[h] = lrow[h] * al + sum;
      mrow[h] = mx;
      alph[h] = al;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < H * D; e += 256) {
      const int h = e / D, d = e % D;
      float acc = os[e] * alph[h];
      for (int j = 0; j < nt; ++j) {
        if (kidx[j] < 0) continue;
        acc = fmaf(sc[h * kGenTile + j], pool_elem(kcomp[j] ? a.comp : a.swa, kidx[j], d), acc);
      }
      os[e] = acc;
    }
    __syncthreads();
  }
  // partials: o as [dim][head], then m and l per head
  float* po = a.part_o + ((int64_t)i * a.n_split + sp) * D * H;
  for (int e = threadIdx.x; e < H * D; e += 256) {
    const int d = e / H, h = e % H;
    po[e] = os[h * D + d];
  }
  float* pml = a.part_ml + ((int64_t)i * a.n_split + sp) * 2 * H;
  for (int h = threadIdx.x; h < H; h += 256) {
    pml[h] = mrow[h];
    pml[H + h] = lrow[h];
  }
}

// ------------------------------------------------------------------------------------------
// MFMA kernel: 64 heads x 512 dims.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = fp8_to_bf16(w0 & 0xffu) | (fp8_to_bf16((w0 >> 8) & 0xffu) << 16);
  r[1] = fp8_to_bf16((w0 >> 16) & 0xffu) | (fp8_to_bf16(w0 >> 24) << 16);
  r[2] = fp8_to_bf16(w1 & 0xffu) | (fp8_to_bf16((w1 >> 8) & 0xffu) << 16);
  r[3] = fp8_to_bf16((w1 >> 16) & 0xffu) | (fp8_to_bf16(w1 >> 24) << 16);
  return __builtin_bit_cast(bf16x8, r);
}

template <bool kFp8>
__global__ __launch_bounds__(256, 1) void attn_mfma(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kKT * kKRow];
  __shared__ float sx[4][16][64];
  __shared__ float kscale[kKT];
  __shared__ int kvalid[kKT];

  const int i = blockIdx.y, sp = blockIdx.x;
  const QueryKeys qk = query_keys(a, i);
  const int j_begin = sp * a.chunk, j_end = min(qk.n_keys, j_begin + a.chunk);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int hh = wave >> 1, dh = wave & 1;

  // Q^T as the QK B operand: column h = 32*hh + col; dims d = 256*dh + 128*hf + 8*s + e
  bf16x8 qb[16];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) +
                           ((int64_t)i * kMH + 32 * hh + col) * kMD + 256 * dh + 128 * hf;
#pragma unroll
    for (int s = 0; s < 16; ++s) qb[s] = *reinterpret_cast<const bf16x8*>(qrow + 8 * s);
  }
  f32x16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;

  for (int j0 = j_begin; j0 < j_end; j0 += kKT) {
    // ---- this lane's key row: key j0 + col, dims 256*dh + 128*hf + [0, 128)
    const int j = j0 + col;
    KeyRef kr{-1, 0};
    if (j < j_end) kr = resolve_key(a, i, qk.seq, qk.ws, qk.n_win, qk.nv, j);
    const PoolDev& P = kr.comp ? a.comp : a.swa;
    bf16x8 ka[16];
    float ksc = 1.f;
    if (kr.idx >= 0) {
      if constexpr (!kFp8) {
        const uint16_t* row =
            reinterpret_cast<const uint16_t*>(P.data + kr.idx * P.entry_bytes) + 256 * dh + 128 * hf;
#pragma unroll
        for (int s = 0; s < 16; ++s) ka[s] = *reinterpret_cast<const bf16x8*>(row + 8 * s);
      } else {
        const uint8_t* row = P.data + kr.idx * P.entry_bytes + 256 * dh + 128 * hf;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          u32x4 w = *reinterpret_cast<const u32x4*>(row + 16 * s);
          ka[2 * s] = fp8x8_to_bf16x8(w[0], w[1]);
          ka[2 * s + 1] = fp8x8_to_bf16x8(w[2], w[3]);
        }
        ksc = reinterpret_cast<const float*>(P.scale)[kr.idx];
      }
    } else {
#pragma unroll
      for (int s = 0; s < 16; ++s) ka[s] = bf16x8{};
    }
    // ---- QK over this wave's 256 dims
    f32x16 st = {};
#pragma unroll
    for (int s = 0; s < 16; ++s) st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s], qb[s], st, 0, 0, 0);
    // ---- share: partial scores, the K tile (natural layout), key scale and validity
#pragma unroll
    for (int r = 0; r < 16; ++r) sx[wave][r][lane] = st[r];
    if (hf == hh) {
      uint16_t* dst = ktile + col * kKRow + 256 * dh + 128 * hh;
#pragma unroll
      for (int s = 0; s < 16; ++s) *reinterpret_cast<bf16x8*>(dst + 8 * s) = ka[s];
    }
    if (wave == 0 && hf == 0) {
      kscale[col] = ksc;
      kvalid[col] = kr.idx >= 0;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) st[r] += sx[wave ^ 1][r][lane];
    // ---- online softmax for head 32*hh + col; this lane's keys are 8*(r/4) + 4*hf + r%4
    float z[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
      float v = st[r] * sl2;
      if constexpr (kFp8) v *= kscale[key];
      z[r] = kvalid[key] ? v : -INFINITY;
      mx = fmaxf(mx, z[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float ref = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = exp2f(m_run - ref);
    float psum = 0.f;
    float pr[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float e = exp2f(z[r] - ref);
      psum += e;
      if constexpr (kFp8) {
        pr[r] = e * kscale[8 * (r >> 2) + 4 * hf + (r & 3)];
      } else {
        pr[r] = e;
      }
    }
    psum += __shfl_xor(psum, 32, 64);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
    // ---- PV: B operand = probabilities (element e of step t <-> key 16t + 8(e/4) + 4hf + e%4)
    bf16x8 pb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(pr[8 * t + 2 * e], pr[8 * t + 2 * e + 1]);
      pb[t] = __builtin_bit_cast(bf16x8, w);
    }
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const int d = 256 * dh + 32 * mb + col;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k0 = 16 * t + 8 * ((2 * e) >> 2) + 4 * hf + ((2 * e) & 3);
          const int k1 = 16 * t + 8 * ((2 * e + 1) >> 2) + 4 * hf + ((2 * e + 1) & 3);
          w[e] = (uint32_t)ktile[k0 * kKRow + d] | ((uint32_t)ktile[k1 * kKRow + d] << 16);
        }
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pb[t], o[mb],
                                                        0, 0, 0);
      }
    }
    __syncthreads();
  }
  // ---- partials: O^T rows d = 256*dh + 32*mb + 8*(r/4) + 4*hf + r%4, column h = 32*hh + col
  float* po = a.part_o + ((int64_t)i * a.n_split + sp) * kMD * kMH;
  const int h = 32 * hh + col;
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int d = 256 * dh + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3);
      po[d * kMH + h] = o[mb][r];
    }
  if (dh == 0 && hf == 0) {
    float* pml = a.part_ml + ((int64_t)i * a.n_split + sp) * 2 * kMH;
    // m is kept in log2 units inside the kernel; store natural-log units for the combine
    pml[h] = m_run == -INFINITY ? -INFINITY : m_run / kLog2e;
    pml[kMH + h] = l_run;
  }
}

// ------------------------------------------------------------------------------------------
// Combine: merge split partials, inverse RoPE at the query position, cast.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int i = blockIdx.x;
  const int H = a.n_heads, D = a.dim, ns = a.n_split;
  int seq, p;
  query_at(a.qd, i, &seq, &p);
  __shared__ float wsplit[kMaxSplit * 128];
  __shared__ float rc[64], rs[64];
  const float* pml = a.part_ml + (int64_t)i * ns * 2 * H;
  for (int h = threadIdx.x; h < H; h += 256) {
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, pml[s * 2 * H + h]);
    float den = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = pml[s * 2 * H + h];
      den += ms == -INFINITY ? 0.f : expf(ms - M) * pml[s * 2 * H + H + h];
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = pml[s * 2 * H + h];
      wsplit[s * H + h] = ms == -INFINITY ? 0.f : expf(ms - M) * inv;
    }
  }
  const int half = a.rope_dim / 2;
  for (int t = threadIdx.x; t < half; t += 256) rope_cs(-(double)p, t, a.rope_dim, a.rope_base, &rc[t], &rs[t]);
  __syncthreads();
  const float* po = a.part_o + (int64_t)i * ns * D * H;
  const int rope_lo = D - a.rope_dim;
  for (int e = threadIdx.x; e < (D / 2) * H; e += 256) {
    const int h = e % H, d = 2 * (e / H);
    float v0 = 0.f, v1 = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float wgt = wsplit[s * H + h];
      v0 = fmaf(wgt, po[((int64_t)s * D + d) * H + h], v0);
      v1 = fmaf(wgt, po[((int64_t)s * D + d + 1) * H + h], v1);
    }
    if (d >= rope_lo) {
      const int t = (d - rope_lo) >> 1;
      const float z0 = v0 * rc[t] - v1 * rs[t];
      const float z1 = v0 * rs[t] + v1 * rc[t];
      v0 = z0;
      v1 = z1;
    }
    const int64_t off = ((int64_t)i * H + h) * D + d;
    if (a.out_dtype == F32) {
      *reinterpret_cast<float2*>(reinterpret_cast<float*>(a.out) + off) = make_float2(v0, v1);
    } else {
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.out) + off) = pack_bf16x2(v0, v1);
    }
  }
}

AttnPlan plan_attention(int32_t n_q, int32_t n_heads, int32_t dim, int32_t max_keys,
                        int32_t q_dtype, int32_t pool_dtype) {
  AttnPlan pl{};
  pl.use_mfma = n_heads == kMH && dim == kMD && q_dtype == BF16 &&
                (pool_dtype == BF16 || pool_dtype == FP8);
  const int tile = pl.use_mfma ? kKT : kGenTile;
  const int target_blocks = pl.use_mfma ? 256 : 512;
  const int min_chunk = 64;
  int max_split = (max_keys + min_chunk - 1) / min_chunk;
  int ns = n_q > 0 ? (target_blocks + n_q - 1) / n_q : 1;
  ns = ns < 1 ? 1 : ns;
  ns = ns > max_split ? max_split : ns;
  ns = ns > kMaxSplit ? kMaxSplit : ns;
  ns = ns < 1 ? 1 : ns;
  int chunk = (max_keys + ns - 1) / ns;
  chunk = (chunk + tile - 1) / tile * tile;
  if (chunk < tile) chunk = tile;
  ns = (max_keys + chunk - 1) / chunk;
  if (ns < 1) ns = 1;
  pl.n_split = ns;
  pl.chunk = chunk;
  pl.ws_bytes = (size_t)n_q * ns * ((size_t)dim * n_heads + 2 * (size_t)n_heads) * sizeof(float);
  return pl;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  dim3 grid(a.n_split, a.n_q);
  if (a.use_mfma) {
    if (a.swa.dtype == FP8)
      hipLaunchKernelGGL(attn_mfma<true>, grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL(attn_mfma<false>, grid, dim3(256), 0, s, a);
  } else {
    size_t lds = sizeof(float) * ((size_t)2 * a.n_heads * a.dim + (size_t)a.n_heads * kGenTile +
                                  3 * (size_t)a.n_heads);
    hipLaunchKernelGGL(attn_generic, grid, dim3(256), lds, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine, dim3(a.n_q), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hyb
