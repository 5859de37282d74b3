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
#include <type_traits>

#include "common.h"

namespace hyb {

constexpr int kMH = 64;         // heads in the MFMA kernel
constexpr int kMD = 512;        // dims in the MFMA kernel
constexpr int kKT = 32;         // keys per tile in the MFMA kernel
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

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

// Masked keys (past the end of a split, absent blocks, unused top-k slots) load this row instead
// of a pool entry, so their operands are zero without any per-use select. Never written.
__device__ __attribute__((aligned(16))) uint8_t kZeroRow[1024];   // zero-initialised device memory

constexpr int kSeg = 2048;           // keys whose entry indices are resolved per segment
constexpr int kPitch = kMD + 16;     // LDS row pitch of a K tile (bf16): 1056 B, 8 banks per row
constexpr int kQPitch = kMD + 8;     // LDS row pitch of the query (bf16): 1040 B, 4 banks per row

// LDS address (in bf16 elements) of dims [d, d + 8) of key row `row` of a K tile. Rows are 1056 B
// apart (8 banks), and the 16-byte chunk index is XORed with bit 3 of the row: sixteen
// consecutive rows written or read 16 bytes each then cover all 64 banks once, while the
// transposed reads (4 consecutive rows, which share bit 3) keep their conflict-free pattern.
__device__ __forceinline__ int tile_off(int row, int d) {
  return row * kPitch + ((((d >> 3) ^ ((row >> 3) & 1)) << 3) | (d & 7));
}

// One wave's quarter (64 of the 512 dims per lane-half) of one 32-key tile, held in registers
// between its global load and its use.
template <bool kFp8>
struct Stage;
template <>
struct Stage<false> {
  bf16x8 v[8];
  float sc;
  int valid;
};
template <>
struct Stage<true> {
  u32x4 v[4];
  float sc;
  int valid;
};

__device__ __forceinline__ bf16x8 lds_tr_pair(const uint16_t* p0, const uint16_t* p1) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1));
  u32x4 w;
  w[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
  w[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
  w[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
  w[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
  return __builtin_bit_cast(bf16x8, w);
}

// MFMA attention. Work of one workgroup: query i, keys [split*chunk, (split+1)*chunk) of its list.
// Waves form a 2 x 2 grid: hh = head half (32 heads), dh = dim half (256 dims). Wave (hh, dh)
// loads only dim quarter qd = 2*dh + hh of every key (each key byte is fetched once per
// workgroup), three tiles deep in registers; the quarter is written to the LDS tile, where the
// partner wave of the same dim half picks it up for its QK and all waves read it transposed for PV.
template <bool kFp8>
__global__ __launch_bounds__(256, 1) void attn_mfma(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ktile[2 * kKT * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t qlds[kMH * kQPitch];   // the query, [head][dim]
  __shared__ __attribute__((aligned(16))) float sx[4][4 * 64 * 4];   // [wave][quad][lane][4]
  __shared__ int32_t kidx[kSeg];
  __shared__ __attribute__((aligned(16))) float kscale[2 * kKT];

  const int i = blockIdx.y, sp = blockIdx.x;
  const QueryKeys qk = query_keys(a, i);
  const int j_begin = sp * a.chunk, j_end = min(qk.n_keys, j_begin + a.chunk);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int hh = wave >> 1, dh = wave & 1;
  const int qd = 2 * dh + hh;          // the dim quarter this wave loads
  const int oq = 2 * dh + (1 - hh);    // the partner's quarter

  // The query stays in LDS (registers go to the O accumulators and the staged K tiles). Q^T is
  // the QK B operand (column = head 32*hh + col); K-step s covers quarter 2*dh + s/8, dims
  // 128*quarter + 64*hf + 8*(s%8) + [0, 8): the same split the K operand uses.
  {
    const uint16_t* qsrc = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)i * kMH * kMD;
    for (int e = tid; e < kMH * kMD / 8; e += 256) {
      const int h = e / (kMD / 8), d = (e % (kMD / 8)) * 8;
      *reinterpret_cast<bf16x8*>(qlds + h * kQPitch + d) = *reinterpret_cast<const bf16x8*>(qsrc + h * kMD + d);
    }
  }
  const uint16_t* qrow = qlds + (32 * hh + col) * kQPitch + 64 * hf;
  auto qb = [&](int s) -> bf16x8 {
    return *reinterpret_cast<const bf16x8*>(qrow + 128 * (2 * dh + (s >> 3)) + 8 * (s & 7));
  };
  f32x16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  const int lane_off = 128 * qd + 64 * hf;   // first dim of this lane's staged run

  for (int seg = j_begin; seg < j_end; seg += kSeg) {
    const int nseg = min(kSeg, j_end - seg);
    __syncthreads();   // readers of the previous segment's index table are done
    for (int jj = tid; jj < nseg; jj += 256) {
      KeyRef r = resolve_key(a, i, qk.seq, qk.ws, qk.n_win, qk.nv, seg + jj);
      kidx[jj] = (int32_t)r.idx;
    }
    __syncthreads();
    const int n_tiles = (nseg + kKT - 1) / kKT;

    // Loads are issued without any branch (masked lanes read the zero row): a branch between a
    // prefetch and the use of an older tile would make the compiler wait for every outstanding
    // load, prefetch included.
    auto load = [&](Stage<kFp8>& st, int tt) {
      const int jraw = tt * kKT + col;
      const int jl = min(jraw, nseg - 1);
      const int idx = kidx[jl];
      const bool ok = jraw < nseg && idx >= 0;
      const bool win = (seg + jl) < qk.n_win;
      const uint8_t* base = win ? a.swa.data : a.comp.data;
      const int64_t eb = win ? a.swa.entry_bytes : a.comp.entry_bytes;
      const uint8_t* entry = ok ? base + (int64_t)idx * eb : kZeroRow;
      st.valid = ok;
      if constexpr (!kFp8) {
        const uint16_t* row = reinterpret_cast<const uint16_t*>(entry) + lane_off;
#pragma unroll
        for (int c = 0; c < 8; ++c) st.v[c] = *reinterpret_cast<const bf16x8*>(row + 8 * c);
        st.sc = 1.f;
      } else {
        const uint8_t* row = entry + lane_off;
#pragma unroll
        for (int c = 0; c < 4; ++c) st.v[c] = *reinterpret_cast<const u32x4*>(row + 16 * c);
        st.sc = reinterpret_cast<const float*>(win ? a.swa.scale : a.comp.scale)[ok ? idx : 0];
      }
    };

    auto own = [&](const Stage<kFp8>& st, int c) -> bf16x8 {
      if constexpr (!kFp8) {
        return st.v[c];
      } else {
        const u32x4 q = st.v[c >> 1];
        return (c & 1) ? fp8x8_to_bf16x8(q[2], q[3]) : fp8x8_to_bf16x8(q[0], q[1]);
      }
    };

    auto process = [&](const Stage<kFp8>& st, int tt) {
      const int kb = tt & 1;
      uint16_t* kt = ktile + kb * kKT * kPitch;
      // ---- publish this wave's quarter of the tile (natural [key][dim] layout)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<bf16x8*>(kt + tile_off(col, lane_off + 8 * c)) = own(st, c);
      if constexpr (kFp8) {
        if (wave == 0 && hf == 0) kscale[kb * kKT + col] = st.valid ? st.sc : 0.f;
      }
      // validity of the tile's 32 keys (every wave resolved the same keys): bit j = key j
      const uint32_t vmask = (uint32_t)__ballot(st.valid);
      __syncthreads();
      // ---- QK over this wave's dim half: own quarter from registers, partner's from LDS
      bf16x8 oth[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        oth[c] = *reinterpret_cast<const bf16x8*>(kt + tile_off(col, 128 * oq + 64 * hf + 8 * c));
      // two independent accumulation chains (even / odd K-steps) keep the MFMA pipe busy
      f32x16 sacc = {}, sacc1 = {};
#pragma unroll
      for (int s = 0; s < 16; s += 2) {
        const bf16x8 ka0 = ((s >> 3) == hh) ? own(st, s & 7) : oth[s & 7];
        const bf16x8 ka1 = (((s + 1) >> 3) == hh) ? own(st, (s + 1) & 7) : oth[(s + 1) & 7];
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0, qb(s), sacc, 0, 0, 0);
        sacc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qb(s + 1), sacc1, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] += sacc1[r];
      {
        // [wave][quad][lane][4]: a wave's 16-byte accesses are lane-contiguous (no conflicts)
        f32x4* mine = reinterpret_cast<f32x4*>(&sx[wave][0]) + lane;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = sacc[4 * q4 + e];
          mine[64 * q4] = v;
        }
      }
      __syncthreads();
      {
        const f32x4* theirs = reinterpret_cast<const f32x4*>(&sx[wave ^ 1][0]) + lane;
        f32x4 t[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) t[q4] = theirs[64 * q4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
          for (int e = 0; e < 4; ++e) sacc[4 * q4 + e] += t[q4][e];
      }
      // ---- online softmax for head 32*hh + col; this lane's keys are 8*(r/4) + 4*hf + r%4
      float ksc[16];
      if constexpr (kFp8) {
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(kscale + kb * kKT + 8 * j4 + 4 * hf);
#pragma unroll
          for (int e = 0; e < 4; ++e) ksc[4 * j4 + e] = v[e];
        }
      }
      float z[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
        float v = sacc[r] * sl2;
        if constexpr (kFp8) v *= ksc[r];
        z[r] = ((vmask >> key) & 1u) ? v : -INFINITY;
        mx = fmaxf(mx, z[r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // The reference maximum only moves when a score exceeds it by more than 2^8 (or on the
      // first keys): probabilities then stay <= 256, and the O rescale is skipped for the wave
      // unless one of its heads moved. Exact: l and O share the same reference.
      if (__ballot(mx > m_run + 8.f) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[mb][r] *= alpha;
        m_run = m_new;
      }
      const float ref = m_run == -INFINITY ? 0.f : m_run;
      float psum = 0.f;
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(z[r] - ref);
        psum += e;
        if constexpr (kFp8) {
          pr[r] = e * ksc[r];
        } else {
          pr[r] = e;
        }
      }
      psum += __shfl_xor(psum, 32, 64);
      l_run += psum;
      // ---- PV: B = probabilities (element e of K-step t <-> key 16t + 8(e/4) + 4hf + e%4),
      //      A = K^T read transposed from LDS: lane j of each 16-lane group points at key
      //      k0 + j/4, dims d0 + 4*(j%4), and receives keys k0..k0+3 of dim d0 + j.
      bf16x8 pb[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(pr[8 * t2 + 2 * e], pr[8 * t2 + 2 * e + 1]);
        pb[t2] = __builtin_bit_cast(bf16x8, w);
      }
      const int i16 = lane & 15;
      const int trow = 4 * hf + (i16 >> 2);                       // + 16*t2 (+ 8 for the 2nd half)
      const int tdim = 256 * dh + (col >> 4) * 16 + 4 * (i16 & 3);  // + 32*mb
      auto trf = [&](int mb, int t2) {
        return lds_tr_pair(kt + tile_off(trow + 16 * t2, tdim + 32 * mb),
                           kt + tile_off(trow + 16 * t2 + 8, tdim + 32 * mb));
      };
      // fragments for block mb + 1 are read while block mb multiplies
      bf16x8 af[2][2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) af[0][t2] = trf(0, t2);
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        if (mb + 1 < 8) {
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) af[(mb + 1) & 1][t2] = trf(mb + 1, t2);
        }
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
          o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb & 1][t2], pb[t2], o[mb], 0, 0, 0);
      }
    };

    // Global loads run two tiles ahead of the tile being processed (three staged tiles fit
    // beside the O accumulators; the query lives in LDS).
    // (tiles past the end are loaded masked: harmless, and it keeps the loop free of branches
    // between a prefetch and the use of the tile before it)
    {
      Stage<kFp8> s0, s1, s2;
      load(s0, 0);
      load(s1, 1);
      for (int t = 0; t < n_tiles; t += 3) {
        load(s2, t + 2);
        process(s0, t);
        if (t + 1 >= n_tiles) break;
        load(s0, t + 3);
        process(s1, t + 1);
        if (t + 2 >= n_tiles) break;
        load(s1, t + 4);
        process(s2, t + 2);
      }
    }
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
// Grid (dim slice of 64, query): each workgroup reads its 64 dims x all heads of every split.
// ------------------------------------------------------------------------------------------
constexpr int kCombineDims = 32;

__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int i = blockIdx.y;
  const int d0 = blockIdx.x * kCombineDims;
  const int H = a.n_heads, D = a.dim, ns = a.n_split;
  int seq, p;
  query_at(a.qd, i, &seq, &p);
  __shared__ float wsplit[kMaxSplit * 128];
  __shared__ float rc[kCombineDims / 2], rs[kCombineDims / 2];
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
  const int rope_lo = D - a.rope_dim;
  const int dend = min(D, d0 + kCombineDims);
  for (int t = threadIdx.x; t < kCombineDims / 2; t += 256) {
    const int d = d0 + 2 * t;
    if (d >= rope_lo && d < dend)
      rope_cs(-(double)p, (d - rope_lo) >> 1, a.rope_dim, a.rope_base, &rc[t], &rs[t]);
  }
  __syncthreads();
  const float* po = a.part_o + (int64_t)i * ns * D * H;
  const int npair = (dend - d0) / 2;
  for (int e = threadIdx.x; e < npair * H; e += 256) {
    const int h = e % H, t = e / H, d = d0 + 2 * t;
    float v0 = 0.f, v1 = 0.f;
#pragma unroll 8
    for (int s = 0; s < ns; ++s) {
      const float wgt = wsplit[s * H + h];
      v0 = fmaf(wgt, po[((int64_t)s * D + d) * H + h], v0);
      v1 = fmaf(wgt, po[((int64_t)s * D + d + 1) * H + h], v1);
    }
    if (d >= rope_lo) {
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
  if (pl.use_mfma && chunk > kSeg && ns < kMaxSplit) {
    // one index-table segment per workgroup when the split count allows it
    ns = (max_keys + kSeg - 1) / kSeg;
    ns = ns > kMaxSplit ? kMaxSplit : ns;
    chunk = (max_keys + ns - 1) / ns;
    chunk = (chunk + tile - 1) / tile * tile;
  }
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
  hipLaunchKernelGGL(attn_combine, dim3((a.dim + kCombineDims - 1) / kCombineDims, a.n_q), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace hyb
