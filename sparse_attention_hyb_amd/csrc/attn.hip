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

// Two transposed 8-byte LDS reads (ds_read_b64_tr_b16) forming one 8 x bf16 MFMA operand.
__device__ __forceinline__ bf16x8 lds_tr_pair(const uint16_t* p0, const uint16_t* p1) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
  const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0)));
  const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1)));
  const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// The hardware hands consecutive workgroup ids to the 8 XCDs in turn. This maps a workgroup id to
// a logical index so that consecutive logical indices - the splits of one query - run on one XCD
// and share its L2 (the query, and for sparse decode the sequence's entries).
__device__ __forceinline__ int xcd_logical(int L, int total) {
  constexpr int X = 8;
  const int per = total / X, rem = total % X;
  const int x = L % X, s = L / X;
  return x < rem ? x * (per + 1) + s : rem * (per + 1) + (x - rem) * per + s;
}

// MFMA attention. Work of one workgroup: query i, keys [split*chunk, (split+1)*chunk) of its list.
// Waves form a 2 x 2 grid: hh = head half (32 heads), dh = dim half (256 dims). Each wave keeps
// its query slice (32 heads x 256 dims) in registers and loads only dim quarter qd = 2*dh + hh of
// every key (each key byte is fetched once per workgroup), one iteration ahead of its publication
// (one staged tile in registers keeps the kernel free of spills). Tiles pass through three LDS
// buffers, and each loop iteration needs a single barrier:
//   iteration t: S(t) = own QK partial + the partner's (exchanged through double-buffered LDS),
//                publish this wave's quarter of tile t+2, issue the loads of tile t+3,
//                QK partial of tile t+1 (MFMA, independent of the softmax below),
//                softmax of tile t, PV of tile t (K tile read back transposed), barrier.
// At the barrier ending iteration t every wave has finished reading the buffer of tile t, which
// iteration t+1 refills with tile t+3, and the score buffer read in iteration t, which iteration
// t+1 refills with the partials of tile t+2.
template <bool kFp8>
__global__ __launch_bounds__(256, 1) void attn_mfma(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t ktile[3 * kKT * kPitch];
  __shared__ __attribute__((aligned(16))) float sx[2][4][4 * 64 * 4];   // [buf][wave][quad][lane][4]
  __shared__ int32_t kidx[kSeg];
  __shared__ __attribute__((aligned(16))) float kscale[3 * kKT];
  __shared__ uint32_t kvalid[3];   // per tile buffer: bit j = key j of the tile is valid

  const int logical = xcd_logical(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
  const int sp = logical % a.n_split, i = logical / a.n_split;
  const QueryKeys qk = query_keys(a, i);
  const int j_begin = sp * a.chunk, j_end = min(qk.n_keys, j_begin + a.chunk);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int hh = wave >> 1, dh = wave & 1;
  const int qd = 2 * dh + hh;          // the dim quarter this wave loads

  // Q^T is the QK B operand (column = head 32*hh + col); K-step s covers quarter 2*dh + s/8, dims
  // 128*quarter + 64*hf + 8*(s%8) + [0, 8): the same split the K operand uses.
  bf16x8 qreg[16];
  {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)i * kMH + 32 * hh + col) * kMD + 64 * hf;
#pragma unroll
    for (int s = 0; s < 16; ++s)
      qreg[s] = *reinterpret_cast<const bf16x8*>(qrow + 128 * (2 * dh + (s >> 3)) + 8 * (s & 7));
  }
  f32x16 o[8];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) o[mb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = a.scale * kLog2e;
  const int lane_off = 128 * qd + 64 * hf;   // first dim of this lane's staged run

  // LDS addresses in a tile buffer (bf16 elements), tile_off() written out as a per-lane base plus
  // a compile-time offset, so that few address registers stay live. Row col's 16-byte chunk c sits
  // at chunk c ^ x (x = bit 3 of the row): +8 elements for even c, -8 for odd c when x = 1.
  const int x8 = 8 * ((col >> 3) & 1);
  const int qk_even = col * kPitch + 256 * dh + 64 * hf + x8;   // + 128*(s/8) + 8*(s%8), s even
  const int qk_odd = col * kPitch + 256 * dh + 64 * hf - x8;    // ... s odd
  const int pub_even = col * kPitch + lane_off + x8;            // + 8c, c even
  const int pub_odd = col * kPitch + lane_off - x8;             // ... c odd
  // transposed PV reads: rows trow + 16*t2 (bit 3 clear) and trow + 16*t2 + 8 (bit 3 set), dims
  // tdim + 32*mb; in the second row the chunk index is flipped: +8 elements if its bit 0 (bit 3 of
  // tdim) is clear, -8 if set
  const int i16 = lane & 15;
  const int trow = 4 * hf + (i16 >> 2);
  const int tdim = 256 * dh + (col >> 4) * 16 + 4 * (i16 & 3);
  const int pv_lo = trow * kPitch + tdim;
  const int pv_hi = (trow + 8) * kPitch + tdim + (((tdim >> 3) & 1) ? -8 : 8);

  for (int seg = j_begin; seg < j_end; seg += kSeg) {
    const int nseg = min(kSeg, j_end - seg);
    __syncthreads();   // readers of the previous segment's index table and tiles are done
    for (int jj = tid; jj < nseg; jj += 256) {
      KeyRef r = resolve_key(a, i, qk.seq, qk.ws, qk.n_win, qk.nv, seg + jj);
      kidx[jj] = (int32_t)r.idx;
    }
    __syncthreads();
    const int n_tiles = (nseg + kKT - 1) / kKT;

    // Loads are issued without any branch (masked lanes read the zero row): a branch between a
    // prefetch and the use of an older tile would make the compiler wait for every outstanding
    // load, prefetch included. Tiles past the end load masked rows.
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
    // This wave's quarter of tile tt into its buffer (natural [key][dim] layout), with the
    // validity of the tile's 32 keys (bit j = key j; every wave resolved the same keys).
    auto publish = [&](const Stage<kFp8>& st, int tt) {
      uint16_t* kt = ktile + (tt % 3) * (kKT * kPitch);
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<bf16x8*>(kt + ((c & 1) ? pub_odd : pub_even) + 8 * c) = own(st, c);
      const uint32_t vm = (uint32_t)__ballot(st.valid);
      if (wave == 0) {
        if constexpr (kFp8) {
          if (hf == 0) kscale[(tt % 3) * kKT + col] = st.valid ? st.sc : 0.f;
        }
        if (lane == 0) kvalid[tt % 3] = vm;
      }
    };
    // QK over this wave's dim half, both quarters read from the tile's buffer; two independent
    // accumulation chains (even / odd K-steps) keep the MFMA pipe busy.
    auto qk_partial = [&](int tt) -> f32x16 {
      const uint16_t* kt = ktile + (tt % 3) * (kKT * kPitch);
      f32x16 acc0 = {}, acc1 = {};
#pragma unroll
      for (int s = 0; s < 16; s += 2) {
        const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(kt + qk_even + 128 * (s >> 3) + 8 * (s & 7));
        const bf16x8 k1 =
            *reinterpret_cast<const bf16x8*>(kt + qk_odd + 128 * ((s + 1) >> 3) + 8 * ((s + 1) & 7));
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qreg[s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qreg[s + 1], acc1, 0, 0, 0);
      }
      return acc0 + acc1;
    };
    // [buf][wave][quad][lane][4]: a wave's 16-byte accesses are lane-contiguous (no conflicts)
    auto write_sx = [&](int tt, const f32x16& v) {
      f32x4* mine = reinterpret_cast<f32x4*>(&sx[tt & 1][wave][0]) + lane;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = v[4 * q4 + e];
        mine[64 * q4] = w;
      }
    };
    auto read_sx = [&](int tt) -> f32x16 {
      const f32x4* theirs = reinterpret_cast<const f32x4*>(&sx[tt & 1][wave ^ 1][0]) + lane;
      f32x16 v;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 w = theirs[64 * q4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * q4 + e] = w[e];
      }
      return v;
    };
    // Online softmax of tile tt for head 32*hh + col (this lane's keys are 8*(r/4) + 4*hf + r%4),
    // then PV over the tile.
    auto soft_pv = [&](const f32x16& S, int tt) {
      const uint16_t* kt = ktile + (tt % 3) * (kKT * kPitch);
      const uint32_t vmask = kvalid[tt % 3];
      float ksc[16];
      if constexpr (kFp8) {
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(kscale + (tt % 3) * kKT + 8 * j4 + 4 * hf);
#pragma unroll
          for (int e = 0; e < 4; ++e) ksc[4 * j4 + e] = v[e];
        }
      }
      float z[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
        float v = S[r] * sl2;
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
      // PV: B = probabilities (element e of K-step t2 <-> key 16*t2 + 8(e/4) + 4hf + e%4),
      //     A = K^T read transposed from LDS: lane j of each 16-lane group points at key
      //     k0 + j/4, dims d0 + 4*(j%4), and receives keys k0..k0+3 of dim d0 + j.
      bf16x8 pb[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(pr[8 * t2 + 2 * e], pr[8 * t2 + 2 * e + 1]);
        pb[t2] = __builtin_bit_cast(bf16x8, w);
      }
      auto trf = [&](int mb, int t2) {
        return lds_tr_pair(kt + pv_lo + 16 * t2 * kPitch + 32 * mb,
                           kt + pv_hi + 16 * t2 * kPitch + 32 * mb);
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

    // One tile is in flight in registers; the tile after it is already in its LDS buffer.
    Stage<kFp8> s0;
    load(s0, 0);
    publish(s0, 0);
    load(s0, 1);
    __syncthreads();
    f32x16 sown = qk_partial(0);
    write_sx(0, sown);
    publish(s0, 1);
    load(s0, 2);
    __syncthreads();
    // iteration t; X holds tile t+2, whose buffer was last read in iteration t-1
    auto iter = [&](int t, Stage<kFp8>& X) {
      const f32x16 S = sown + read_sx(t);
      publish(X, t + 2);
      load(X, t + 3);
      f32x16 snext = {};
      if (t + 1 < n_tiles) {
        snext = qk_partial(t + 1);
        write_sx(t + 1, snext);
      }
      soft_pv(S, t);
      sown = snext;
      __syncthreads();
    };
    for (int t = 0; t < n_tiles; ++t) iter(t, s0);
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
// Workgroup (dim slice of 32, query), mapped to the XCD that ran the query's splits so that their
// partials are read from its L2. Thread t owns dims d0 + 2(t/16) + {0, 1} of heads 4(t%16) + [0, 4):
// per split two 16-byte loads (the partials are [dim][head], heads contiguous), all issued before
// any is used.
// ------------------------------------------------------------------------------------------
constexpr int kCombineDims = 32;
constexpr int kCombineHeads = 64;   // heads of either attention kernel

__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int logical = xcd_logical(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
  const int i = logical / gridDim.x;
  const int d0 = (logical % gridDim.x) * kCombineDims;
  const int H = a.n_heads, D = a.dim, ns = a.n_split;
  int seq, p;
  query_at(a.qd, i, &seq, &p);
  __shared__ __attribute__((aligned(16))) float wsplit[kMaxSplit * kCombineHeads];   // [split][head]
  __shared__ float ml[kMaxSplit * 2 * kCombineHeads];   // (m, l) staged as [split][2][head]
  __shared__ float rc[kCombineDims / 2], rs[kCombineDims / 2];
  const int tid = threadIdx.x;
  {
    const float* pml = a.part_ml + (int64_t)i * ns * 2 * H;
    for (int e = tid; e < ns * 2 * H; e += 256) ml[e] = pml[e];
  }
  const int rope_lo = D - a.rope_dim;
  const int dend = min(D, d0 + kCombineDims);
  for (int t = tid; t < kCombineDims / 2; t += 256) {
    const int d = d0 + 2 * t;
    if (d >= rope_lo && d < dend)
      rope_cs(-(double)p, (d - rope_lo) >> 1, a.rope_dim, a.rope_base, &rc[t], &rs[t]);
  }
  __syncthreads();
  for (int h = tid; h < H; h += 256) {
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[s * 2 * H + h]);
    float den = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = ml[s * 2 * H + h];
      den += ms == -INFINITY ? 0.f : expf(ms - M) * ml[s * 2 * H + H + h];
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = ml[s * 2 * H + h];
      wsplit[s * H + h] = ms == -INFINITY ? 0.f : expf(ms - M) * inv;
    }
  }
  __syncthreads();
  const float* po = a.part_o + (int64_t)i * ns * D * H;
  auto store = [&](int h, int d, float x0, float x1, int pr) {
    if (d >= rope_lo) {
      const float z0 = x0 * rc[pr] - x1 * rs[pr];
      const float z1 = x0 * rs[pr] + x1 * rc[pr];
      x0 = z0;
      x1 = z1;
    }
    const int64_t off = ((int64_t)i * H + h) * D + d;
    if (a.out_dtype == F32) {
      *reinterpret_cast<float2*>(reinterpret_cast<float*>(a.out) + off) = make_float2(x0, x1);
    } else {
      *reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(a.out) + off) = pack_bf16x2(x0, x1);
    }
  };
  if ((H & 3) == 0) {
    // thread t: dim pair d0 + 2(t/16), heads 4(t%16) + [0, 4)
    const int pr = tid >> 4, h4 = 4 * (tid & 15);
    const int d = d0 + 2 * pr;
    if (h4 >= H || d >= dend) return;
    f32x4 v0 = {}, v1 = {};
    for (int s0 = 0; s0 < ns; s0 += 8) {
      f32x4 x0[8], x1[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int s = min(s0 + q, ns - 1);
        x0[q] = *reinterpret_cast<const f32x4*>(po + ((int64_t)s * D + d) * H + h4);
        x1[q] = *reinterpret_cast<const f32x4*>(po + ((int64_t)s * D + d + 1) * H + h4);
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const f32x4 wq = s0 + q < ns ? *reinterpret_cast<const f32x4*>(wsplit + (s0 + q) * H + h4)
                                     : f32x4{};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v0[e] = fmaf(wq[e], x0[q][e], v0[e]);
          v1[e] = fmaf(wq[e], x1[q][e], v1[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) store(h4 + e, d, v0[e], v1[e], pr);
  } else {
    // any head count: one (head, dim pair) per thread and step
    const int npair = (dend - d0) / 2;
    for (int e = tid; e < npair * H; e += 256) {
      const int h = e % H, pr = e / H, d = d0 + 2 * pr;
      float x0 = 0.f, x1 = 0.f;
      for (int s = 0; s < ns; ++s) {
        const float wgt = wsplit[s * H + h];
        x0 = fmaf(wgt, po[((int64_t)s * D + d) * H + h], x0);
        x1 = fmaf(wgt, po[((int64_t)s * D + d + 1) * H + h], x1);
      }
      store(h, d, x0, x1, pr);
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
