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
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "compress_dev.h"
#include "select_dev.h"

namespace hyb {

constexpr int kMH = 64;         // heads in the MFMA kernel
constexpr int kMD = 512;        // dims in the MFMA kernel
constexpr int kKT = 32;         // keys per tile in the MFMA kernel
constexpr int kGenTile = 64;    // keys per tile in the generic kernel
constexpr int kMaxSplit = 64;
constexpr int kBalancedSlots = 256;         // balanced plan: slots beyond one per query
constexpr int kBalancedMaxQueries = 2048;   // balanced plan: queries per launch at most
constexpr int kBalancedMinTiles = 4;        // balanced plan: 32-key tiles per piece at least
constexpr int kShareCands = 8;              // balanced plan: piece sizes tried at once
constexpr int kMaxRopePairs = 64;   // rope_dim <= 128
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

// The keys of a query at sequence seq, position p.
__device__ __forceinline__ QueryKeys query_keys_at(const AttnArgs& a, int seq, int p) {
  QueryKeys k;
  k.seq = seq;
  k.p = p;
  k.ws = window_start(k.p, a.window);
  k.n_win = k.p - k.ws + 1;
  k.nv = n_visible(k.p, a.comp.ratio, a.window);
  k.n_keys = k.n_win + ((a.topk || a.sel.pairs) ? a.k : k.nv);
  return k;
}

__device__ __forceinline__ QueryKeys query_keys(const AttnArgs& a, int i) {
  QueryKeys k;
  query_at(a.qd, i, &k.seq, &k.p);
  k.ws = window_start(k.p, a.window);
  k.n_win = k.p - k.ws + 1;
  k.nv = n_visible(k.p, a.comp.ratio, a.window);
  k.n_keys = k.n_win + ((a.topk || a.sel.pairs) ? a.k : k.nv);
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
  // partials: o / l as [head][dim] (zero for a split without keys), then m and l per head
  float* po = reinterpret_cast<float*>(a.part_o) + ((int64_t)i * a.n_split + sp) * D * H;
  for (int e = threadIdx.x; e < H * D; e += 256) {
    const float l = lrow[e / D];
    po[e] = l > 0.f ? os[e] / l : 0.f;
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
// Eight E4M3 codes (two words, element 0 in the low byte) -> eight bf16 values, exactly: gfx950's
// scaled conversion with scale 1, two codes of one 16-bit half per instruction (it matches the
// arithmetic widening for every non-NaN code; E4M3 NaN is never stored).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  return __builtin_bit_cast(bf16x8, r);
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;

// Masked keys (past the end of a split, absent blocks, unused top-k slots) load this row instead
// of a pool entry, so their operands are zero without any per-use select. Never written.
__device__ __attribute__((aligned(16))) uint8_t kZeroRow[1024];   // zero-initialised device memory

constexpr int kSeg = 2048;           // keys whose entry indices are resolved per segment
constexpr int kRow = kMD;            // LDS row of a K tile: 512 bf16 = 1024 B, no padding
constexpr int kTileElems = kKT * kRow;
constexpr int kPPitch = 40;          // bf16 per head row of a probability tile (80 B)

// K tiles sit in LDS as [key][dim] rows of 1024 B (64 chunks of 16 B, 4 chunks per bank sweep).
// Chunk c of row r is stored at chunk c ^ swz(r), swz(r) = 4*(r%4) + (r/4)%4, which keeps both
// access patterns free of bank conflicts: 16 consecutive rows reading one chunk (score operands
// and stores) hit 16 different 4-bank groups, and 4 consecutive rows reading 4 consecutive
// chunks (transposed reads for the value operand) hit 16 different groups as well.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// Two transposed 8-byte LDS reads (ds_read_b64_tr_b16) forming one 8 x bf16 MFMA operand.
__device__ __forceinline__ bf16x8 lds_tr_pair(const uint16_t* p0, const uint16_t* p1) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0)));
  const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p1)));
  const u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, w);
}

// Reductions over the four 16-lane rows of a wave (lanes with equal lane % 16), without LDS.
// v_permlane16_swap / v_permlane32_swap exchange rows between their two operands; with both
// operands holding x, the two results are rows {0,0,2,2} and {1,1,3,3} (resp. {lo,lo}, {hi,hi}).
// Compiler pitfalls avoided here: the returned pair is read into two scalars (built into a
// two-element vector, or bit-cast to one, the optimiser reads its first element twice), and the
// second operand is an opaque copy so that the two results are never taken to be equal.
template <bool kRow32>
__device__ __forceinline__ void swap_rows(float x, float& r0, float& r1) {
  const uint32_t a = __builtin_bit_cast(uint32_t, x);
  uint32_t b = a;
  asm volatile("" : "+v"(b));
  uint32_t u0, u1;
  if constexpr (kRow32) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    u0 = r[0];
    u1 = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    u0 = r[0];
    u1 = r[1];
  }
  r0 = __builtin_bit_cast(float, u0);
  r1 = __builtin_bit_cast(float, u1);
}
__device__ __forceinline__ float rows_max(float x) {
  float a, b;
  swap_rows<false>(x, a, b);
  swap_rows<true>(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float rows_sum(float x) {
  float a, b;
  swap_rows<false>(x, a, b);
  swap_rows<true>(a + b, a, b);
  return a + b;
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

// Balanced decode plan, formed alike by every workgroup of the launch (all 512 threads call it).
// Query q has tiles_q = ceil(n_keys_q / 32) key tiles; with T = sum_q tiles_q and M = max_q tiles_q,
// pieces hold share = max(kBalancedMinTiles, ceil(T / (n_slots - n_q)), ceil(M / n_split)) tiles,
// so query q takes ns_q = ceil(tiles_q / share) <= n_split pieces and sum_q ns_q <= T / share + n_q
// <= n_slots: one slot per piece. Slots go out in query order (query q: slots first_q .. first_q +
// ns_q - 1). Workgroup `bid` takes slot w = xcd_logical(bid, total) when bid < total (so the used
// slots spread evenly over the XCDs and a query's pieces share one XCD), and returns false
// otherwise. Its query i, piece and key range [j_begin, j_end) (j_end not yet clamped to the
// query's keys). The first piece's workgroup records (first_q, ns_q) in qplan for the combine.
// qk: query i's keys (its position kept in LDS from the plan: no second read of its length).
// lds: 3 n_q + 27 words.
__device__ __forceinline__ bool balanced_piece(const AttnArgs& a, int bid, uint32_t* lds, int& i,
                                               int& piece, int& j_begin, int& j_end, int& w,
                                               QueryKeys& qk) {
  const int tid = threadIdx.x, lane = tid & 63, nq = a.n_q;
  uint32_t* first_s = lds;                            // [nq + 1]
  int* seq_s = reinterpret_cast<int*>(lds + nq + 1);  // [nq]
  int* pos_s = seq_s + nq;                            // [nq]
  uint32_t* wt = lds + 3 * nq + 1;                    // [16] wave totals of the scan
  uint32_t* red = wt + 16;                            // [2] T, M, [8] piece counts
  uint32_t t4[4], sum = 0, mx = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {   // queries 4 tid .. 4 tid + 3 (n_q <= 2048)
    const int q = 4 * tid + e;
    uint32_t t = 0u;
    if (q < nq) {
      int seq, p;
      query_at(a.qd, q, &seq, &p);
      seq_s[q] = seq;
      pos_s[q] = p;
      t = (uint32_t)((query_keys_at(a, seq, p).n_keys + kKT - 1) / kKT);
    }
    t4[e] = t;
    sum += t;
    mx = max(mx, t);
  }
  if (tid == 0) red[0] = red[1] = 0u;
  __syncthreads();
  const uint32_t wsum = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(sum), 63);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
  if (lane == 0) {
    atomicAdd(&red[0], wsum);
    atomicMax(&red[1], mx);
  }
  __syncthreads();
  const uint32_t T = red[0], M = red[1];
  const uint32_t free_slots = (uint32_t)(a.n_slots - nq);
  const uint32_t share0 = max(max((uint32_t)kBalancedMinTiles, (T + free_slots - 1) / free_slots),
                              (M + (uint32_t)a.n_split - 1) / (uint32_t)a.n_split);
  // share0 bounds the pieces by T / share0 + n_q <= n_slots, but the pieces beyond one per compute
  // unit (kBalancedSlots of them, one workgroup each) would run as a second round. When they do not
  // fit, of kShareCands piece sizes from share0 up to one whose bound is kBalancedSlots
  // (T / (kBalancedSlots - n_q)), the smallest whose actual piece count fits is taken (the largest
  // when none does).
  uint32_t share = share0;
  uint32_t ns4[4], loc = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ns4[e] = (t4[e] + share - 1) / share;
    loc += ns4[e];
  }
  uint32_t total = 0;
  uint32_t run = block_scan_excl<512>(loc, wt, &total);
  const uint32_t room = nq < kBalancedSlots ? (uint32_t)(kBalancedSlots - nq) : 1u;
  const uint32_t share_hi = max(share0, (T + room - 1) / room);
  if (total > (uint32_t)kBalancedSlots && share_hi > share0) {   // uniform
    if (tid < kShareCands) red[2 + tid] = 0u;
    __syncthreads();
#pragma unroll 1
    for (int c = 1; c < kShareCands; ++c) {
      const uint32_t cand = share0 + ((share_hi - share0) * (uint32_t)c + kShareCands - 2) / (kShareCands - 1);
      uint32_t cnt = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) cnt += (t4[e] + cand - 1) / cand;
      cnt = (uint32_t)__builtin_amdgcn_readlane((int)wave_inclusive_scan(cnt), 63);
      if (lane == 0) atomicAdd(&red[2 + c], cnt);
    }
    __syncthreads();
    share = share_hi;
    for (int c = kShareCands - 1; c >= 1; --c)
      if (red[2 + c] <= (uint32_t)kBalancedSlots)
        share = share0 + ((share_hi - share0) * (uint32_t)c + kShareCands - 2) / (kShareCands - 1);
    loc = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ns4[e] = (t4[e] + share - 1) / share;
      loc += ns4[e];
    }
    run = block_scan_excl<512>(loc, wt, &total);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int q = 4 * tid + e;
    if (q < nq) first_s[q] = run;
    run += ns4[e];
  }
  if (tid == 0) first_s[nq] = total;
  __syncthreads();
  if (bid >= (int)total) return false;   // uniform
  w = xcd_logical(bid, (int)total);
  int lo = 0, hi = nq - 1;             // last query whose first slot is <= w (every ns_q >= 1)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int)first_s[mid] <= w) lo = mid; else hi = mid - 1;
  }
  i = lo;
  qk = query_keys_at(a, seq_s[lo], pos_s[lo]);
  piece = w - (int)first_s[lo];
  j_begin = piece * (int)share * kKT;
  j_end = j_begin + (int)share * kKT;
  if (piece == 0 && tid == 0) {
    a.qplan[2 * i] = (int32_t)first_s[lo];
    a.qplan[2 * i + 1] = (int32_t)(first_s[lo + 1] - first_s[lo]);
  }
  return true;
}


// A value pinned to scalar registers: the optimiser can no longer trace it back to the kernel's
// argument segment.
template <typename T>
__device__ __forceinline__ T in_sgpr(T v) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "one or two scalar registers");
  if constexpr (sizeof(T) == 8) {
    uint64_t u = __builtin_bit_cast(uint64_t, v);
    asm volatile("" : "+s"(u));
    return __builtin_bit_cast(T, u);
  } else {
    uint32_t u = __builtin_bit_cast(uint32_t, v);
    asm volatile("" : "+s"(u));
    return __builtin_bit_cast(T, u);
  }
}

// The fields of the window pool (w*) and the compressed pool (c*) that a lane chooses between per
// key. A per-lane choice between two fields of the kernel argument is otherwise compiled into a
// vector load from the argument segment at a per-lane address, and the wait for that load also
// waits for every tile load in flight, which empties the load pipeline on every tile. The
// compressed pool's data and scales are reached as byte offsets from the window pool's, so that
// every address still derives from a kernel-argument pointer (global memory: loads stay global
// loads, counted by the vector-memory counter alone).
struct KeyPools {
  int64_t cd_off;        // a.comp.data - a.swa.data, bytes
  int64_t csc_off;       // a.comp.scale - a.swa.scale, bytes (fp8 pools)
  int64_t web, ceb;
  const int32_t* wbt;
  const int32_t* cbt;
  int wper, cper, wmb, cmb, wnb, cnb;
};
__device__ __forceinline__ KeyPools key_pools(const AttnArgs& a) {
  KeyPools k;
  k.cd_off = in_sgpr((int64_t)((uintptr_t)a.comp.data - (uintptr_t)a.swa.data));
  k.csc_off = in_sgpr((int64_t)((uintptr_t)a.comp.scale - (uintptr_t)a.swa.scale));
  k.web = in_sgpr(a.swa.entry_bytes);
  k.ceb = in_sgpr(a.comp.entry_bytes);
  k.wbt = a.swa.block_table;
  k.cbt = a.comp.block_table;
  k.wper = in_sgpr(a.swa.per_block);
  k.cper = in_sgpr(a.comp.per_block);
  k.wmb = in_sgpr(a.swa.max_blocks);
  k.cmb = in_sgpr(a.comp.max_blocks);
  k.wnb = in_sgpr(a.swa.num_blocks);
  k.cnb = in_sgpr(a.comp.num_blocks);
  return k;
}

// One thread's share of one 32-key tile between its global load and its LDS store: key t/16,
// chunks t%16 + 16c (c < 4) of the row (bf16: 16 B each; fp8: 8 codes each).
template <bool kFp8>
struct Stage;
template <>
struct Stage<false> {
  bf16x8 v[4];
  float sc;
};
template <>
struct Stage<true> {
  u32x2 v[4];
  float sc;
};

// MFMA attention. Work of one workgroup: query i, keys [split*chunk, (split+1)*chunk) of its list.
// Eight waves, two per SIMD, in two roles:
//   score waves 0..3: wave q owns heads 16q..16q+15. S^T[key][h] = sum_d K[key][d] Q[h][d] on
//        v_mfma_f32_16x16x32_bf16 (two 16-key blocks x 16 steps of 32 dims, query in registers,
//        keys from the LDS tile), then the online softmax of those heads; the probabilities go to
//        LDS as bf16 [head][key], with the factor that rescales the running output.
//   value waves 4..7: wave (hh, dh) owns O^T for dims 256dh..+256 x heads 32hh..+32.
//        O^T[d][h] += sum_key K^T[d][key] P^T[key][h] on v_mfma_f32_32x32x16_bf16, the K tile (the
//        same bytes as the values) read back transposed.
// All eight waves load the tiles: each thread carries its share of three tiles in registers
// (loads are issued three tiles ahead of their store to LDS). Tiles rotate through three LDS
// buffers and probabilities through two, with one barrier per tile:
//   iteration t: store tile t+2 and issue the loads of tile t+5; score waves: scores and softmax
//                of tile t+1; value waves: PV of tile t; barrier.
// The buffer stored in iteration t held tile t-1, last read by PV in iteration t-1; the
// probability buffer written in iteration t was last read in iteration t-1.
// fp8 pools: codes are widened to bf16 exactly; the per-entry scale multiplies the score before
// the softmax and the probability before PV (so no rounding of scaled values).
// kSel: the decode step's form, which selects each query's top k itself from the indexer's
// hand-off (every workgroup of the query, before its keys are resolved; see select_finish) and
// clears the row's bin counts for the next call once all of the query's workgroups have read them.
// Workgroups from n_split x n_q on run the compressor calls c0 (n_c0 of them), then c1.
template <bool kFp8, bool kDirect, bool kSel>
__global__ __launch_bounds__(512, 1) void attn_mfma(AttnArgs a, CompressArgs c0, CompressArgs c1,
                                                    int n_c0, int n_c1) {
  __shared__ __attribute__((aligned(16))) uint16_t ktile[3 * kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t ptile[2 * kMH * kPPitch];
  __shared__ __attribute__((aligned(16))) float alpha_s[2 * kMH];
  __shared__ uint32_t rflag[2 * 4];
  __shared__ int32_t kidx[kSeg];
  __shared__ uint32_t tmask[kSeg / kKT];   // per tile of the segment: bit j = key j is valid
  __shared__ __attribute__((aligned(16))) float kscale[3 * kKT];
  __shared__ float lfin[kMH];
  __shared__ float2 orope[kMaxRopePairs];   // RoPE(-p) table of the one-split output
  __shared__ int32_t lsel[kSel ? kMaxTopK : 1];   // the query's selected compressed entries
  __shared__ uint32_t last_reader;
  static_assert(sizeof(ktile) >= kCompressFusedLds, "a compressor workgroup fits the tile buffers");
  static_assert(!kSel || sizeof(ktile) >= kSelLdsWords * sizeof(uint32_t), "the selection fits the tile buffers");

  const bool balanced = !kSel && a.qplan != nullptr;   // uniform
  const int n_attn = balanced ? a.n_slots : a.n_split * a.n_q;
  const int bid = blockIdx.x + blockIdx.y * gridDim.x;
  if (bid >= n_attn) {   // compressor workgroups riding along (first four waves; all take barriers)
    const int k = bid - n_attn;
    if (k < n_c0) compress_fused<4>(c0, k, reinterpret_cast<float*>(ktile));
    else compress_fused<4>(c1, k - n_c0, reinterpret_cast<float*>(ktile));
    return;
  }
  // the query, its piece (split) and the piece's key range; slot: where the partial goes
  int i, sp, j_begin, j_end, slot;
  QueryKeys qk;
  if (balanced) {
    if (!balanced_piece(a, bid, reinterpret_cast<uint32_t*>(ktile), i, sp, j_begin, j_end, slot, qk))
      return;
    __syncthreads();   // the plan's LDS words are read before the tiles reuse them
  } else {
    const int logical = xcd_logical(bid, n_attn);
    sp = logical % a.n_split;
    i = logical / a.n_split;
    j_begin = sp * a.chunk;
    j_end = j_begin + a.chunk;
    slot = i * a.n_split + sp;
  }
  SelRegs sreg;
  if constexpr (kSel) select_issue(a.sel, i, sreg);   // the hand-off loads go out first
  const KeyPools kp = key_pools(a);
  if (!balanced) qk = query_keys(a, i);
  j_end = min(qk.n_keys, j_end);
  const int tid = threadIdx.x;
  if constexpr (!kDirect) {
    // the query's RoPE(-p) table for the combine, formed by its first split's last wave while the
    // first loads are in flight (the combine then starts without this dependent chain)
    if (sp == 0 && a.rope_tab != nullptr && tid >= 448 && tid - 448 < (a.rope_dim >> 1)) {
      float* t = a.rope_tab + ((int64_t)i * kMaxRopePairs + (tid - 448)) * 2;
      rope_cs(-(double)qk.p, tid - 448, a.rope_dim, a.rope_base, t, t + 1);
    }
  }
  if constexpr (kSel) {
    // Every workgroup of the query selects (the first one also writes the top-k row out); one with
    // no keys of its own (j_begin >= n_keys, uniform) does not. Then each counts itself as done
    // reading the row's bin counts - the selection's first scan has consumed them - and the last
    // one clears them at the end.
    if (j_begin < qk.n_keys)
      select_finish(a.sel, i, qk.nv, a.k, reinterpret_cast<uint32_t*>(ktile), lsel,
                    sp == 0 && a.sel.out != nullptr, sreg);
    if (tid == 0) last_reader = atomicAdd(a.sel.row_done + i, 1u) == (uint32_t)(a.n_split - 1) ? 1u : 0u;
  }
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool scorer = wave < 4;
  const float sl2 = a.scale * kLog2e;

  // loader: key lk of a tile, chunks lp + 16c
  const int lk = tid >> 4, lp = tid & 15;
  const int st_base = lk * kRow + 8 * (lp ^ swz(lk));   // + 128*c elements

  // score waves: head 16*wave + sh, keys 16b + 4*sg + r of the tile
  const int sh = lane & 15, sg = lane >> 4;
  // value waves
  const int vw = wave - 4;
  const int hh = (vw >> 1) & 1, dh = vw & 1;
  const int col = lane & 31, hf = lane >> 5, i16 = lane & 15;

  // The two roles run separate copies of the tile loop (same loads, stores and barriers), so that
  // neither keeps the other's state (query registers, output accumulators) live.
  auto role = [&](auto score_role) {
  constexpr bool kScore = decltype(score_role)::value;
  bf16x8 qreg[16];
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 o[8];
  if constexpr (!kScore) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) o[mb] = f32x16{};
  }

  for (int seg = j_begin; seg < j_end; seg += kSeg) {
    const int nseg = min(kSeg, j_end - seg);
    const int n_tiles = (nseg + kKT - 1) / kKT;
    __syncthreads();   // every reader of the previous segment's tables and tiles is done
    {
      // Entry index of every key of the segment (-1 = masked), with its loads batched: each
      // thread issues the top-k reads of its (up to four) keys, then their block-table reads, so
      // the whole table costs two dependent global round trips. Every load is in bounds
      // (clamped indices); masked keys discard the value read.
      constexpr int kR = kSeg / 512;
      const int nres = n_tiles * kKT;
      int g[kR];
      bool win[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const int j = seg + r * 512 + tid;
        win[r] = j < qk.n_win;
        g[r] = win[r] ? qk.ws + j : j - qk.n_win;   // window position or compressed slot
      }
      if (kSel || a.topk != nullptr) {
        int tv[kR];
#pragma unroll
        for (int r = 0; r < kR; ++r) {
          const int c = min(max(g[r], 0), a.k - 1);
          tv[r] = kSel ? lsel[c] : a.topk[(int64_t)i * a.k + c];
        }
#pragma unroll
        for (int r = 0; r < kR; ++r)
          if (!win[r]) g[r] = tv[r];
      }
      int lb[kR], phys[kR];
      bool lok[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const bool w = win[r];
        const int per = w ? kp.wper : kp.cper;
        const bool gok = r * 512 + tid < nseg && g[r] >= 0 && (w || g[r] < qk.nv);
        lb[r] = gok ? g[r] / per : 0;
        lok[r] = gok && lb[r] < (w ? kp.wmb : kp.cmb);
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const bool w = win[r];
        const int mbk = w ? kp.wmb : kp.cmb;
        const int64_t off = (int64_t)qk.seq * mbk + (lok[r] ? lb[r] : 0);
        phys[r] = w ? kp.wbt[off] : kp.cbt[off];
      }
      int idxr[kR];
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        const bool w = win[r];
        const int per = w ? kp.wper : kp.cper;
        const int nbk = w ? kp.wnb : kp.cnb;
        idxr[r] = (lok[r] && phys[r] >= 0 && phys[r] < nbk) ? phys[r] * per + (g[r] - lb[r] * per) : -1;
        if (lok[r] && phys[r] >= nbk) {
          uint32_t* err = w ? a.swa.err : a.comp.err;   // rare: a corrupt table entry
          if (err != nullptr) atomicOr(err, kErrBadPage);
        }
      }
#pragma unroll
      for (int r = 0; r < kR; ++r) {
        if (r * 512 >= nres) continue;
        const int jj = r * 512 + tid;
        kidx[jj] = idxr[r];
        const uint64_t vb = __ballot(idxr[r] >= 0);   // keys r*512 + 64*wave + [0, 64): two tiles
        if (lane == 0) {
          tmask[jj / kKT] = (uint32_t)vb;
          tmask[jj / kKT + 1] = (uint32_t)(vb >> 32);
        }
      }
    }
    __syncthreads();

    // Loads are issued without any branch (masked keys read the zero row): a branch between a
    // prefetch and the use of an older tile would make the compiler wait for every outstanding
    // load, prefetch included. Tiles past the end load masked rows.
    auto load = [&](Stage<kFp8>& st, int tt) {
      const int jraw = tt * kKT + lk;
      const int jl = min(jraw, nseg - 1);
      const int idx = kidx[jl];
      const bool ok = jraw < nseg && idx >= 0;
      const bool win = (seg + jl) < qk.n_win;
      const int64_t eb = win ? kp.web : kp.ceb;
      const uint8_t* entry = ok ? a.swa.data + ((win ? 0 : kp.cd_off) + (int64_t)idx * eb) : kZeroRow;
      // Decode launches read every entry once (nontemporal: streamed past the caches, which a
      // row-gather probe measured 11-15 % faster than plain loads); the one-split form also
      // serves prefill, where the queries of a sequence re-read the same entries from cache.
      if constexpr (!kFp8) {
        const uint16_t* row = reinterpret_cast<const uint16_t*>(entry) + 8 * lp;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x4* src = reinterpret_cast<const u32x4*>(row + 128 * c);
          st.v[c] = __builtin_bit_cast(bf16x8, kDirect ? *src : __builtin_nontemporal_load(src));
        }
        st.sc = 1.f;
      } else {
        const uint8_t* row = entry + 8 * lp;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const u32x2* src = reinterpret_cast<const u32x2*>(row + 128 * c);
          st.v[c] = kDirect ? *src : __builtin_nontemporal_load(src);
        }
        const float s = *reinterpret_cast<const float*>(
            reinterpret_cast<const uint8_t*>(a.swa.scale) + ((win ? 0 : kp.csc_off) + 4 * (int64_t)(ok ? idx : 0)));
        st.sc = ok ? s : 0.f;
      }
    };
    auto publish = [&](const Stage<kFp8>& st, int tt) {
      uint16_t* kt = ktile + (tt % 3) * kTileElems + st_base;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (!kFp8) {
          *reinterpret_cast<bf16x8*>(kt + 128 * c) = st.v[c];
        } else {
          *reinterpret_cast<bf16x8*>(kt + 128 * c) = fp8x8_to_bf16x8(st.v[c][0], st.v[c][1]);
        }
      }
      if constexpr (kFp8) {
        if (lp == 0) kscale[(tt % 3) * kKT + lk] = st.sc;
      }
    };

    // ---- score waves: scores and softmax of tile tt into probability buffer tt % 2
    auto score_tile = [&](int tt) {
      // A operand (16 keys x 32 dims): row 16b + sh, logical chunk 4ks + sg, stored at
      // 16(ks/4) + 4((ks%4) ^ (sh%4)) + (sg ^ (sh/4)%4). The four per-lane bases (one per ks%4)
      // are made opaque to the optimiser so that it uses the reads' immediate offsets.
      int qb[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        qb[m] = (tt % 3) * kTileElems + sh * kRow + 8 * (4 * (m ^ (sh & 3)) + (sg ^ ((sh >> 2) & 3)));
      asm volatile("" : "+v"(qb[0]), "+v"(qb[1]), "+v"(qb[2]), "+v"(qb[3]));
      f32x4 acc[2][2] = {};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(ktile + qb[ks & 3] + 16 * b * kRow + 128 * (ks >> 2));
          acc[b][ks & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qreg[ks], acc[b][ks & 1], 0, 0, 0);
        }
      // this lane: head 16*wave + sh, key 16b + 4sg + r <-> z[4b + r]
      float z[8];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) z[4 * b + r] = acc[b][0][r] + acc[b][1][r];
      float ksc[8];
      if constexpr (kFp8) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(kscale + (tt % 3) * kKT + 16 * b + 4 * sg);
#pragma unroll
          for (int r = 0; r < 4; ++r) ksc[4 * b + r] = v[r];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] *= ksc[e];
      }
      const uint32_t vm = __builtin_amdgcn_readfirstlane(tmask[tt]);
      if (vm != 0xffffffffu) {   // only tiles with masked keys pay for the mask
        const uint32_t lm = vm >> (4 * sg);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = ((lm >> (16 * (e >> 2) + (e & 3))) & 1u) ? z[e] : -INFINITY;
      }
      // The scores stay unscaled: max(z) * sl2 = max(z * sl2) for sl2 > 0, and the exponent takes
      // sl2 in a fused multiply-add.
      float mx = z[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, z[e]);
      mx = rows_max(mx) * sl2;
      // The reference maximum only moves when a score exceeds it by more than 2^8 (or on the
      // first keys): probabilities then stay <= 256, and the value waves rescale O only for
      // tiles where one of the wave's heads moved. Exact: l and O share the same reference.
      float alpha = 1.f;
      const bool moved = __ballot(mx > m_run + 8.f) != 0;
      if (moved) {
        const float m_new = fmaxf(m_run, mx);
        alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
        m_run = m_new;
      }
      const int pb = tt & 1;
      if (sg == 0) alpha_s[pb * kMH + 16 * wave + sh] = alpha;
      if (lane == 0) rflag[pb * 4 + wave] = moved ? 1u : 0u;
      const float nref = m_run == -INFINITY ? 0.f : -m_run;
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(z[e], sl2, nref));
        psum += p[e];
      }
      l_run += rows_sum(psum);
      if constexpr (kFp8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] *= ksc[e];
      }
      // [head][key] rows; key 16b + 4sg + r sits at 16b + 8(sg%2) + 4(sg/2) + r, the order of the
      // value waves' B operand (element e of step t2 <-> key 16t2 + 8(e/4) + 4hf + e%4)
      uint16_t* prow = ptile + pb * kMH * kPPitch + (16 * wave + sh) * kPPitch + 8 * (sg & 1) + 4 * (sg >> 1);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const u32x2 w = {pack_bf16x2(p[4 * b], p[4 * b + 1]), pack_bf16x2(p[4 * b + 2], p[4 * b + 3])};
        *reinterpret_cast<u32x2*>(prow + 16 * b) = w;
      }
    };

    // ---- value waves: rescale and PV of tile tt
    auto value_tile = [&](int tt) {
      const int pb = tt & 1;
      const uint32_t fl = __builtin_amdgcn_readfirstlane(rflag[pb * 4 + 2 * hh] | rflag[pb * 4 + 2 * hh + 1]);
      if (fl) {
        const float al = alpha_s[pb * kMH + 32 * hh + col];
#pragma unroll
        for (int mb = 0; mb < 8; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[mb][r] *= al;
      }
      // B = P^T: 8 keys of step t2 for head 32hh + col
      const uint16_t* prow = ptile + pb * kMH * kPPitch + (32 * hh + col) * kPPitch + 8 * hf;
      bf16x8 pbf[2];
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2) pbf[t2] = *reinterpret_cast<const bf16x8*>(prow + 16 * t2);
      // A = K^T (32 dims x 16 keys) read transposed: lane j of each 16-lane group points at row
      // k0 + j/4 (+8 for the second read), dims d0 + 4(j%4), and receives 4 keys of dim d0 + j.
      // Rows 16t2 + 4hf + i16/4 (+8x), dims 256dh + 32mb + 16(col/16) + 4(i16%4); stored chunk
      // = logical chunk ^ swz(row), with swz(row) = 4(i16/4) + hf + 2x. One base per (x, mb%4).
      int vb[2][4];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int m = 0; m < 4; ++m)
          vb[x][m] = (tt % 3) * kTileElems + (4 * hf + (i16 >> 2) + 8 * x) * kRow +
                     8 * (32 * dh + 4 * (m ^ (i16 >> 2)) +
                          ((2 * (col >> 4) + ((i16 & 3) >> 1)) ^ (hf + 2 * x))) +
                     4 * (i16 & 1);
      asm volatile("" : "+v"(vb[0][0]), "+v"(vb[0][1]), "+v"(vb[0][2]), "+v"(vb[0][3]));
      asm volatile("" : "+v"(vb[1][0]), "+v"(vb[1][1]), "+v"(vb[1][2]), "+v"(vb[1][3]));
      auto trf = [&](int mb, int t2) {
        const int off = 16 * t2 * kRow + 128 * (mb >> 2);
        return lds_tr_pair(ktile + vb[0][mb & 3] + off, ktile + vb[1][mb & 3] + off);
      };
      // Step s: key half t2 = s / 8, dim block mb = s % 8 (consecutive products accumulate into
      // different blocks). The A operands are read kAhead steps ahead into a small ring, so the
      // transposed LDS reads overlap the products instead of each product waiting for its read.
      constexpr int kAhead = 3;
      bf16x8 opa[kAhead + 1];
#pragma unroll
      for (int s = 0; s < kAhead; ++s) opa[s] = trf(s & 7, s >> 3);
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if (s + kAhead < 16) opa[(s + kAhead) % (kAhead + 1)] = trf((s + kAhead) & 7, (s + kAhead) >> 3);
        o[s & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(opa[s % (kAhead + 1)], pbf[s >> 3], o[s & 7], 0, 0, 0);
      }
    };

    if constexpr (kScore) {
      // Q^T is the B operand: column = head, k-step ks covers dims 32ks + 8*sg + [0, 8). Read
      // here (again for a later segment) so that its latency overlaps the first tile loads
      // rather than the key resolution.
      const uint16_t* qrow =
          reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)i * kMH + 16 * wave + sh) * kMD + 8 * sg;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
    }
    Stage<kFp8> s0, s1, s2;
    load(s0, 0);
    load(s1, 1);
    load(s2, 2);
    publish(s0, 0);
    load(s0, 3);
    __syncthreads();
    if constexpr (kScore) score_tile(0);
    publish(s1, 1);
    load(s1, 4);
    __syncthreads();
    // iteration t: X holds tile t+2 (stored now, then reloaded with tile t+5)
    auto iter = [&](int t, Stage<kFp8>& X) {
      publish(X, t + 2);
      load(X, t + 5);
      if constexpr (kScore) {
        if (t + 1 < n_tiles) score_tile(t + 1);
      } else {
        value_tile(t);
      }
      __syncthreads();
    };
    // One exit, at the bottom: an exit from the middle of the body makes the control-flow
    // structuriser add a path into the loop header on which the stage stored there looks freshly
    // loaded, and the header's wait then drains every load in flight.
    int t = 0;
    for (; t + 3 <= n_tiles; t += 3) {
      iter(t, s2);
      iter(t + 1, s0);
      iter(t + 2, s1);
    }
    if (t < n_tiles) {
      iter(t, s2);
      if (t + 1 < n_tiles) iter(t + 1, s0);
    }
  }
  // ---- partials: m and l per head from the score waves; O / l as bf16 [head][dim] (zero for a
  // split without keys), staged through LDS by the value waves so that every global store writes
  // one contiguous 1 KB row. With one split and a bf16 output the partial is the output: the
  // value waves rotate it by RoPE(-p) before staging and the rows go straight to `out` (the
  // launch then skips the combine).
  constexpr int kOPitch = kMD + 8;   // staged row (bf16): 1040 B, rows 4 banks apart
  uint16_t* ost = ktile;             // the tile buffers are free after the last barrier
  constexpr bool direct = kDirect;   // one split and a bf16 output (the launch decides)
  const int rope_lo = kMD - a.rope_dim;
  if constexpr (kScore) {
    if constexpr (direct) {
      // cos / sin of -p * theta_t for the value waves (the score waves are idle here)
      for (int t = tid; t < (a.rope_dim >> 1); t += 256) {
        float c, sn;
        rope_cs(-(double)qk.p, t, a.rope_dim, a.rope_base, &c, &sn);
        orope[t] = make_float2(c, sn);
      }
    }
    if (sg == 0) {
      const int h = 16 * wave + sh;
      if constexpr (!direct) {
        float* pml = a.part_ml + (int64_t)slot * 2 * kMH;
        // m is kept in log2 units inside the kernel; store natural-log units for the combine
        pml[h] = m_run == -INFINITY ? -INFINITY : m_run / kLog2e;
        pml[kMH + h] = l_run;
      }
      lfin[h] = l_run;
    }
    __syncthreads();
    __syncthreads();
  } else {
    __syncthreads();
    // O^T rows d = 256*dh + 32*mb + 8*(r/4) + 4*hf + r%4, column h = 32*hh + col: four
    // consecutive dims per (mb, r/4), 8 bytes each
    const int h = 32 * hh + col;
    const float l = lfin[h];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* orow = ost + h * kOPitch + 256 * dh + 4 * hf;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x16& v = o[mb];
        float y[4] = {v[4 * q4] * inv, v[4 * q4 + 1] * inv, v[4 * q4 + 2] * inv, v[4 * q4 + 3] * inv};
        const int d = 256 * dh + 32 * mb + 8 * q4 + 4 * hf;   // first of the four dims
        if (kDirect && d >= rope_lo) {
#pragma unroll
          for (int e = 0; e < 4; e += 2) {
            const float2 cs = orope[(d + e - rope_lo) >> 1];
            const float y0 = y[e] * cs.x - y[e + 1] * cs.y;
            const float y1 = y[e] * cs.y + y[e + 1] * cs.x;
            y[e] = y0;
            y[e + 1] = y1;
          }
        }
        const u32x2 w = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
        *reinterpret_cast<u32x2*>(orow + 32 * mb + 8 * q4) = w;
      }
    __syncthreads();
  }
  // wave w stores rows 8w..8w+7, one row (64 lanes x 16 B) per instruction
  {
    uint16_t* po = direct ? reinterpret_cast<uint16_t*>(a.out) + (int64_t)i * kMH * kMD
                          : reinterpret_cast<uint16_t*>(a.part_o) + (int64_t)slot * kMH * kMD;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int row = 8 * wave + c;
      *reinterpret_cast<u32x4*>(po + row * kMD + 8 * lane) =
          *reinterpret_cast<const u32x4*>(ost + row * kOPitch + 8 * lane);
    }
  }
  };
  if (scorer)
    role(std::true_type{});
  else
    role(std::false_type{});
  if constexpr (kSel) {
    if (last_reader) {   // uniform: every workgroup of the query has read the row's bin counts
      uint32_t* rh = a.sel.row_hist + (int64_t)i * kTopBins;
      for (int j = tid; j < kTopBins; j += 512) rh[j] = 0u;
      if (tid == 0) a.sel.row_done[i] = 0u;
    }
  }
}
// ------------------------------------------------------------------------------------------
// Combine: merge the split partials, inverse RoPE at the query position, cast.
// Split s of a query holds O_s / l_s with its (m_s, l_s); the output is sum_s w_s O_s / l_s with
// w_s = l_s exp(m_s - M) / sum_s' l_s' exp(m_s' - M), M = max_s m_s.
// Workgroup (group of hpw heads, query), mapped to the XCD that ran the query's splits so that the
// partials come from its L2; thread = 8 consecutive dims of one head (one 16- or 32-byte load per
// split, eight splits in flight), or single dims when dim % 8 != 0.
// ------------------------------------------------------------------------------------------
constexpr int kCombineHeads = 64;     // heads per combine workgroup at most
constexpr int kCombineElems = 2048;   // elements per combine workgroup (hpw = 2048 / dim, >= 1)

// Raw 8-element load of a partial (16 bytes of bf16 or 32 bytes of fp32), widened later.
template <typename PT>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  u32x4 w;
};
template <>
struct Raw8<float> {
  f32x4 a, b;
};
template <typename PT>
__device__ __forceinline__ Raw8<PT> load8(const PT* p) {
  Raw8<PT> r;
  if constexpr (sizeof(PT) == 2) {
    r.w = *reinterpret_cast<const u32x4*>(p);
  } else {
    r.a = *reinterpret_cast<const f32x4*>(p);
    r.b = *reinterpret_cast<const f32x4*>(p + 4);
  }
  return r;
}
template <typename PT>
__device__ __forceinline__ void widen8(const Raw8<PT>& r, float* x) {
  if constexpr (sizeof(PT) == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __builtin_bit_cast(float, r.w[e] << 16);
      x[2 * e + 1] = __builtin_bit_cast(float, r.w[e] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = r.a[e];
      x[4 + e] = r.b[e];
    }
  }
}

template <typename PT>
__device__ __forceinline__ float load1(const PT* p) {
  if constexpr (sizeof(PT) == 2) {
    return bf16_to_f32(*p);
  } else {
    return *p;
  }
}

// LDS of one combine workgroup: split weights [split][head of the group] and the splits' (m, l)
// [split][m, l][head of the group], sized by the split count.
__host__ __device__ inline size_t combine_lds_bytes(int n_split) {
  return (size_t)n_split * 3 * kCombineHeads * sizeof(float);
}

// Workgroup `logical` of the combine: head group logical % gx (gx groups of hpw heads), query
// logical / gx. sm: combine_lds_bytes(n_split) of LDS.
template <typename PT>
__device__ __forceinline__ void combine_group(const AttnArgs& a, int hpw, int logical, int gx,
                                              float* sm) {
  const int i = logical / gx;
  const int h0 = (logical % gx) * hpw;
  const int H = a.n_heads, D = a.dim;
  // the query's partials: n_split of them from slot i * n_split, or as the balanced plan recorded
  int ns = a.n_split;
  int64_t first = (int64_t)i * ns;
  if (a.qplan != nullptr) {
    first = a.qplan[2 * i];
    ns = a.qplan[2 * i + 1];
  }
  const int nh = min(hpw, H - h0);
  float* wsp = sm;                              // [split][head of the group]
  float* mls = sm + ns * kCombineHeads;         // [split][m, l][head of the group]
  __shared__ float rc[kMaxRopePairs], rs[kMaxRopePairs];
  __shared__ uint32_t lamax[kCombineHeads];   // FP8 output: bits of each head's largest |value|
  const int tid = threadIdx.x;
  const int64_t sstride = (int64_t)H * D;
  const PT* po = reinterpret_cast<const PT*>(a.part_o) + first * sstride;
  // the first eight splits' partials are requested before the weights are formed
  const bool oct = (D & 7) == 0;
  const int n8 = oct ? nh * (D / 8) : 0;
  Raw8<PT> pre[8];
  if (oct && tid < n8) {
    const PT* base = po + (int64_t)(h0 + tid / (D / 8)) * D + 8 * (tid % (D / 8));
#pragma unroll
    for (int q = 0; q < 8; ++q) pre[q] = load8<PT>(base + min(q, ns - 1) * sstride);
  }
  const float* pml = a.part_ml + first * 2 * H;
  for (int e = tid; e < ns * 2 * nh; e += 256) {
    const int s2 = e / nh, hl = e % nh;   // s2 = 2 * split + (0: m, 1: l)
    mls[e] = pml[s2 * H + h0 + hl];
  }
  if (tid < kCombineHeads) lamax[tid] = 0u;
  const int rope_lo = D - a.rope_dim;
  if (a.rope_tab != nullptr) {   // formed by the attention kernel with rope_cs
    const float* tab = a.rope_tab + (int64_t)i * kMaxRopePairs * 2;
    for (int t = tid; t < a.rope_dim / 2; t += 256) {
      rc[t] = tab[2 * t];
      rs[t] = tab[2 * t + 1];
    }
  } else {
    int seq, p;
    query_at(a.qd, i, &seq, &p);
    for (int t = tid; t < a.rope_dim / 2; t += 256)
      rope_cs(-(double)p, t, a.rope_dim, a.rope_base, &rc[t], &rs[t]);
  }
  __syncthreads();
  for (int hl = tid; hl < nh; hl += 256) {
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, mls[(2 * s) * nh + hl]);
    float den = 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = mls[(2 * s) * nh + hl];
      den += ms == -INFINITY ? 0.f : expf(ms - M) * mls[(2 * s + 1) * nh + hl];
    }
    const float inv = den > 0.f ? 1.0f / den : 0.f;
    for (int s = 0; s < ns; ++s) {
      const float ms = mls[(2 * s) * nh + hl];
      wsp[s * kCombineHeads + hl] = ms == -INFINITY ? 0.f : expf(ms - M) * mls[(2 * s + 1) * nh + hl] * inv;
    }
  }
  __syncthreads();
  auto rope8 = [&](int d, float* x) {   // RoPE(-p) of dims d..d+7
    if (d + 8 > rope_lo) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        if (d + e >= rope_lo) {
          const int pr = (d + e - rope_lo) >> 1;
          const float z0 = x[e] * rc[pr] - x[e + 1] * rs[pr];
          const float z1 = x[e] * rs[pr] + x[e + 1] * rc[pr];
          x[e] = z0;
          x[e + 1] = z1;
        }
      }
    }
  };
  auto finish = [&](int h, int d, float* x, int n) {   // n = 8 or 1 values at dims d..d+n-1
    if (n == 8) rope8(d, x);
    const int64_t off = ((int64_t)i * H + h) * D + d;
    if (n == 8) {
      if (a.out_dtype == F32) {
        float* o = reinterpret_cast<float*>(a.out) + off;
        *reinterpret_cast<f32x4*>(o) = f32x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<f32x4*>(o + 4) = f32x4{x[4], x[5], x[6], x[7]};
      } else {
        const u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                         pack_bf16x2(x[6], x[7])};
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.out) + off) = w;
      }
    } else {
      if (a.out_dtype == F32)
        reinterpret_cast<float*>(a.out)[off] = x[0];
      else
        reinterpret_cast<uint16_t*>(a.out)[off] = (uint16_t)(pack_bf16x2(x[0], 0.f) & 0xffffu);
    }
  };
  // weighted sum of the splits' partials at chunk e8 (head e8 / (D/8), dims 8 (e8 % (D/8)) + [0, 8))
  auto accumulate = [&](int e8, float* acc) __attribute__((always_inline)) {
      const int hl = e8 / (D / 8), d = 8 * (e8 % (D / 8));
      const PT* base = po + (int64_t)(h0 + hl) * D + d;
      for (int s0 = 0; s0 < ns; s0 += 8) {
        Raw8<PT> raw[8];
        if (e8 == tid && s0 == 0) {
#pragma unroll
          for (int q = 0; q < 8; ++q) raw[q] = pre[q];
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) raw[q] = load8<PT>(base + min(s0 + q, ns - 1) * sstride);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          float x[8];
          widen8<PT>(raw[q], x);
          const float w = s0 + q < ns ? wsp[(s0 + q) * kCombineHeads + hl] : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, x[e], acc[e]);
        }
      }
  };
  if (oct && a.out_dtype == FP8) {
    // Inverse RoPE + fp8 output ([vLLM] fused "inverse RoPE + fp8 quant"): each thread holds one
    // chunk (n8 <= 256 for dim <= 2048); the head's largest magnitude gathers in LDS, then every
    // row is encoded with scale = amax / 448 and written with its scale.
    const bool have = tid < n8;
    const int hl = have ? tid / (D / 8) : 0, d = 8 * (tid % (D / 8)), h = h0 + hl;
    float acc[8] = {};
    if (have) {
      accumulate(tid, acc);
      rope8(d, acc);
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(acc[e]));
      atomicMax(&lamax[hl], __float_as_uint(m));
    }
    __syncthreads();
    if (have) {
      const float amax = __uint_as_float(lamax[hl]);
      const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
      uint32_t b[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = f32_to_e4m3(__fdiv_rn(acc[e], scale));
      store_bytes<8>(reinterpret_cast<uint8_t*>(a.out) + ((int64_t)i * H + h) * D + d, b);
      if (d == 0) a.out_scale[(int64_t)i * H + h] = scale;
    }
  } else if (oct) {
    for (int e8 = tid; e8 < n8; e8 += 256) {
      const int hl = e8 / (D / 8), d = 8 * (e8 % (D / 8));
      const int h = h0 + hl;
      const PT* base = po + (int64_t)h * D + d;
      float acc[8] = {};
      for (int s0 = 0; s0 < ns; s0 += 8) {
        Raw8<PT> raw[8];
        if (e8 == tid && s0 == 0) {
#pragma unroll
          for (int q = 0; q < 8; ++q) raw[q] = pre[q];
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) raw[q] = load8<PT>(base + min(s0 + q, ns - 1) * sstride);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          float x[8];
          widen8<PT>(raw[q], x);
          const float w = s0 + q < ns ? wsp[(s0 + q) * kCombineHeads + hl] : 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, x[e], acc[e]);
        }
      }
      finish(h, d, acc, 8);
    }
  } else {
    // any dim: one element per thread and step; RoPE pairs are formed from both elements
    for (int e = tid; e < nh * D; e += 256) {
      const int hl = e / D, d = e % D, h = h0 + hl;
      const int dp = d >= rope_lo ? rope_lo + ((d - rope_lo) & ~1) : d;   // first of the pair
      float x0 = 0.f, x1 = 0.f;
      for (int s = 0; s < ns; ++s) {
        const float w = wsp[s * kCombineHeads + hl];
        x0 = fmaf(w, load1<PT>(po + s * sstride + (int64_t)h * D + dp), x0);
        if (d >= rope_lo) x1 = fmaf(w, load1<PT>(po + s * sstride + (int64_t)h * D + dp + 1), x1);
      }
      float y = x0;
      if (d >= rope_lo) {
        const int pr = (dp - rope_lo) >> 1;
        y = d == dp ? x0 * rc[pr] - x1 * rs[pr] : x0 * rs[pr] + x1 * rc[pr];
      }
      finish(h, d, &y, 1);
    }
  }
}

template <typename PT>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, int hpw) {
  extern __shared__ __attribute__((aligned(16))) float csm[];
  combine_group<PT>(a, hpw, xcd_logical(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y),
                    gridDim.x, csm);
}

// The combine of the MFMA kernel's splits with a compressor call riding along: workgroups
// [0, n_comb) combine (mapped as attn_combine's), the rest each pool one compressor group with
// four waves (float or bf16 x, dim <= 512 in 16-byte chunks). The compressor's latency then hides
// behind the combine instead of taking a launch of its own. Nothing here orders the two: the
// caller guarantees that neither reads what the other writes.
template <typename T, int kRB, int kV>
__global__ __launch_bounds__(256, 4) void attn_combine_compress(AttnArgs a, int hpw, int gx,
                                                             int n_comb, CompressArgs c,
                                                             int comp_gx) {
  // dynamic LDS: the combine's (combine_lds_bytes) or the compressor's ((3 dim + 128) floats)
  extern __shared__ __attribute__((aligned(16))) float csm[];
  const int bid = blockIdx.x;
  if (bid < n_comb) {
    combine_group<uint16_t>(a, hpw, xcd_logical(bid, n_comb), gx, csm);
  } else {
    const int k = bid - n_comb;
    constexpr int kVec = 16 / (int)sizeof(T);   // 16-byte chunks: dim <= 512 is one or two per lane
    compress_group<T, kVec, 512 / kVec / 64, kRB, kV>(c, k % comp_gx, k / comp_gx, csm);
  }
}

// Fewest keys per split of the MFMA kernel: below this the fixed cost of a workgroup (key
// resolution, pipeline fill, writing its partial) outweighs the parallelism gained.
constexpr int kMfmaMinChunk = 128;

AttnPlan plan_attention(int32_t n_q, int32_t n_heads, int32_t dim, int32_t max_keys,
                        int32_t q_dtype, int32_t pool_dtype, bool balanced) {
  AttnPlan pl{};
  pl.use_mfma = n_heads == kMH && dim == kMD && q_dtype == BF16 &&
                (pool_dtype == BF16 || pool_dtype == FP8);
  const int tile = pl.use_mfma ? kKT : kGenTile;
  const int target_blocks = pl.use_mfma ? 256 : 512;
  const int min_chunk = pl.use_mfma ? kMfmaMinChunk : 64;
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
  // Decode launches with several splits take the balanced plan: n_q + kBalancedSlots slots, pieces
  // cut on the device from the actual lengths (a batch of mixed lengths then spreads its long
  // queries over many workgroups instead of sizing every query's splits by the longest).
  pl.balanced = balanced && pl.use_mfma && ns > 1 && n_q <= kBalancedMaxQueries;
  size_t slots = (size_t)n_q * ns;
  if (pl.balanced) {
    pl.n_split = kMaxSplit;   // pieces per query at most (the combine's LDS bound)
    pl.n_slots = n_q + kBalancedSlots;
    slots = (size_t)pl.n_slots;
  }
  const size_t elem = pl.use_mfma ? sizeof(uint16_t) : sizeof(float);
  pl.o_bytes = (slots * dim * n_heads * elem + 255) / 256 * 256;
  pl.ws_bytes = pl.o_bytes + slots * 2 * n_heads * sizeof(float);
  if (pl.use_mfma) {
    pl.rope_off = (pl.ws_bytes + 255) / 256 * 256;
    pl.ws_bytes = pl.rope_off + (size_t)n_q * kMaxRopePairs * 2 * sizeof(float);
  }
  if (pl.balanced) {
    pl.qplan_off = (pl.ws_bytes + 255) / 256 * 256;
    pl.ws_bytes = pl.qplan_off + (size_t)n_q * 2 * sizeof(int32_t);
  }
  return pl;
}

namespace {
hipError_t launch_attention_kernel(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.n_split, a.n_q);
  if (a.qplan != nullptr) grid = dim3(a.n_slots);
  if (a.use_mfma) {
    const bool direct = a.n_split == 1 && a.out_dtype == BF16;   // writes_output(a)
    const CompressArgs none{};
#define HYB_ATTN_MFMA(F, D) \
  hipLaunchKernelGGL((attn_mfma<F, D, false>), grid, dim3(512), 0, s, a, none, none, 0, 0)
    if (a.swa.dtype == FP8) {
      if (direct) HYB_ATTN_MFMA(true, true);
      else HYB_ATTN_MFMA(true, false);
    } else {
      if (direct) HYB_ATTN_MFMA(false, true);
      else HYB_ATTN_MFMA(false, false);
    }
#undef HYB_ATTN_MFMA
  } else {
    size_t lds = sizeof(float) * ((size_t)2 * a.n_heads * a.dim + (size_t)a.n_heads * kGenTile +
                                  3 * (size_t)a.n_heads);
    hipLaunchKernelGGL(attn_generic, grid, dim3(256), lds, s, a);
  }
  return hipGetLastError();
}

int combine_heads_per_wg(const AttnArgs& a) {
  return std::max(1, std::min(kCombineHeads, std::min(a.n_heads, kCombineElems / a.dim)));
}
}  // namespace

// The MFMA kernel writes the output itself when there is one split and the output is bf16.
static bool writes_output(const AttnArgs& a) { return a.use_mfma && a.n_split == 1 && a.out_dtype == BF16; }

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  hipError_t e = launch_attention_kernel(a, s);
  if (e != hipSuccess || writes_output(a)) return e;
  const int hpw = combine_heads_per_wg(a);
  const dim3 cgrid((a.n_heads + hpw - 1) / hpw, a.n_q);
  const size_t lds = combine_lds_bytes(a.n_split);
  if (a.use_mfma)
    hipLaunchKernelGGL(attn_combine<uint16_t>, cgrid, dim3(256), lds, s, a, hpw);
  else
    hipLaunchKernelGGL(attn_combine<float>, cgrid, dim3(256), lds, s, a, hpw);
  return hipGetLastError();
}

// The fused selection pays off while every part's candidates usually lie among its prefetched
// pairs: at most kSelFusedParts parts per row (contexts up to 256K tokens at ratio 4), 64 or more
// pairs per part. Longer rows go through the selection kernel (measured: the quantised batch of
// 64 rows of up to 2^20 tokens took 167 us per C4 step with the selection fused at 16 pairs per
// part, 136 us with the selection kernel).
constexpr int kSelFusedParts = kSelPrefetch / 64;
bool attention_select_supported(const AttnArgs& a) {
  return a.use_mfma && a.sel.pairs != nullptr && a.k <= kMaxTopK && a.n_q <= kRowHistRows &&
         (a.sel.max_nv + kScorePartKeys - 1) / kScorePartKeys <= kSelFusedParts;
}

hipError_t launch_attention_select(const AttnArgs& a, const SideWork* side, hipStream_t s) {
  if (a.n_q == 0) return hipSuccess;
  if (!attention_select_supported(a)) return hipErrorInvalidValue;
  SideWork none{};
  const SideWork& sw = side ? *side : none;
  const dim3 grid(a.n_split * a.n_q + sw.n[0] + sw.n[1]);
  const bool direct = writes_output(a);
#define HYB_ATTN_SEL(F, D) \
  hipLaunchKernelGGL((attn_mfma<F, D, true>), grid, dim3(512), 0, s, a, sw.c[0], sw.c[1], sw.n[0], sw.n[1])
  if (a.swa.dtype == FP8) {
    if (direct) HYB_ATTN_SEL(true, true);
    else HYB_ATTN_SEL(true, false);
  } else {
    if (direct) HYB_ATTN_SEL(false, true);
    else HYB_ATTN_SEL(false, false);
  }
#undef HYB_ATTN_SEL
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || direct) return e;
  const int hpw = combine_heads_per_wg(a);
  const dim3 cgrid((a.n_heads + hpw - 1) / hpw, a.n_q);
  hipLaunchKernelGGL(attn_combine<uint16_t>, cgrid, dim3(256), combine_lds_bytes(a.n_split), s, a, hpw);
  return hipGetLastError();
}

// Attention, then the compressor call c. With the MFMA kernel and a compressor call that four
// waves can run in four-dim chunks (dim <= 512, dim % 4 == 0 for float x and % 8 for bf16 x,
// x / state / pool 16-byte aligned), the compressor's workgroups join the combine's launch;
// otherwise the compressor gets its own launch after the combine.
hipError_t launch_attention_compress(const AttnArgs& a, const CompressArgs& c, hipStream_t s) {
  const int r = c.out.ratio, D = c.out.dim;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  const bool fuse = a.n_q > 0 && a.use_mfma && !writes_output(a) && c.batch > 0 && c.max_new_tokens > 0 && D <= 512 &&
                    D % (c.x_dtype == F32 ? 4 : 8) == 0 && al16(c.x) && al16(c.state) &&
                    al16(c.out.data) && (r == 4 || r == 128) && (c.out.dtype == F32 || c.out.dtype == BF16);
  if (!fuse) {
    hipError_t e = launch_attention(a, s);
    if (e != hipSuccess) return e;
    return c.batch > 0 && c.max_new_tokens > 0 ? launch_compress(c, s) : hipSuccess;
  }
  hipError_t e = launch_attention_kernel(a, s);
  if (e != hipSuccess) return e;
  const int hpw = combine_heads_per_wg(a);
  const int gx = (a.n_heads + hpw - 1) / hpw;
  const int n_comb = gx * a.n_q;
  const int comp_gx = (c.max_new_tokens + r - 1) / r + 1;
  const dim3 grid(n_comb + comp_gx * c.batch);
  const size_t lds = std::max(combine_lds_bytes(a.n_split), (size_t)(3 * D + 128) * sizeof(float));
  // four waves run pooled_waves(r, D) virtual waves: 4 (r = 4) or 16 (r = 128, D <= 512); at
  // r = 128 a batch holds two (float) or four (bf16) rows of each of a wave's four virtual waves
  // (the kernel keeps to 128 registers, so that four of its workgroups fit on a compute unit)
  if (c.x_dtype == F32) {
    if (r == 4)
      hipLaunchKernelGGL((attn_combine_compress<float, 1, 1>), grid, dim3(256), lds, s, a, hpw, gx, n_comb, c, comp_gx);
    else
      hipLaunchKernelGGL((attn_combine_compress<float, 2, 4>), grid, dim3(256), lds, s, a, hpw, gx, n_comb, c, comp_gx);
  } else {
    if (r == 4)
      hipLaunchKernelGGL((attn_combine_compress<uint16_t, 1, 1>), grid, dim3(256), lds, s, a, hpw, gx, n_comb, c, comp_gx);
    else
      hipLaunchKernelGGL((attn_combine_compress<uint16_t, 4, 4>), grid, dim3(256), lds, s, a, hpw, gx, n_comb, c, comp_gx);
  }
  return hipGetLastError();
}

}  // namespace hyb
