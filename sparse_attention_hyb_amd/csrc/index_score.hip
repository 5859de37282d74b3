// Indexer scores over the visible compressed entries:
//   score[i][g] = sum_h w[i][h] * max(0, q_idx[i][h] . key_g).
// Method: vLLM DeepSeek-V4 day-0 post ("DeepSeek Sparse Attention over compressed tokens"; fp4
// indexer cache) and the SGLang DeepSeek-V4 day-0 blog ("Shadow Radix": C4 keeps the top-512 of
// the indexer's scores).
//
// Two kernels:
//  * score_mfma: 64 heads x 128 dims, bf16 query, bf16 or fp4 (E2M1 + E8M0 per 32) keys. The
//    step streams every visible key once (the step's dominant HBM traffic), so each wave reads
//    its 32-key tiles straight into MFMA operand registers: no LDS round trip. S = Q . K^T runs on
//    v_mfma_f32_32x32x16_bf16 with the 64 heads as the M dimension (two 32-row blocks) and the 32
//    keys as N; each lane then owns one key column and 32 of its heads, so the ReLU-weighted head
//    sum is 32 in-lane FMAs plus one cross-half add.
//  * score_generic: any (heads x dim) <= 8192, fp32 / bf16 / fp4 - one thread per key.
// For the selector that follows, all can instead hand over each part of kScorePartKeys keys as a
// cumulative histogram of the top kTopBits bits of the scores' order keys plus the part's
// (order key, index) pairs bucketed by those bits (see finish_parts): the first radix pass of the
// top-k, and the gathering of its candidates, ride along with the score stream.
#include <type_traits>

#include "common.h"

namespace hyb {

constexpr int kScoreKeysPerBlock = 2 * kScorePartKeys;  // keys per workgroup (MFMA kernel)
constexpr int kScoreParts = kScoreKeysPerBlock / kScorePartKeys;
constexpr int kMfmaHeads = 64;
constexpr int kMfmaDim = 128;

__device__ __forceinline__ float canonical_zero(float v) { return v == 0.0f ? 0.0f : v; }

// Eight E2M1 nibbles (one 32-bit word, element 0 in the low nibble) times a power-of-two block
// scale -> eight bf16 values, exactly, with gfx950's scaled conversion (two elements of one byte
// per instruction, low nibble first; it matches the arithmetic conversion bit for bit for every
// code and scales from 2^-100 to 2^60).
__device__ __forceinline__ bf16x8 fp4x8_to_bf16x8(uint32_t w, float sc) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  return __builtin_bit_cast(bf16x8, r);
}

// Selector hand-off (part_hist set). For each part of kScorePartKeys keys a workgroup writes
//  * its cumulative histogram over the top kTopBits bits of the order keys: part_hist[b] = number
//    of the part's keys whose top bits are >= b (uint16, <= kScorePartKeys), and
//  * the part's (order key, row index) pairs bucketed by those bits, highest bin first (order
//    within a bin unspecified), as uint2 at pairs + kScorePartKeys * part,
// so that the selector, once it knows the bin b0 of the k-th largest key, reads only the leading
// part_hist[b0] pairs of every part. The workgroup's keys are in lkeys[0, P * kScorePartKeys)
// (index g - base) and its per-part counts in lhist[P][kTopBins], which become bucket cursors;
// lsorted (P * kScorePartKeys uint2) is scratch. 256 threads.
template <int P, bool kPacked = false>
__device__ __forceinline__ void finish_parts(const ScoreArgs& a, int i, int part0, int base, int end,
                                             const uint32_t* lkeys, uint32_t* lhist, uint2* lsorted,
                                             uint32_t* wtot) {
  static_assert(kTopBins == 4 * 256, "four bins per thread");
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  __syncthreads();   // keys and counts complete
#pragma unroll
  for (int q = 0; q < P; ++q) {
    if (base + q * kScorePartKeys >= end) break;   // uniform
    uint32_t* h = lhist + q * (kPacked ? kTopBins / 2 : kTopBins);
    // thread t owns bins 1023 - 4t - e (e < 4), i.e. bins in descending order across threads
    // (packed: two 16-bit counts per word, bin b in half b % 2 of word b / 2)
    uint32_t c[4], tot = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int bin = kTopBins - 1 - 4 * t - e;
      c[e] = kPacked ? (h[bin >> 1] >> (16 * (bin & 1))) & 0xffffu : h[bin];
      tot += c[e];
    }
    const uint32_t incl = wave_inclusive_scan(tot);
    if (lane == 63) wtot[q * 4 + w] = incl;
    __syncthreads();
    uint32_t before = incl - tot;
    for (int v = 0; v < w; ++v) before += wtot[q * 4 + v];
    // cum[b] = keys with top bits >= b; bucket b starts at cum[b] - count[b]
    uint32_t run = before;
    uint32_t cum[4], cur[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      cur[e] = run;   // cursor: start of the bucket
      run += c[e];
      cum[e] = run;
    }
    if constexpr (kPacked) {   // bins 1020 - 4t .. 1023 - 4t: words 510 - 2t, 511 - 2t
      h[kTopBins / 2 - 2 - 2 * t] = cur[3] | (cur[2] << 16);
      h[kTopBins / 2 - 1 - 2 * t] = cur[1] | (cur[0] << 16);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) h[kTopBins - 1 - 4 * t - e] = cur[e];
    }
    // bins 1020 - 4t .. 1023 - 4t, ascending in memory
    uint2 wv;
    wv.x = cum[3] | (cum[2] << 16);
    wv.y = cum[1] | (cum[0] << 16);
    *reinterpret_cast<uint2*>(a.part_hist + ((int64_t)i * a.part_ld + part0 + q) * kTopBins +
                              (kTopBins - 4 - 4 * t)) = wv;
  }
  __syncthreads();
  const int nk = min(P * kScorePartKeys, end - base);
  for (int j = t; j < nk; j += 256) {
    const uint32_t key = lkeys[j];
    const int q = j / kScorePartKeys;
    const uint32_t bin = key >> (32 - kTopBits);
    uint32_t slot;
    if constexpr (kPacked) {
      const uint32_t sh = 16 * (bin & 1u);
      slot = (atomicAdd(&lhist[q * (kTopBins / 2) + (bin >> 1)], 1u << sh) >> sh) & 0xffffu;
    } else {
      slot = atomicAdd(&lhist[q * kTopBins + bin], 1u);
    }
    lsorted[q * kScorePartKeys + slot] = make_uint2(key, (uint32_t)(base + j));
  }
  __syncthreads();
  uint2* pairs = reinterpret_cast<uint2*>(a.scores) + (int64_t)i * (a.ld / 2) +
                 (int64_t)part0 * kScorePartKeys;
  for (int j = t; j < nk; j += 256) pairs[j] = lsorted[j];
}

// The hand-off of one part for one query by one wave (no workgroup barrier): the wave's 16-bit
// packed histogram of the part's keys becomes the cumulative histogram (written out) and bucket
// cursors (written back), then every key is scattered to its bucket in the output pairs. Lane l
// owns bins 1023 - 16 l - e (e < 16), i.e. bins in descending order across lanes.
__device__ __forceinline__ void finish_part_wave(const ScoreArgs& a, int i, int part, int base,
                                                 int end, const uint32_t* lkeys, uint32_t* lhist,
                                                 int lane) {
  uint32_t c[16], tot = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int bin = kTopBins - 1 - 16 * lane - e;
    c[e] = (lhist[bin >> 1] >> (16 * (bin & 1))) & 0xffffu;
    tot += c[e];
  }
  const uint32_t incl = wave_inclusive_scan(tot);
  uint32_t run = incl - tot;
  uint32_t cur[16], cum[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    cur[e] = run;
    run += c[e];
    cum[e] = run;
  }
  // bins 1008 - 16l .. 1023 - 16l: ascending in memory, bin 1023 - 16l - e holds cum[e]
  u32x4 w0, w1;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    w0[m] = cum[15 - 2 * m] | (cum[14 - 2 * m] << 16);
    w1[m] = cum[7 - 2 * m] | (cum[6 - 2 * m] << 16);
  }
  uint16_t* ph = a.part_hist + ((int64_t)i * a.part_ld + part) * kTopBins + (kTopBins - 16 - 16 * lane);
  *reinterpret_cast<u32x4*>(ph) = w0;
  *reinterpret_cast<u32x4*>(ph + 8) = w1;
#pragma unroll
  for (int m = 0; m < 8; ++m)   // word 504 - 8l + m: bins 1008 - 16l + 2m (low), + 1 (high)
    lhist[kTopBins / 2 - 8 - 8 * lane + m] = cur[15 - 2 * m] | (cur[14 - 2 * m] << 16);
  __builtin_amdgcn_wave_barrier();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the cursors before any lane's atomics
  __builtin_amdgcn_wave_barrier();
  uint2* pairs = reinterpret_cast<uint2*>(a.scores) + (int64_t)i * (a.ld / 2) +
                 (int64_t)part * kScorePartKeys;
  const int nk = min(kScorePartKeys, end - base);
  for (int j = lane; j < nk; j += 64) {
    const uint32_t key = lkeys[j];
    const uint32_t bin = key >> (32 - kTopBits);
    const uint32_t sh = 16 * (bin & 1u);
    const uint32_t slot = (atomicAdd(&lhist[bin >> 1], 1u << sh) >> sh) & 0xffffu;
    pairs[slot] = make_uint2(key, (uint32_t)(base + j));
  }
}

template <bool kFp4>
__global__ __launch_bounds__(256, 2) void score_mfma(ScoreArgs a) {
  __shared__ uint32_t lhist[kScoreParts * kTopBins];   // one histogram per kScorePartKeys keys
  __shared__ uint32_t lkeys[kScoreKeysPerBlock];
  __shared__ uint2 lsorted[kScoreKeysPerBlock];
  __shared__ uint32_t wtot[kScoreParts * 4];
  // physical blocks of this workgroup's keys (at least 2 entries per block: ratio <= 128)
  __shared__ int32_t tbl[kScoreKeysPerBlock / 2 + 2];
  const int i = blockIdx.y;
  int seq, p;
  query_at(a.qd, i, &seq, &p);
  // rows hold n_visible(max_pos) scores; a query past max_pos is clamped to that width
  const int nv = min(n_visible(p, a.pool.ratio, a.window), n_visible(a.max_pos, a.pool.ratio, a.window));
  const int base = blockIdx.x * kScoreKeysPerBlock;
  if (base >= nv) return;
  const int end = min(nv, base + kScoreKeysPerBlock);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;
  const int hf = lane >> 5;
  if (a.part_hist)
    for (int j = threadIdx.x; j < kScoreParts * kTopBins; j += 256) lhist[j] = 0;
  // The block table entries of the workgroup's key range are read once: a table lookup inside the
  // tile loop would be a load that the data loads depend on, and waiting for it would also wait
  // for the prefetched tile.
  const int per_block = a.pool.per_block;           // 256 / ratio: a power of two
  const int pb_shift = __builtin_ctz(per_block);
  const int lb0 = base >> pb_shift;
  const int n_lb = ((end - 1) >> pb_shift) - lb0 + 1;
  for (int j = threadIdx.x; j < n_lb; j += 256) {
    const int lb = lb0 + j;
    const int phys = lb < a.pool.max_blocks ? a.pool.block_table[(int64_t)seq * a.pool.max_blocks + lb] : -1;
    tbl[j] = (phys >= 0 && phys < a.pool.num_blocks) ? phys : -1;
  }
  __syncthreads();

  // The contraction index d is split as d = 64*hf + 8*s + e for K-step s (0..7) and element e of
  // a lane's 8-wide operand; query and keys use the same split, so each lane holds 64 contiguous
  // dims of its row.
  bf16x8 qa[2][8];
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)i * kMfmaHeads * kMfmaDim;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qa[mb][s] = *reinterpret_cast<const bf16x8*>(q + (32 * mb + col) * kMfmaDim + 64 * hf + 8 * s);
  // weights of the 32 (head) rows this lane accumulates: row = 32*mb + 8*(r/4) + 4*hf + r%4
  float wv[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wv[mb][r] = a.w[(int64_t)i * kMfmaHeads + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3)];

  float* out = a.scores + (int64_t)i * a.ld;
  // Each wave walks 32-key tiles with stride 128; the next two tiles' keys are loaded while the
  // current one is multiplied. fp4 tiles stay packed (32 B + 2 scale bytes per lane) until used.
  struct KeysBf16 {
    bf16x8 v[8];
    bool valid;
  };
  struct KeysFp4 {
    u32x4 w0, w1;
    float s0, s1;
    bool valid;
  };
  using Keys = std::conditional_t<kFp4, KeysFp4, KeysBf16>;
  // Branch-free loads (out-of-range or absent keys read entry 0 of the pool; their scores are
  // written as -inf or not at all), so the prefetch never forces a wait on itself.
  // pool entry of key g (entry 0 when its block is absent; such keys score -inf)
  auto entry_of = [&](int g) -> int64_t {
    g = min(g, end - 1);
    const int phys = tbl[(g >> pb_shift) - lb0];
    return phys >= 0 ? ((int64_t)phys << pb_shift) + (g & (per_block - 1)) : 0;
  };
  auto key_valid = [&](int g) { return tbl[(min(g, end - 1) >> pb_shift) - lb0] >= 0; };
  auto load = [&](Keys& kb, int t0) {
    const int64_t e = entry_of(t0 + col);
    kb.valid = key_valid(t0 + col);
    if constexpr (!kFp4) {
      const uint16_t* row =
          reinterpret_cast<const uint16_t*>(a.pool.data + e * a.pool.entry_bytes) + 64 * hf;
#pragma unroll
      for (int s = 0; s < 8; ++s) kb.v[s] = *reinterpret_cast<const bf16x8*>(row + 8 * s);
    } else {
      const uint8_t* row = a.pool.data + e * a.pool.entry_bytes + 32 * hf;
      // the two E8M0 scale bytes of this lane's 64 dims, one 2-byte read
      const uint16_t scl = *reinterpret_cast<const uint16_t*>(
          reinterpret_cast<const uint8_t*>(a.pool.scale) + e * 4 + 2 * hf);
      kb.w0 = *reinterpret_cast<const u32x4*>(row);
      kb.w1 = *reinterpret_cast<const u32x4*>(row + 16);
      kb.s0 = e8m0_to_f32(scl & 0xffu);
      kb.s1 = e8m0_to_f32(scl >> 8);
    }
  };
  auto operand = [&](const Keys& kb, int s) -> bf16x8 {
    if constexpr (!kFp4) {
      return kb.v[s];
    } else {
      return s < 4 ? fp4x8_to_bf16x8(kb.w0[s], kb.s0) : fp4x8_to_bf16x8(kb.w1[s - 4], kb.s1);
    }
  };
  auto score = [&](const Keys& kb, int t0) {
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 b = operand(kb, s);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], b, acc1, 0, 0, 0);
    }
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      part = fmaf(wv[0][r], fmaxf(acc0[r], 0.f), part);
      part = fmaf(wv[1][r], fmaxf(acc1[r], 0.f), part);
    }
    part += __shfl_xor(part, 32, 64);
    const int g = t0 + col;
    if (hf == 0 && g < end) {
      const float v = kb.valid ? canonical_zero(part) : -INFINITY;
      if (a.part_hist) {
        const uint32_t key = order_key(v);
        lkeys[g - base] = key;
        atomicAdd(&lhist[((g - base) / kScorePartKeys) * kTopBins + (key >> (32 - kTopBits))], 1u);
      } else {
        out[g] = v;
      }
    }
  };
  // three tiles per wave in flight: two loading while one is multiplied
  Keys k0, k1, k2;
  int t0 = base + wave * 32;
  if (t0 < end) {
    load(k0, t0);
    load(k1, t0 + 128);
    for (; t0 < end; t0 += 384) {
      load(k2, t0 + 256);
      score(k0, t0);
      if (t0 + 128 >= end) break;
      load(k0, t0 + 384);
      score(k1, t0 + 128);
      if (t0 + 256 >= end) break;
      load(k1, t0 + 512);
      score(k2, t0 + 256);
    }
  }
  if (a.part_hist)
    finish_parts<kScoreParts>(a, i, blockIdx.x * kScoreParts, base, end, lkeys, lhist, lsorted, wtot);
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4): lane i's bytes land
// at LDS byte address lds + 16i. Issued through inline asm: with the compiler builtin every LDS
// read waits for all outstanding loads (the compiler cannot tell which LDS bytes a load writes),
// which would serialise the prefetch; here the caller waits with wait_vmcnt for exactly the tiles
// it reads. Younger loads or stores issued by the compiler only make such a wait stricter.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// bf16 keys: the same contraction as score_mfma, with the keys streamed into LDS by coalesced
// direct loads (each load instruction moves 1 KB = four whole key rows) instead of row-wise loads
// into operand registers; row-wise loads reach only about 5 TB/s on this access pattern.
// Each wave owns four 8 KB stages (32 keys x 256 B) and keeps three tiles in flight. In a stage,
// 16-byte chunk c of key n sits at chunk c ^ (n % 16) of its row, so the operand reads (32 keys,
// one logical chunk) hit 16 different bank groups per 16 lanes; the loads pick their source
// chunks to match.
constexpr int kDmaStages = 4;

__global__ __launch_bounds__(256, 1) void score_mfma_dma(ScoreArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage[kDmaStages][4][8192];
  __shared__ uint32_t lhist[kScoreParts * kTopBins];
  __shared__ int32_t tbl[kScoreKeysPerBlock / 2 + 2];
  __shared__ uint32_t lkeys[kScoreKeysPerBlock];
  __shared__ uint32_t wtot[kScoreParts * 4];
  const int i = blockIdx.y;
  const int base = blockIdx.x * kScoreKeysPerBlock;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31;
  const int hf = lane >> 5;
  // In decode form the sequence is the query index itself, so the block table of the
  // workgroup's whole key range is read in parallel with the sequence length (which only bounds
  // the range); in prefill form the sequence comes from q_seq first.
  const int seq = (a.qd.seq_lens || !a.qd.q_seq) ? i : a.qd.q_seq[i];
  const int per_block = a.pool.per_block;   // 256 / ratio: a power of two
  const int pb_shift = __builtin_ctz(per_block);
  const int lb0 = base >> pb_shift;
  const int n_lb_max = ((base + kScoreKeysPerBlock - 1) >> pb_shift) - lb0 + 1;
  for (int j = threadIdx.x; j < n_lb_max; j += 256) {
    const int lb = lb0 + j;
    const int phys = lb < a.pool.max_blocks ? a.pool.block_table[(int64_t)seq * a.pool.max_blocks + lb] : -1;
    tbl[j] = (phys >= 0 && phys < a.pool.num_blocks) ? phys : -1;
  }
  const int p = a.qd.seq_lens ? a.qd.seq_lens[i] - 1 : a.qd.q_pos[i];
  const int nv = min(n_visible(p, a.pool.ratio, a.window), n_visible(a.max_pos, a.pool.ratio, a.window));
  if (base >= nv) return;   // uniform, before any barrier
  const int end = min(nv, base + kScoreKeysPerBlock);
  if (a.part_hist)
    for (int j = threadIdx.x; j < kScoreParts * kTopBins; j += 256) lhist[j] = 0;
  __syncthreads();

  // operands as in score_mfma: d = 64*hf + 8*s + e, i.e. lane (key col, hf) takes logical chunk
  // 8*hf + s of its key at K-step s
  bf16x8 qa[2][8];
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)i * kMfmaHeads * kMfmaDim;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qa[mb][s] = *reinterpret_cast<const bf16x8*>(q + (32 * mb + col) * kMfmaDim + 64 * hf + 8 * s);
  float wv[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wv[mb][r] = a.w[(int64_t)i * kMfmaHeads + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3)];
  float* out = a.scores + (int64_t)i * a.ld;

  auto entry_of = [&](int g) -> int64_t {   // entry 0 when the block is absent (scored -inf)
    g = min(g, end - 1);
    const int phys = tbl[(g >> pb_shift) - lb0];
    return phys >= 0 ? ((int64_t)phys << pb_shift) + (g & (per_block - 1)) : 0;
  };
  const uint32_t st0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&stage[0][wave][0]);
  constexpr uint32_t kStageBytes = 4 * 8192;
  // tile m of this wave: keys base + 32*wave + 128*m + [0, 32)
  const int first = base + 32 * wave;
  const int n_mine = first < end ? (end - first + 127) / 128 : 0;
  // load instruction j: LDS bytes 1024j + 16*lane <- key n = 4j + lane/16, chunk (lane%16) ^ (n%16)
  auto issue = [&](int s, int m) {
    const int tb = first + 128 * m;
    int64_t e[8];
    if (per_block >= 32) {
      // uniform: the 32-key tile lies in one block; tiles past the end re-read the last tile's
      // block (in bounds, unused)
      const int gb = min(tb, (end - 1) & ~31);
      const int phys = tbl[(gb >> pb_shift) - lb0];
      const int64_t e0 = (phys >= 0 ? ((int64_t)phys << pb_shift) : 0) + (gb & (per_block - 1));
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = e0 + 4 * j + (lane >> 4);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = entry_of(tb + 4 * j + (lane >> 4));
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // earlier reads of this stage are done
    const uint32_t lds = st0 + s * kStageBytes;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int n = 4 * j + (lane >> 4);
      const int c = (lane & 15) ^ (n & 15);
      lds_dma16(a.pool.data + e[j] * a.pool.entry_bytes + 16 * c, lds + 1024 * j);
    }
  };
  // operand read offsets (bytes within a stage): key col, chunk (8hf + s) ^ (col % 16)
  uint32_t roff[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) roff[s] = wave * 8192 + col * 256 + 16 * ((8 * hf + s) ^ (col & 15));
  auto score = [&](int st, int m) {
    const uint8_t* sb = &stage[st][0][0];
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(sb + roff[s]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], b, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], b, acc1, 0, 0, 0);
    }
    float part = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      part = fmaf(wv[0][r], fmaxf(acc0[r], 0.f), part);
      part = fmaf(wv[1][r], fmaxf(acc1[r], 0.f), part);
    }
    part += __shfl_xor(part, 32, 64);
    const int g = first + 128 * m + col;
    if (hf == 0 && g < end) {
      const bool valid = tbl[(g >> pb_shift) - lb0] >= 0;
      const float v = valid ? canonical_zero(part) : -INFINITY;
      if (a.part_hist) {
        const uint32_t key = order_key(v);
        lkeys[g - base] = key;
        atomicAdd(&lhist[((g - base) / kScorePartKeys) * kTopBins + (key >> (32 - kTopBits))], 1u);
      } else {
        out[g] = v;
      }
    }
  };
  if (n_mine > 0) {
    // three tiles in flight; tiles past the wave's last one load clamped (real) rows, unused
    issue(0, 0);
    issue(1, 1);
    issue(2, 2);
    for (int m = 0; m < n_mine; m += 4) {
      issue(3, m + 3);
      wait_vmcnt<24>();
      score(0, m);
      if (m + 1 >= n_mine) break;
      issue(0, m + 4);
      wait_vmcnt<24>();
      score(1, m + 1);
      if (m + 2 >= n_mine) break;
      issue(1, m + 5);
      wait_vmcnt<24>();
      score(2, m + 2);
      if (m + 3 >= n_mine) break;
      issue(2, m + 6);
      wait_vmcnt<24>();
      score(3, m + 3);
    }
  }
  wait_vmcnt<0>();   // no load may still be writing this workgroup's LDS when it exits
  if (a.part_hist)   // the stages are free now: the sorted pairs use them
    finish_parts<kScoreParts>(a, i, blockIdx.x * kScoreParts, base, end, lkeys, lhist,
                              reinterpret_cast<uint2*>(&stage[0][0][0]), wtot);
}

// Prefill form, bf16 keys: four query tokens per workgroup, one per wave, share every key tile.
// Queries of one sequence see the same keys, so a tile streamed once into LDS serves all of them:
// the key traffic of a prefill chunk drops fourfold and the kernel becomes MFMA-bound. The waves'
// queries are grouped by sequence (consecutive queries of a chunk usually share one): each group
// streams the keys up to its longest visible range, the four waves loading a quarter of each
// tile (two direct loads of four keys each) into a ring of kMStages shared tiles; after a barrier
// every wave whose query is in the group scores the tile. Each query's keys and histograms then go
// through the same hand-off (or plain scores) as in the one-query kernels.
constexpr int kMQ = 4;                       // queries per workgroup (one per wave)
constexpr int kMKeys = kScorePartKeys;       // keys per workgroup: one hand-off part
constexpr int kMParts = kMKeys / kScorePartKeys;
constexpr int kMStages = 3;                  // shared 8 KB tiles in the ring (two in flight)
// LDS: ring 24 KB + per query 1024 keys (16 KB for four queries) and 1024 16-bit bin counts
// packed two to a word (8 KB) + block table: about 50 KB, so that three workgroups (three waves
// per SIMD) share a compute unit and one's barriers, operand reads and hand-off overlap the
// others' MFMA work.
// Launches with explicit sequence ids and at least this many queries take the shared-tile kernel.
// A workgroup whose four queries belong to different sequences streams each sequence's keys in
// turn, which is only cheap when most workgroups hold one sequence and the grid is large; a decode
// batch (one or a few queries per sequence) keeps the one-query kernel.
constexpr int kMultiMinQueries = 256;

__global__ __launch_bounds__(256, 3) void score_mfma_multi(ScoreArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage[kMStages][8192];
  __shared__ uint32_t lhist[kMQ][kMParts * kTopBins / 2];   // counts <= 1024: 16 bits each
  __shared__ uint32_t lkeys[kMQ][kMKeys];
  __shared__ int32_t tbl[kMKeys / 2 + 2];
  __shared__ uint32_t wtot[kMParts * 4];
  __shared__ int32_t gseq[kMQ], gnv[kMQ];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hf = lane >> 5;
  const int base = blockIdx.x * kMKeys;
  const int i = blockIdx.y * kMQ + wave;   // this wave's query
  const bool has_q = i < a.n_q;
  const int iq = min(i, a.n_q - 1);        // in-bounds row for the loads of an absent query
  const int seq = a.qd.q_seq ? a.qd.q_seq[iq] : iq;
  const int p = a.qd.q_pos[iq];
  const int nv = has_q ? min(n_visible(p, a.pool.ratio, a.window),
                             n_visible(a.max_pos, a.pool.ratio, a.window)) : 0;
  const int end_w = min(nv, base + kMKeys);   // this wave's keys: [base, end_w)
  if (lane == 0) {
    gseq[wave] = has_q ? seq : -1;
    gnv[wave] = nv;
  }
  if (a.part_hist)
    for (int j = tid; j < kMQ * kMParts * kTopBins / 2; j += 256) (&lhist[0][0])[j] = 0;

  // this wave's query and head weights (as in score_mfma_dma)
  bf16x8 qa[2][8];
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q) + (int64_t)iq * kMfmaHeads * kMfmaDim;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qa[mb][s] = *reinterpret_cast<const bf16x8*>(q + (32 * mb + col) * kMfmaDim + 64 * hf + 8 * s);
  float wv[2][16];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      wv[mb][r] = a.w[(int64_t)iq * kMfmaHeads + 32 * mb + 8 * (r >> 2) + 4 * hf + (r & 3)];
  __syncthreads();   // gseq / gnv / histograms ready

  const int per_block = a.pool.per_block;   // 256 / ratio: a power of two
  const int pb_shift = __builtin_ctz(per_block);
  const int lb0 = base >> pb_shift;
  const uint32_t st0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)&stage[0][0]);
  uint32_t roff[8];   // operand read offsets within a tile: key col, chunk (8hf + s) ^ (col % 16)
#pragma unroll
  for (int s = 0; s < 8; ++s) roff[s] = col * 256 + 16 * ((8 * hf + s) ^ (col & 15));

  for (int w0 = 0; w0 < kMQ; ++w0) {
    const int sq = gseq[w0];
    bool lead = sq >= 0;   // w0 is the first wave of its sequence
    int nv_s = 0;
    for (int w1 = 0; w1 < kMQ; ++w1) {
      if (gseq[w1] != sq) continue;
      if (w1 < w0) lead = false;
      nv_s = max(nv_s, gnv[w1]);
    }
    const int end_s = min(nv_s, base + kMKeys);
    if (!lead || base >= end_s) continue;   // uniform
    const bool mine = has_q && seq == sq;   // uniform per wave
    __syncthreads();   // the previous group's readers of tbl and of the tiles are done
    const int n_lb = ((end_s - 1) >> pb_shift) - lb0 + 1;
    for (int j = tid; j < n_lb; j += 256) {
      const int lb = lb0 + j;
      const int phys = lb < a.pool.max_blocks ? a.pool.block_table[(int64_t)sq * a.pool.max_blocks + lb] : -1;
      tbl[j] = (phys >= 0 && phys < a.pool.num_blocks) ? phys : -1;
    }
    __syncthreads();
    const int n_tiles = (end_s - base + 31) / 32;
    // tile t into stage t % kMStages: this wave moves keys 8 wave .. 8 wave + 7 (two loads of
    // four keys); keys past the group's range re-read its last key (in bounds, unused)
    auto issue = [&](int t) {
      const int tb = base + 32 * t;
      const uint32_t lds = st0 + (t % kMStages) * 8192;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = 8 * wave + 4 * j + (lane >> 4);
        const int g = min(tb + n, end_s - 1);
        const int phys = tbl[(g >> pb_shift) - lb0];
        const int64_t e = phys >= 0 ? ((int64_t)phys << pb_shift) + (g & (per_block - 1)) : 0;
        const int c = (lane & 15) ^ (n & 15);
        lds_dma16(a.pool.data + e * a.pool.entry_bytes + 16 * c, lds + 1024 * (2 * wave + j));
      }
    };
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // tbl reads of the address math above
#pragma unroll
    for (int t = 0; t < kMStages - 1; ++t) issue(t);
    for (int t = 0; t < n_tiles; ++t) {
      wait_vmcnt<2 * (kMStages - 2)>();   // this wave's loads of tile t are done
      __syncthreads();                    // everyone's are, and tile t - 1 has been read
      issue(t + kMStages - 1);
      if (mine) {
        const uint8_t* sb = &stage[t % kMStages][0];
        f32x16 acc0 = {}, acc1 = {};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 b = *reinterpret_cast<const bf16x8*>(sb + roff[s]);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], b, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], b, acc1, 0, 0, 0);
        }
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          part = fmaf(wv[0][r], fmaxf(acc0[r], 0.f), part);
          part = fmaf(wv[1][r], fmaxf(acc1[r], 0.f), part);
        }
        part += __shfl_xor(part, 32, 64);
        const int g = base + 32 * t + col;
        if (hf == 0 && g < end_w) {
          const bool valid = tbl[(g >> pb_shift) - lb0] >= 0;
          const float v = valid ? canonical_zero(part) : -INFINITY;
          if (a.part_hist) {
            const uint32_t key = order_key(v);
            lkeys[wave][g - base] = key;
            const uint32_t bin = key >> (32 - kTopBits);   // one part per workgroup
            atomicAdd(&lhist[wave][bin >> 1], 1u << (16 * (bin & 1u)));
          } else {
            a.scores[(int64_t)i * a.ld + g] = v;
          }
        }
      }
    }
    wait_vmcnt<0>();   // no load may still be writing a tile when the ring is reused
  }
  if (a.part_hist && has_q && base < end_w) {
    // each wave hands off its own query's part (its keys and counts are its own LDS writes)
    finish_part_wave(a, i, blockIdx.x, base, end_w, lkeys[wave], lhist[wave], lane);
  }
}

// One thread per key (workgroups of kScorePartKeys keys, four per thread); query rows and weights
// staged in LDS as float.
__global__ __launch_bounds__(256) void score_generic(ScoreArgs a) {
  extern __shared__ float sm[];
  __shared__ uint32_t lhist[kTopBins];
  __shared__ uint32_t lkeys[kScorePartKeys];
  __shared__ uint2 lsorted[kScorePartKeys];
  __shared__ uint32_t wtot[4];
  const int i = blockIdx.y;
  int seq, p;
  query_at(a.qd, i, &seq, &p);
  const int nv = min(n_visible(p, a.pool.ratio, a.window), n_visible(a.max_pos, a.pool.ratio, a.window));
  const int base = blockIdx.x * kScorePartKeys;
  if (base >= nv) return;
  const int H = a.n_heads, Dk = a.pool.dim;
  float* qs = sm;
  float* ws = sm + H * Dk;
  for (int e = threadIdx.x; e < H * Dk; e += 256) {
    int64_t off = (int64_t)i * H * Dk + e;
    qs[e] = a.q_dtype == F32 ? reinterpret_cast<const float*>(a.q)[off]
                             : bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[off]);
  }
  for (int h = threadIdx.x; h < H; h += 256) ws[h] = a.w[(int64_t)i * H + h];
  if (a.part_hist)
    for (int j = threadIdx.x; j < kTopBins; j += 256) lhist[j] = 0;
  __syncthreads();
  for (int r = 0; r < kScorePartKeys / 256; ++r) {
    const int g = base + threadIdx.x + 256 * r;
    if (g >= nv) break;
    const int64_t idx = entry_index(a.pool, seq, g);
    float v = -INFINITY;
    if (idx >= 0) {
      const uint8_t* row = a.pool.data + idx * a.pool.entry_bytes;
      float total = 0.f;
      for (int h = 0; h < H; ++h) {
        float dot = 0.f;
        for (int d = 0; d < Dk; ++d) {
          float kd;
          if (a.pool.dtype == F32) {
            kd = reinterpret_cast<const float*>(row)[d];
          } else if (a.pool.dtype == BF16) {
            kd = bf16_to_f32(reinterpret_cast<const uint16_t*>(row)[d]);
          } else {
            uint32_t byte = row[d >> 1];
            uint32_t nib = (d & 1) ? (byte >> 4) : (byte & 0xfu);
            const uint8_t* scl = reinterpret_cast<const uint8_t*>(a.pool.scale) + idx * (Dk / 32);
            kd = fp4_to_f32(nib) * e8m0_to_f32(scl[d >> 5]);
          }
          dot = fmaf(qs[h * Dk + d], kd, dot);
        }
        total = fmaf(ws[h], fmaxf(dot, 0.f), total);
      }
      v = canonical_zero(total);
    }
    if (a.part_hist) {
      const uint32_t key = order_key(v);
      lkeys[g - base] = key;
      atomicAdd(&lhist[key >> (32 - kTopBits)], 1u);
    } else {
      a.scores[(int64_t)i * a.ld + g] = v;
    }
  }
  if (a.part_hist)
    finish_parts<1>(a, i, blockIdx.x, base, min(nv, base + kScorePartKeys), lkeys, lhist, lsorted, wtot);
}

hipError_t launch_index_score(const ScoreArgs& a, hipStream_t s) {
  const int max_nv = (a.max_pos - a.window + 1 > 0)
                         ? (a.max_pos - a.window + 1 + a.pool.ratio - 1) / a.pool.ratio
                         : 0;
  if (max_nv == 0 || a.n_q == 0) return hipSuccess;
  const bool mfma = a.n_heads == kMfmaHeads && a.pool.dim == kMfmaDim && a.q_dtype == BF16 &&
                    (a.pool.dtype == BF16 || a.pool.dtype == FP4);
  if (mfma) {
    dim3 grid((max_nv + kScoreKeysPerBlock - 1) / kScoreKeysPerBlock, a.n_q);
    if (a.pool.dtype == BF16 && a.qd.q_seq && a.n_q >= kMultiMinQueries) {
      // a prefill chunk: runs of queries of one sequence share the key stream, kMQ per workgroup
      grid.x = (max_nv + kMKeys - 1) / kMKeys;
      grid.y = (a.n_q + kMQ - 1) / kMQ;
      hipLaunchKernelGGL(score_mfma_multi, grid, dim3(256), 0, s, a);
    } else if (a.pool.dtype == BF16) {
      hipLaunchKernelGGL(score_mfma_dma, grid, dim3(256), 0, s, a);
    } else {
      hipLaunchKernelGGL(score_mfma<true>, grid, dim3(256), 0, s, a);
    }
  } else {
    dim3 grid((max_nv + kScorePartKeys - 1) / kScorePartKeys, a.n_q);
    size_t lds = sizeof(float) * ((size_t)a.n_heads * a.pool.dim + a.n_heads);
    hipLaunchKernelGGL(score_generic, grid, dim3(256), lds, s, a);
  }
  return hipGetLastError();
}

}  // namespace hyb
