// Device-side helpers shared by the HIP kernels of the hybrid attention library (gfx950 only).
//
// Storage formats (OCP E4M3 with a float32 scale per entry, OCP MX E2M1 with an E8M0 scale per
// 32 elements), the paged-pool address rule (one logical block = 256 native positions for every
// compression rate, per the "vLLM side" list of the vLLM DeepSeek-V4 day-0 post), the visibility
// rule and RoPE angles (formed and reduced in double precision).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hyb_internal.h"

namespace hyb {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// Two floats -> packed bf16x2 (low half = a), rounded to nearest even: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// OCP E4M3 (no inf, max 448, NaN = S.1111.111) -> float, exact. Normal codes map straight onto a
// bf16 bit pattern (exponent + 120, mantissa << 4); subnormals are m * 2^-9.
__device__ __forceinline__ float fp8_to_f32(uint32_t c) {
  uint32_t u = c & 0x7fu;
  float mag = (u >= 8u) ? __uint_as_float(((u << 4) + 0x3c00u) << 16) : (float)u * 0x1p-9f;
  if (u == 0x7fu) mag = __builtin_nanf("");
  return (c & 0x80u) ? -mag : mag;
}

// E4M3 code -> bf16 bits, exact (every finite E4M3 value is a bf16 value).
__device__ __forceinline__ uint32_t fp8_to_bf16(uint32_t c) {
  return __float_as_uint(fp8_to_f32(c)) >> 16;
}

// OCP MX E2M1 nibble -> float (without its block scale): 0, .5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float fp4_to_f32(uint32_t nib) {
  uint32_t m = nib & 7u;
  float mag = (m < 2u) ? 0.5f * (float)m
                       : __uint_as_float((((m >> 1) + 126u) << 23) | ((m & 1u) << 22));
  return (nib & 8u) ? -mag : mag;
}

// E8M0 scale byte -> 2^(e - 127) (255 is not produced by the quantiser; it decodes as inf here).
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  return e == 0u ? 0x1p-127f : __uint_as_float(e << 23);
}

// A physical block id >= num_blocks in a table: recorded in the pool's error word when there is
// one (the block still counts as absent).
__device__ __forceinline__ void note_bad_page(const PoolDev& p, int phys) {
  if (phys >= p.num_blocks && p.err != nullptr) atomicOr(p.err, kErrBadPage);
}

// Index of entry g of sequence `seq` in the flattened [num_blocks * per_block] entry array, or -1
// when its block is absent or out of range (then nothing is read or written).
__device__ __forceinline__ int64_t entry_index(const PoolDev& p, int seq, int g) {
  if (g < 0) return -1;
  int lb = g / p.per_block;
  if (lb >= p.max_blocks) return -1;
  int phys = p.block_table[(int64_t)seq * p.max_blocks + lb];
  note_bad_page(p, phys);
  if (phys < 0 || phys >= p.num_blocks) return -1;
  return (int64_t)phys * p.per_block + (g - lb * p.per_block);
}

__device__ __forceinline__ int window_start(int p, int window) {
  int ws = p - window + 1;
  return ws > 0 ? ws : 0;
}

// Compressed entries visible to a query at position p: ceil(window_start / ratio).
__device__ __forceinline__ int n_visible(int p, int ratio, int window) {
  return (window_start(p, window) + ratio - 1) / ratio;
}

// RoPE angle brought to [-pi, pi] in double precision by Cody-Waite additive range reduction
// (W. J. Cody and W. Waite, "Software Manual for the Elementary Functions", 1980): k * 2pi is
// subtracted with 2pi split in three parts (24 + 24 + 53 bits). For |angle| < 2^31, k < 2^29, so
// the first two products are exact and the residue keeps full double precision.
__device__ __forceinline__ double rope_reduce(double ang) {
  constexpr double kInv2Pi = 0.15915494309189535;
  constexpr double kP1 = 6.2831854820251465;        // 2pi rounded to 24 bits
  constexpr double kP2 = -1.7484555314695172e-07;   // next 24 bits
  constexpr double kP3 = -6.8604979977715316e-15;   // the rest, to double precision
  const double k = rint(ang * kInv2Pi);
  return ((ang - k * kP1) - k * kP2) - k * kP3;
}

// cos / sin of pos * base^(-2i / rope_dim), formed and reduced in double precision (sincos then
// stays on its short path instead of a large-argument reduction).
__device__ __forceinline__ void rope_cs(double pos, int i, int rope_dim, double base, float* c,
                                        float* s) {
  const double theta = exp(-2.0 * (double)i / (double)rope_dim * log(base));
  double sn, cs;
  sincos(rope_reduce(pos * theta), &sn, &cs);
  *c = (float)cs;
  *s = (float)sn;
}

// cos / sin of pos * theta for a frequency theta formed on the host: the angle is formed and
// reduced in double precision, the reduced angle's cos / sin are taken in float (a few float
// ulps; the double path above costs far more registers and time).
__device__ __forceinline__ void rope_cs_theta(double pos, double theta, float* c, float* s) {
  sincosf((float)rope_reduce(pos * theta), s, c);
}

// Query i -> (sequence, position).
__device__ __forceinline__ void query_at(const QueryDev& q, int i, int* seq, int* pos) {
  if (q.seq_lens) {
    *seq = i;
    *pos = q.seq_lens[i] - 1;
  } else {
    *seq = q.q_seq ? q.q_seq[i] : i;
    *pos = q.q_pos[i];
  }
}

// Order-preserving 32-bit key of a float (larger float -> larger key); -0.0 maps to +0.0's key.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS round trips): shifts by
// 1, 2, 4, 8 inside each row of 16 lanes, then row 0's / rows 0-1's totals are broadcast into the
// rows above (lanes a DPP move does not feed keep the 0 passed as `old`).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += __builtin_amdgcn_update_dpp(0u, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0u, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0u, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0u, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0u, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0u, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace hyb
