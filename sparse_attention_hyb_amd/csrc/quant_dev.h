// Quantised stores of computed rows: fp8 E4M3 with one float32 scale per row, and OCP MX fp4
// E2M1 with one E8M0 exponent byte per 32 values. The pages name an fp8 attention cache and an
// fp4 indexer cache ("Day-0 support for DeepSeek V4 Pro and Flash on vLLM", the paragraph after
// the "four moves" list) and fused quantising writes (its "vLLM side" list: compressor + cache
// insert, inverse RoPE + fp8 quant); the encodings are the readings stated with hyb_dtype:
//   fp8 row:   scale = amax / 448 (1 for an all-zero row), code = E4M3 nearest to x / scale,
//              ties to the even code, magnitudes above 448 saturating;
//   fp4 block: e = floor(log2 amax) - 2 clamped to [-100, 60], byte e + 127, code = E2M1 nearest
//              to x * 2^-e, ties to the even code, saturating at 6.
// Every step is float32: the scale and the quotients are correctly rounded divisions, the
// power-of-two scaling is exact, and the rounding to the code is rintf (ties to even).
#pragma once

#include "common.h"

namespace hyb {

// E4M3 code of v: |v| < 2^-6 counts steps of 2^-9 (a count of 8 is the code of 2^-6), else the
// mantissa is rounded to 3 bits and a carry moves into the exponent field.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;   // -6 .. 8
    const float m = ldexpf(a, -e);                                      // [1, 2), exact
    code = ((uint32_t)(e + 7) << 3) + (uint32_t)rintf((m - 1.0f) * 8.0f);
  }
  return code | sign;
}

// E2M1 code of v (low 4 bits): below 1 in steps of 0.5 (a count of 2 is the code of 1.0), else a
// 1-bit mantissa with carry; 6 and above saturate.
__device__ __forceinline__ uint32_t f32_to_e2m1(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 28) & 0x8u;
  const float a = fabsf(v);
  uint32_t code;
  if (!(a < 6.0f)) {
    code = 7u;
  } else if (a < 1.0f) {
    code = (uint32_t)rintf(a * 2.0f);
  } else {
    const int e = (int)((__float_as_uint(a) >> 23) & 0xffu) - 127;   // 0 .. 2
    const float m = ldexpf(a, -e);
    code = ((uint32_t)(e + 1) << 1) + (uint32_t)rintf((m - 1.0f) * 2.0f);
  }
  return code | sign;
}

// Shared exponent of an fp4 block from its largest magnitude: floor(log2 amax) - 2 read from the
// exponent field (zero and subnormal maxima fall to the lower clamp).
__device__ __forceinline__ int mx_block_exponent(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xffu) - 129;
  return e < -100 ? -100 : (e > 60 ? 60 : e);
}

// kVec codes of one chunk as bytes (fp8) or nibbles (fp4, element 2m in the low nibble of byte m),
// stored with one write at byte offset `off` of the row.
template <int kBytes>
__device__ __forceinline__ void store_bytes(uint8_t* dst, const uint32_t (&b)[kBytes]) {
  if constexpr (kBytes == 8) {
    *reinterpret_cast<u32x2*>(dst) =
        u32x2{b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24), b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24)};
  } else if constexpr (kBytes == 4) {
    *reinterpret_cast<uint32_t*>(dst) = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
  } else if constexpr (kBytes == 2) {
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(b[0] | (b[1] << 8));
  } else {
    *dst = (uint8_t)b[0];
  }
}

// Entry idx of an FP8_E4M3 or FP4_E2M1 pool from one wave: lane holds chunks c = lane + 64 j
// (j < kJ, c < nchunks) of kVec consecutive values each. Every lane of the wave must call it.
// fp4 needs 32 % kVec == 0 and nchunks * kVec % 32 == 0 (a block is 32 / kVec adjacent lanes).
template <int kVec, int kJ>
__device__ __forceinline__ void store_quantized(const PoolDev& p, int64_t idx, int lane, int nchunks,
                                                const float (&y)[kJ][kVec]) {
  uint8_t* row = p.data + idx * p.entry_bytes;
  if (p.dtype == FP8) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < kJ; ++j)
      if (lane + 64 * j < nchunks)
#pragma unroll
        for (int e = 0; e < kVec; ++e) amax = fmaxf(amax, fabsf(y[j][e]));
    amax = wave_max(amax);
    const float scale = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int c = lane + 64 * j;
      if (c < nchunks) {
        uint32_t b[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) b[e] = f32_to_e4m3(__fdiv_rn(y[j][e], scale));
        store_bytes<kVec>(row + c * kVec, b);
      }
    }
    if (lane == 0) reinterpret_cast<float*>(const_cast<void*>(p.scale))[idx] = scale;
  } else {
    constexpr int kG = 32 / kVec;   // lanes per block
    uint8_t* sc = reinterpret_cast<uint8_t*>(const_cast<void*>(p.scale)) + idx * (p.dim / 32);
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int c = lane + 64 * j;
      float bmax = 0.f;
      if (c < nchunks)
#pragma unroll
        for (int e = 0; e < kVec; ++e) bmax = fmaxf(bmax, fabsf(y[j][e]));
#pragma unroll
      for (int o = 1; o < kG; o <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, o, 64));
      const int ex = mx_block_exponent(bmax);
      if (c < nchunks) {
        uint32_t b[kVec / 2];
#pragma unroll
        for (int m = 0; m < kVec / 2; ++m)
          b[m] = f32_to_e2m1(ldexpf(y[j][2 * m], -ex)) | (f32_to_e2m1(ldexpf(y[j][2 * m + 1], -ex)) << 4);
        store_bytes<kVec / 2>(row + c * (kVec / 2), b);
        if ((c * kVec) % 32 == 0) sc[c * kVec / 32] = (uint8_t)(ex + 127);
      }
    }
  }
}

}  // namespace hyb
