// Device-side helpers shared by the MSA kernels (gfx950 / CDNA4).
//
// Formats follow the OCP definitions of E2M1 (FP4) and E4M3 (FP8), the
// element formats of the NVFP4 and FP8 caches in "vLLM 為 MiniMax-M3.1-Flash
// 提供 Day-0 支援" (sections "What is new in the MiniMax-M3.1 architecture"
// and "NVIDIA Blackwell optimized MSA kernels").
//
// Every contraction in this library runs on the f16 MFMA with fp32
// accumulation.  FP8 and NVFP4 values (and NVFP4 values re-rounded to E4M3)
// are exact in f16, so the products are exact; the FP8/FP4 MFMA forms were
// measured to accumulate with a relative error near 2e-5 of sum|a*b|, which
// is too coarse for a top-16 selection that must agree with an fp64 oracle
// whenever the 16th and 17th block scores differ by more than 1e-5.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 128;        // tokens per block / page
constexpr int kHeadDim = 128;
constexpr int kGroups = 4;         // GQA groups = KV heads
constexpr int kHeadsPerGroup = 16;
constexpr int kHeads = kGroups * kHeadsPerGroup;
constexpr int kTopK = 16;
constexpr int kNvfp4RowBytes = kHeadDim / 2;     // codes per 128-dim row
constexpr int kNvfp4ScaleBytes = kHeadDim / 16;  // E4M3 scales per row
// Word 3 of a raw buffer resource on gfx950: 32-bit data format, no swizzle,
// no index stride (byte offsets only).
constexpr int kBufferFlags = 0x00020000;

// ------------------------------------------------------------------ MFMA
__device__ __forceinline__ f4 mfma_16x16x32(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f4 mfma_16x16x16(h4 a, h4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ decode
// Two E4M3 bytes (low or high half-word of w) -> two exact f16.
template <bool HI>
__device__ __forceinline__ h2 fp8x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}
// Two E2M1 codes (byte B of w, low nibble first) -> two exact f16.  A unit
// scale is used: the conversion only honours the exponent of its scale.
template <int B>
__device__ __forceinline__ h2 fp4x2_to_h2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B);
}
__device__ __forceinline__ h8 cat(h2 a, h2 b, h2 c, h2 d) {
  return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// 8 E4M3 bytes (two dwords) -> 8 f16, element order preserved.
__device__ __forceinline__ h8 fp8x8_to_h8(uint32_t lo, uint32_t hi) {
  return cat(fp8x2_to_h2<false>(lo), fp8x2_to_h2<true>(lo), fp8x2_to_h2<false>(hi),
             fp8x2_to_h2<true>(hi));
}
// 8 E2M1 codes (one dword, even element in the low nibble) -> 8 f16.
__device__ __forceinline__ h8 fp4x8_to_h8(uint32_t w) {
  return cat(fp4x2_to_h2<0>(w), fp4x2_to_h2<1>(w), fp4x2_to_h2<2>(w), fp4x2_to_h2<3>(w));
}
// E4M3 byte -> f16 (exact).
__device__ __forceinline__ _Float16 e4m3_to_h(uint32_t byte) {
  return fp8x2_to_h2<false>(byte & 0xFFu)[0];
}
__device__ __forceinline__ float e4m3_to_f(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte & 0xFFu, 0);
}

// FP8-rounded NVFP4 decode: a 256 x 8 byte table (scale byte x magnitude)
// of E4M3 values.  8 codes of one dword (one scale) -> 8 FP8 bytes with one
// byte permute per 4 codes plus a sign XOR.  The bytes come out in the order
// (0,2,4,6 | 1,3,5,7); callers lay the other operand out the same way.
__device__ __forceinline__ h8 fp4x8_lut_to_h8(uint32_t w, uint32_t lut_lo, uint32_t lut_hi) {
  const uint32_t me = w & 0x07070707u, mo = (w >> 4) & 0x07070707u;
  const uint32_t fe = __builtin_amdgcn_perm(lut_hi, lut_lo, me) ^ ((w << 4) & 0x80808080u);
  const uint32_t fo = __builtin_amdgcn_perm(lut_hi, lut_lo, mo) ^ (w & 0x80808080u);
  return fp8x8_to_h8(fe, fo);
}
// Element order produced by fp4x8_lut_to_h8: position e holds element kLutPerm[e].
__device__ __forceinline__ int lut_perm(int e) { return (e & 3) * 2 + (e >> 2); }

// ------------------------------------------------------------------ encode
// E4M3 value of a byte, as float (exact; NaN for 0x7F/0xFF).
__host__ __device__ inline float e4m3_value(uint32_t byte) {
  const uint32_t s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  float v;
  if (e == 15u && m == 7u) {
    v = __builtin_nanf("");
  } else if (e == 0u) {
    v = (float)m * 0.001953125f;                  // m * 2^-9
  } else {
    v = (1.0f + (float)m * 0.125f) * __builtin_ldexpf(1.0f, (int)e - 7);
  }
  return s ? -v : v;
}
// Round a finite float to E4M3, nearest-even, saturating at +-448; the sign
// bit is the float's sign bit.
__host__ __device__ inline uint32_t e4m3_encode(float x) {
  uint32_t bits;
  __builtin_memcpy(&bits, &x, 4);
  const uint32_t sign = (bits >> 31) << 7;
  const float a = __builtin_fabsf(x);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {                     // below 2^-6: subnormal grid of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f); // exact scaling, RNE; 8 -> 0x08 = 2^-6
  } else {
    uint32_t ab;
    __builtin_memcpy(&ab, &a, 4);
    int e = (int)((ab >> 23) & 0xFFu) - 127;      // -6 .. 8
    const float m = a * __builtin_ldexpf(1.0f, -e);   // [1, 2), exact
    uint32_t q = (uint32_t)__builtin_rintf((m - 1.0f) * 8.0f);
    if (q == 8u) { q = 0u; ++e; }
    code = ((uint32_t)(e + 7) << 3) | q;
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}
// Round a finite float to E2M1 (nearest-even on 0,.5,1,1.5,2,3,4,6), clamped
// to 6; sign = the float's sign bit.
__host__ __device__ inline uint32_t e2m1_encode(float x) {
  uint32_t bits;
  __builtin_memcpy(&bits, &x, 4);
  const float a = __builtin_fabsf(x);
  const uint32_t code = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                        (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                        (uint32_t)(a > 5.0f);
  return ((bits >> 31) << 3) | code;
}
// The two roundings above with gfx950's conversion instructions, two values
// at a time.  For every input that is not NaN they give the same bits as
// e4m3_encode / e2m1_encode (compared over all 2^32 float patterns); NaN
// inputs have no defined code in either.  The E4M3 instruction turns
// magnitudes beyond 464 into the NaN code, so its inputs are first clamped
// to +-448, which is where the saturating encoder sends them; the E2M1 one
// saturates at 6 by itself (its scale operand is 1, i.e. none).
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b) {   // byte 0: a, byte 1: b
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_fmed3f(a, -448.0f, 448.0f),
                                                   __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f), 0, false) &
         0xFFFFu;
}
__device__ __forceinline__ uint32_t e2m1_encode2(float a, float b) {   // low nibble: a, high nibble: b
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0) & 0xFFu;
}
__host__ __device__ inline float e2m1_magnitude(uint32_t m) {
  const float t[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};
  return t[m & 7u];
}

// FP8-rounded NVFP4 table: 256 scale bytes x 8 magnitudes of E4M3 bytes, as
// two dwords per scale ("NVFP4 MSA kernel": 256 scales x 8 magnitudes, every
// product pre-rounded to FP8, 2 KB in LDS).  Undefined scale bytes map to NaN.
__device__ inline void build_fp8_lut(uint32_t* lut) {
  for (int s = threadIdx.x; s < 256; s += blockDim.x) {
    const bool bad = (s & 0x80) || s == 0x7F;
    const float sv = e4m3_value((uint32_t)s);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t byte = bad ? 0x7Fu : e4m3_encode2(e2m1_magnitude((uint32_t)m) * sv, 0.0f) & 0xFFu;
      w[m >> 2] |= byte << (8 * (m & 3));
    }
    lut[2 * s] = w[0];
    lut[2 * s + 1] = w[1];
  }
}

// ------------------------------------------------------------------ ordering
// Monotone map float -> uint32 (NaN lowest, -0 == +0).
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;
  if (x == 0.0f) x = 0.0f;
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 2^x with the hardware exponential alone (results below the smallest normal
// float flush to zero; exact enough for softmax weights in [0, 1]).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ waves
// The number of lanes for which c holds, counted in 32-bit halves (a 64-bit
// count would be compared on the vector unit).
__device__ __forceinline__ uint32_t ballot_count(bool c) {
  const uint64_t b = __ballot(c);
  return (uint32_t)__builtin_popcount((uint32_t)b) + (uint32_t)__builtin_popcount((uint32_t)(b >> 32));
}

// Cross-lane exchanges on the vector unit, with no LDS round trip.
// swap32(a, b): gfx950's 32-lane swap trades lanes 32..63 of a for lanes
// 0..31 of b, so it returns {a.lo | b.lo, a.hi | b.hi} (halves of 32 lanes).
// swap16(a, b): the row swap trades rows 1 and 3 of a for rows 0 and 2 of b,
// returning {a.r0 b.r0 a.r2 b.r2, a.r1 b.r1 a.r3 b.r3} (rows of 16 lanes).
// dpp(v, ctrl): lane l reads the lane of its 16-lane row that ctrl names.
// (Lane mappings fixed by an in-bounds probe.)
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
constexpr int kDppQuad1032 = 0xB1;       // lanes 4k + {1, 0, 3, 2}
constexpr int kDppQuad2301 = 0x4E;       // lanes 4k + {2, 3, 0, 1}
constexpr int kDppRowHalfMirror = 0x141; // lane 7 - i within each 8 lanes
constexpr int kDppRowMirror = 0x140;     // lane 15 - i within each row
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float max16(float v) {   // max over the 16 lanes of a row
  v = fmaxf(v, dpp<kDppQuad1032>(v));
  v = fmaxf(v, dpp<kDppQuad2301>(v));
  v = fmaxf(v, dpp<kDppRowHalfMirror>(v));
  return fmaxf(v, dpp<kDppRowMirror>(v));
}
__device__ __forceinline__ float max_over_quarters(float v) {   // lanes l, l^16, l^32, l^48
  float a = v, b = v;
  swap32(a, b);             // a = v.lo | v.lo, b = v.hi | v.hi
  float c = fmaxf(a, b), d = c;
  swap16(c, d);             // rows 0 and 1 of the pair maxima, in every row
  return fmaxf(c, d);
}
__device__ __forceinline__ float sum_over_quarters(float v) {   // the same sum in every lane
  float a = v, b = v;
  swap32(a, b);
  float c = a + b, d = c;
  swap16(c, d);
  return c + d;
}
// Lane l = 16Q + n returns the maximum of value Q over lanes n, n+16, n+32,
// n+48: two half swaps pair value 0 (lanes below 32) and value 2 (above)
// across halves, and values 1 and 3 likewise; one row swap then pairs rows.
__device__ __forceinline__ float quarter_max4(f4 v) {
  float a = v[0], b = v[2], c = v[1], d = v[3];
  swap32(a, b);             // a = v0.lo | v2.lo, b = v0.hi | v2.hi
  swap32(c, d);             // c = v1.lo | v3.lo, d = v1.hi | v3.hi
  float e = fmaxf(a, b), f = fmaxf(c, d);   // halves: value 0 | value 2, value 1 | value 3
  swap16(e, f);             // e = e.r0 f.r0 e.r2 f.r2, f = e.r1 f.r1 e.r3 f.r3
  return fmaxf(e, f);
}
// IEEE 754-2019 maximum (a NaN operand gives NaN).  gfx950 folds chains of
// it into v_maximum3_f32 and needs no quieting of the operands, which fmaxf
// (maxNum) costs on values the compiler cannot prove canonical, such as MFMA
// results and cross-lane moves.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// Two values: lane l = 32h + 16q + n returns the maximum of value h over
// lanes n, n+16, n+32, n+48 (one half swap, then one row swap).
__device__ __forceinline__ float quarter_max2(float v0, float v1) {
  float a = v0, b = v1;
  swap32(a, b);             // a = v0.lo | v1.lo, b = v0.hi | v1.hi
  float e = vmax(a, b), f = e;
  swap16(e, f);             // e = rows 0, 0, 2, 2 and f = rows 1, 1, 3, 3 of the half maxima
  return vmax(e, f);
}
// Max over the 64 lanes of 4 values.  Lane l returns the maximum of value
// g = 2*(l/32) + (l/16)%2.
__device__ __forceinline__ float wave_max4(f4 v) {
  return max16(quarter_max4(v));
}
__device__ __forceinline__ void lds_wait() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

}  // namespace msa
