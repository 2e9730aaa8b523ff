// Device-side helpers shared by the HIP kernels of the MoE layer (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_rocm.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(4))) int i32x4_t;

constexpr int kWave = 64;

// ---- bf16 <-> fp32 (round to nearest even; inputs are finite) -------------
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// ---- silu / sigmoid in fp32 ---------------------------------------------------
// 1 / (1 + e^-g) with the hardware reciprocal (about 1 ulp) instead of an
// IEEE division; the results are stored as bf16.
__device__ __forceinline__ float sigmoidf_(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// ---- MXFP8 element and scale (OCP E4M3FN, E8M0) --------------------------------
// floor(log2 a) of a positive finite fp32 value, read from its bit fields.
__device__ __forceinline__ int floor_log2_bits(float a) {
  uint32_t b = __float_as_uint(a) & 0x7FFFFFFFu;
  int ef = (int)(b >> 23);
  if (ef != 0) return ef - 127;
  uint32_t m = b & 0x7FFFFFu;
  return -149 + (31 - __clz((int)m));
}

// Scale exponent of a block from its absolute maximum: clamp(floor(log2 amax)-8,
// -127, 127); an all-zero block takes -127.  Returns the E8M0 code (e + 127).
__device__ __forceinline__ int e8m0_code(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e = floor_log2_bits(amax) - 8;
  e = e < -127 ? -127 : (e > 127 ? 127 : e);
  return e + 127;
}

// 2^k as fp32 for k in [-127, 127] (exact, including the subnormal 2^-127).
__device__ __forceinline__ float exp2i(int k) {
  if (k >= -126) return __uint_as_float((uint32_t)(k + 127) << 23);
  return __uint_as_float(1u << (k + 149));
}

// E4M3FN encode of y = v * 2^-e, with the scaling done exactly.  v is a bf16
// value and e in [-127, 127], so v * 2^-e may leave the fp32 range only above
// 2^128, which saturates anyway; below the E4M3 grid everything rounds in the
// integer domain.  Round to nearest even, saturate to 448, keep the sign.
__device__ __forceinline__ uint32_t e4m3_from_scaled(float v, int e) {
  uint32_t bits = __float_as_uint(v);
  uint32_t sign = (bits >> 24) & 0x80u;
  uint32_t a = bits & 0x7FFFFFFFu;
  if (a == 0) return sign;
  // exponent of |v| and its 24-bit significand (bf16 inputs are normal or
  // subnormal fp32; handle both)
  int ev = (int)(a >> 23);
  uint32_t sig;
  int E;                       // |v| = sig * 2^(E - 23), sig in [2^23, 2^24)
  if (ev != 0) {
    sig = (a & 0x7FFFFFu) | 0x800000u;
    E = ev - 127;
  } else {
    uint32_t m = a;
    int lz = __clz((int)m) - 8;  // shift to put the top bit at bit 23
    sig = m << lz;
    E = -126 - lz;
  }
  int Ey = E - e;              // exponent of |y|
  // quantum exponent: max(Ey, -6) - 3
  int qe = (Ey > -6 ? Ey : -6) - 3;
  // n = |y| / 2^qe = sig * 2^(Ey - 23 - qe); round to nearest even
  int sh = 23 + qe - Ey;       // >= 20 (qe >= Ey - 3)
  uint32_t n;
  if (sh >= 32) {
    n = 0;                     // sig < 2^24 < 2^(sh-1): below half a quantum
  } else {
    uint32_t q = sig >> sh;
    uint32_t rem = sig & ((1u << sh) - 1u);
    uint32_t half = 1u << (sh - 1);
    n = q + ((rem > half || (rem == half && (q & 1u))) ? 1u : 0u);
  }
  // value = n * 2^qe; encode
  uint32_t code;
  if (qe == -9) {
    // subnormal grid (or rounded up to the first normal 8 * 2^-9 = 2^-6)
    code = n;                  // n in [0, 8]; n = 8 encodes 0x08 = 2^-6
  } else {
    // n in [8, 16]; n = 16 moves to the next binade
    int Eo = qe + 3;
    if (n == 16) { n = 8; Eo += 1; }
    if (Eo > 8 || (Eo == 8 && n > 14)) {
      code = 0x7Eu;            // saturate to 448
    } else {
      code = ((uint32_t)(Eo + 7) << 3) | (n - 8);
    }
  }
  return sign | code;
}

// ---- small vector helpers ---------------------------------------------------
__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void stg16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace moe
