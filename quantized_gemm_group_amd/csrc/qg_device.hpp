// Device-side numeric helpers shared by the quantization and GEMM kernels.
//
// Everything here is exact by construction: round-to-nearest-even
// conversions written with integer arithmetic on the IEEE encodings, the
// saturating FP8 E4M3 encoder and the E2M1 encoder built from the format
// definitions (《量化与加速》 float formula and format table; E2M1 maximum 6 from
// the MX scale rule of 《大模型量化推理引擎全景大复盘》 section 3), and the MX
// shared exponent decided with integer logic instead of a floating-point log.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// ---------------------------------------------------------------- bf16 / fp16

// fp32 -> bf16 bits, round to nearest even (IEEE: overflow goes to inf).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// fp32 -> fp16 round to nearest even, results that would overflow to
// infinity clamped to +-65504 (scale storage).  Returns the stored value
// widened back to fp32.
__device__ __forceinline__ float f32_to_f16_sat(float f, uint16_t* bits) {
  _Float16 h = (_Float16)f;                       // v_cvt_f16_f32, RNE
  float back = (float)h;
  if (__builtin_isinf(back) && !__builtin_isinf(f)) {
    h = (_Float16)(f > 0.f ? 65504.f : -65504.f);
    back = (float)h;
  }
  *bits = __builtin_bit_cast(uint16_t, h);
  return back;
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// ------------------------------------------------------------------ FP8 E4M3

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e ? __builtin_ldexpf((float)(8u + m), (int)e - 10)
                : __builtin_ldexpf((float)m, -9);
  return (c & 0x80u) ? -mag : mag;
}

// ------------------------------------------------------------------ FP4 E2M1

__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  const uint32_t m = c & 7u;
  // codes 0,1 are subnormal (0, 0.5); codes 2..7 are 2^(e-1) * (1 + f/2) with
  // e = m >> 1, f = m & 1, i.e. (2 + f) * 2^(e-2): 1 1.5 2 3 4 6
  float mag = (m < 2u) ? 0.5f * (float)m
                       : __builtin_ldexpf((float)(2u + (m & 1u)), (int)(m >> 1) - 2);
  return (c & 8u) ? -mag : mag;
}

// MX shared exponent: smallest integer e with m <= 6 * 2^e, for m = f * 2^E
// (f in [1,2)) that is E - 2 + [f > 1.5]; clamped to [-127, 127]; 0 for m == 0.
__device__ __forceinline__ int mx_shared_exponent(float m) {
  if (m == 0.f) return 0;
  int ex;
  float fr = __builtin_frexpf(m, &ex);            // m = fr * 2^ex, fr in [0.5, 1)
  int e = (ex - 1) - 2 + (fr > 0.75f ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// ------------------------------------------------------------ debug outputs

// Built with QG_DEBUG_FP32 (the debug library libqgemm_debug.so): every
// kernel that rounds a product to bf16 also stores the fp32 value it rounds,
// at the same index of an fp32 buffer shaped like the output, when
// qg_debug_fp32_output has set one (one pointer per translation unit, set
// through the function that QG_DEBUG_TU_SETTER defines).  Without the macro
// none of this is compiled.
#ifdef QG_DEBUG_FP32
static __device__ float* g_qg_debug_out = nullptr;
#define QG_DEBUG_STORE(idx, v)              \
  do {                                      \
    float* qg_dbg_p_ = g_qg_debug_out;      \
    if (qg_dbg_p_) qg_dbg_p_[idx] = (v);    \
  } while (0)
#define QG_DEBUG_TU_SETTER(name)                                          \
  hipError_t name(float* p) {                                             \
    return hipMemcpyToSymbol(HIP_SYMBOL(g_qg_debug_out), &p, sizeof(p));   \
  }
#else
#define QG_DEBUG_STORE(idx, v) \
  do {                         \
  } while (0)
#define QG_DEBUG_TU_SETTER(name)
#endif

// ------------------------------------------------------------ wave utilities

// xor-shuffle within a wave (ds_bpermute based).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

__device__ __forceinline__ float wave_max_seg(float v, int seg) {
  for (int o = 1; o < seg; o <<= 1) v = __builtin_fmaxf(v, shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_min_seg(float v, int seg) {
  for (int o = 1; o < seg; o <<= 1) v = __builtin_fminf(v, shfl_xor(v, o));
  return v;
}

}  // namespace qg
