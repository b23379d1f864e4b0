// Quantization, dequantization and MXFP4 quantization kernels.
//
// Group-wise quantization follows the affine equations of 《量化与加速》
// ("INT8 量化原理": x_q = clip(round(x/s) + z), x_hat = s (x_q - z)) with the
// symmetric and asymmetric scale rules of 《推理优化与量化算子深度技术调研》
// section 1.2 (max|x|/q_max; (max-min)/(2^b-1) with z = round(-min/s)), the
// zero-block rule of the practice exercise in 《第 6 课：量化源码走读》 (scale 1)
// and its packing of eight INT4 codes per int32 (section 2).  Per-row FP8
// (scale max|x|/448, E4M3 range from the format table of 《量化与加速》) is the
// dynamic per-token activation quantization of that lesson's section 2.
// MXFP4 follows 《大模型量化推理引擎全景大复盘》 section 2 eq. 3 and section 3
// (32 elements share 2^ceil(log2(max/6))).
//
// Work unit: a "vec" of 8 consecutive elements along K (one int32 of INT4
// codes, 8 bytes of INT8/FP8 codes, 4 bytes of MXFP4 codes).  A group is
// T = group/8 consecutive vecs; groups tile the row-major [rows][K] array in
// order, so the group of vec v is v / T.
//  - T a power of two <= 64: one lane per vec, the group's T lanes reduce
//    with xor-shuffles (no LDS, one pass over HBM).
//  - groups of 64, 128, 256, 512 or 1024 vecs (per-row scales of rows up to
//    8192 elements): one wave per group, kept in registers, one pass.
//  - otherwise (other large groups): one 256-thread workgroup per group, a
//    block reduction, then a second pass that re-reads the group from cache
//    and writes the codes.
// Every kernel is HBM bound (4 B read + <= 1 B written per fp32 weight).

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

enum QKind { K_INT4_SYM = 0, K_INT4_ASYM = 1, K_INT8_SYM = 2, K_INT8_ASYM = 3, K_FP8 = 4,
             K_MX = 5 /* MXFP4 output of the fused normalization only */ };

constexpr int kThreads = 256;

template <bool BF16>
__device__ __forceinline__ void load_vec(const void* src, int64_t vec, float (&v)[8]) {
  if constexpr (BF16) {
    const u32x4 w = reinterpret_cast<const u32x4*>(src)[vec];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
      v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(src) + 2 * vec;
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// SmoothQuant folding (《第 1 章：推理加速全景》 section 4.3; 《推理优化与量化算子深度
// 技术调研》 section 1.5): column j of the operand is multiplied (weights,
// W diag(s)) or divided (activations, X diag(s)^-1) by s_j before the group
// statistics, one fp32 rounding per element.  A null factor pointer leaves
// the operand as it is.
struct Smooth {
  const float* s;    // factors [K], 16-byte aligned, or null
  int64_t kvecs;     // vecs per row (K / 8)
  int div;           // 1: x / s_j, 0: x * s_j
};

// Fold the factors of column vec c (elements 8c .. 8c + 7) into v.
__device__ __forceinline__ void apply_smooth(float (&v)[8], const Smooth& sm, uint32_t c) {
  const f32x4* p = reinterpret_cast<const f32x4*>(sm.s) + 2 * (size_t)c;
  const f32x4 a = p[0], b = p[1];
  const float f[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  if (sm.div) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] / f[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = v[i] * f[i];
  }
}

struct Stats {
  float amax, lo, hi;
};

// Only the statistics a format uses are formed and reduced: the range (lo,
// hi) for the asymmetric kinds, the absolute maximum for the others; the
// unused ones keep their identity values.
template <int K>
constexpr bool kRange = K == K_INT4_ASYM || K == K_INT8_ASYM;

template <int K>
__device__ __forceinline__ Stats stats_of(const float (&v)[8]) {
  Stats s{0.f, __builtin_inff(), -__builtin_inff()};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (kRange<K>) {
      s.lo = __builtin_fminf(s.lo, v[i]);
      s.hi = __builtin_fmaxf(s.hi, v[i]);
    } else {
      s.amax = __builtin_fmaxf(s.amax, __builtin_fabsf(v[i]));
    }
  }
  return s;
}

template <int K>
__device__ __forceinline__ void merge(Stats& a, const Stats& b) {
  if constexpr (kRange<K>) {
    a.lo = __builtin_fminf(a.lo, b.lo);
    a.hi = __builtin_fmaxf(a.hi, b.hi);
  } else {
    a.amax = __builtin_fmaxf(a.amax, b.amax);
  }
}

// merge with the statistics of lane (lane ^ o)
template <int K>
__device__ __forceinline__ void merge_xor(Stats& a, int o) {
  if constexpr (kRange<K>) {
    a.lo = __builtin_fminf(a.lo, shfl_xor(a.lo, o));
    a.hi = __builtin_fmaxf(a.hi, shfl_xor(a.hi, o));
  } else {
    a.amax = __builtin_fmaxf(a.amax, shfl_xor(a.amax, o));
  }
}

struct Params {
  float s;          // stored scale, as fp32
  float z;          // stored zero point, as fp32 (0 for symmetric kinds)
  uint32_t s_bits;  // fp16 bits (INT4) -- unused for fp32 storage
  uint32_t z_bits;
  double r;         // 1 / s, correctly rounded fp64
};

// fl32(x / s) for the group's stored scale s, without the fp32 division
// sequence per element: r = 1/s in fp64 (one correctly rounded fp64
// division per group), then x * r in fp64, rounded once to fp32.  The
// quotient of two 24-bit significands lies at least 2^-49 (relative) away
// from every fp32 rounding midpoint, and the fp64 product is within 2^-52 of
// the quotient, so for a normal fp32 quotient the result is the correctly
// rounded x / s.  A quotient in the fp32 subnormal range may differ in its
// last bit, which no code decision sees (such values quantize to zero in
// every format, sign kept).
__device__ __forceinline__ float quot(float x, const Params& p) {
  return (float)((double)x * p.r);
}

// Scale (and zero point) of one group, rounded to the storage dtype first;
// a stored scale of 0 becomes 1.
template <int K>
__device__ __forceinline__ Params make_params(const Stats& st) {
  Params p{1.f, 0.f, 0x3C00u, 0u, 1.0};
  if constexpr (K == K_INT4_SYM) {
    uint16_t b;
    float s = f32_to_f16_sat(st.amax / 7.0f, &b);
    if (s == 0.f) { s = 1.f; b = 0x3C00; }
    p.s = s; p.s_bits = b;
  } else if constexpr (K == K_INT4_ASYM) {
    uint16_t b, zb;
    float s = f32_to_f16_sat((st.hi - st.lo) / 15.0f, &b);
    if (s == 0.f) { s = 1.f; b = 0x3C00; }
    float z = f32_to_f16_sat(__builtin_rintf(-st.lo / s), &zb);
    p.s = s; p.s_bits = b; p.z = z; p.z_bits = zb;
  } else if constexpr (K == K_INT8_SYM) {
    float s = st.amax / 127.0f;
    p.s = (s == 0.f) ? 1.f : s;
  } else if constexpr (K == K_INT8_ASYM) {
    float s = (st.hi - st.lo) / 255.0f;
    s = (s == 0.f) ? 1.f : s;
    p.s = s;
    p.z = __builtin_rintf(-st.lo / s);
  } else {  // K_FP8
    float s = st.amax / 448.0f;
    p.s = (s == 0.f) ? 1.f : s;
  }
  p.r = 1.0 / (double)p.s;
  return p;
}

template <int K>
__device__ __forceinline__ void store_params(const Params& p, void* scales, void* zeros,
                                             int64_t g) {
  if constexpr (K == K_INT4_SYM || K == K_INT4_ASYM) {
    reinterpret_cast<uint16_t*>(scales)[g] = (uint16_t)p.s_bits;
    if constexpr (K == K_INT4_ASYM) reinterpret_cast<uint16_t*>(zeros)[g] = (uint16_t)p.z_bits;
  } else {
    reinterpret_cast<float*>(scales)[g] = p.s;
    if constexpr (K == K_INT8_ASYM) reinterpret_cast<float*>(zeros)[g] = p.z;
  }
}

// Quantize 8 values with the group parameters and store their codes.
template <int K>
__device__ __forceinline__ void quantize_store(const float (&v)[8], const Params& p,
                                               void* codes, int64_t vec) {
  if constexpr (K == K_INT4_SYM || K == K_INT4_ASYM) {
    constexpr float lo = (K == K_INT4_SYM) ? -8.f : 0.f;
    constexpr float hi = (K == K_INT4_SYM) ? 7.f : 15.f;
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float q = __builtin_rintf(quot(v[i], p)) + p.z;    // round, then add z
      q = __builtin_fminf(__builtin_fmaxf(q, lo), hi);    // then clip
      word |= ((uint32_t)(int)q & 0xFu) << (4 * i);
    }
    reinterpret_cast<uint32_t*>(codes)[vec] = word;
  } else if constexpr (K == K_FP8) {
    // the gfx950 conversion rounds to nearest even into OCP E4M3; |x / s| <=
    // 448 (1 + 2^-23) by construction of s, which rounds to 448, so the
    // saturating and the plain conversion agree
    uint2 out;
    out.x = __builtin_amdgcn_cvt_pk_fp8_f32(quot(v[0], p), quot(v[1], p), 0u, false);
    out.x = __builtin_amdgcn_cvt_pk_fp8_f32(quot(v[2], p), quot(v[3], p), out.x, true);
    out.y = __builtin_amdgcn_cvt_pk_fp8_f32(quot(v[4], p), quot(v[5], p), 0u, false);
    out.y = __builtin_amdgcn_cvt_pk_fp8_f32(quot(v[6], p), quot(v[7], p), out.y, true);
    reinterpret_cast<uint2*>(codes)[vec] = out;
  } else {
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      {
        constexpr float lo = (K == K_INT8_SYM) ? -127.f : 0.f;
        constexpr float hi = (K == K_INT8_SYM) ? 127.f : 255.f;
        float q = __builtin_rintf(quot(v[i], p)) + p.z;
        q = __builtin_fminf(__builtin_fmaxf(q, lo), hi);
        b[i] = (uint32_t)(int)q & 0xFFu;
      }
    }
    uint2 out;
    out.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
    out.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
    reinterpret_cast<uint2*>(codes)[vec] = out;
  }
}

// A wave covers 64 * kVpl consecutive vecs: lane l takes vecs l + 64 i, so
// every load is a coalesced 1 KiB (bf16) piece; all loads go out before the
// first reduction.
constexpr int kVpl = 4;

template <int K, bool BF16>
__global__ __launch_bounds__(kThreads) void quant_wave_kernel(const void* __restrict__ src,
                                                              int64_t total_vecs, int t_log2,
                                                              void* __restrict__ codes,
                                                              void* __restrict__ scales,
                                                              void* __restrict__ zeros,
                                                              Smooth sm) {
  const int lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 64 * kVpl;
  float v[kVpl][8];
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const int64_t vec = base + 64 * i + lane;
    if (vec < total_vecs) {
      load_vec<BF16>(src, vec, v[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    }
  }
  if (sm.s) {
    // column of the wave's first vec once, then 32-bit arithmetic
    const uint32_t c0 = (uint32_t)(base % sm.kvecs), kv = (uint32_t)sm.kvecs;
#pragma unroll
    for (int i = 0; i < kVpl; ++i) {
      uint32_t c = c0 + 64 * i + lane;
      if (c >= kv) c %= kv;
      if (base + 64 * i + lane < total_vecs) apply_smooth(v[i], sm, c);
    }
  }
  const int seg = 1 << t_log2;
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const int64_t vec = base + 64 * i + lane;
    Stats st = stats_of<K>(v[i]);
    // segments never straddle valid and invalid lanes (total_vecs % seg == 0)
    for (int o = 1; o < seg; o <<= 1) {
      merge_xor<K>(st, o);
    }
    if (vec < total_vecs) {
      const Params p = make_params<K>(st);
      quantize_store<K>(v[i], p, codes, vec);
      if ((vec & (seg - 1)) == 0) store_params<K>(p, scales, zeros, vec >> t_log2);
    }
  }
}

// One wave per group of 64 * VPL vecs (per-row scales of rows up to 8192
// elements): the group stays in registers, the statistics are reduced across
// the wave, the codes are written from the registers (one pass over HBM).
template <int K, bool BF16, int VPL>
__global__ __launch_bounds__(kThreads) void quant_rowwave_kernel(const void* __restrict__ src,
                                                                 int64_t groups,
                                                                 void* __restrict__ codes,
                                                                 void* __restrict__ scales,
                                                                 void* __restrict__ zeros,
                                                                 Smooth sm) {
  const int lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (g >= groups) return;
  const int64_t v0 = g * 64 * VPL;
  float v[VPL][8];
#pragma unroll
  for (int i = 0; i < VPL; ++i) load_vec<BF16>(src, v0 + 64 * i + lane, v[i]);
  if (sm.s) {
    // a group never crosses a row
    const uint32_t c0 = (uint32_t)(v0 % sm.kvecs);
#pragma unroll
    for (int i = 0; i < VPL; ++i) apply_smooth(v[i], sm, c0 + 64 * i + lane);
  }
  Stats st{0.f, __builtin_inff(), -__builtin_inff()};
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const Stats s = stats_of<K>(v[i]);
    merge<K>(st, s);
  }
  for (int o = 1; o < 64; o <<= 1) {
    merge_xor<K>(st, o);
  }
  const Params p = make_params<K>(st);
#pragma unroll
  for (int i = 0; i < VPL; ++i) quantize_store<K>(v[i], p, codes, v0 + 64 * i + lane);
  if (lane == 0) store_params<K>(p, scales, zeros, g);
}

template <int K, bool BF16>
__global__ __launch_bounds__(kThreads) void quant_block_kernel(const void* __restrict__ src,
                                                               int64_t t_vecs,
                                                               void* __restrict__ codes,
                                                               void* __restrict__ scales,
                                                               void* __restrict__ zeros,
                                                               Smooth sm) {
  __shared__ float red[3][kThreads / 64];
  const int64_t g = blockIdx.x;
  const int64_t v0 = g * t_vecs;
  const uint32_t c0 = sm.s ? (uint32_t)(v0 % sm.kvecs) : 0u;   // a group never crosses a row
  Stats st{0.f, __builtin_inff(), -__builtin_inff()};
  for (int64_t i = threadIdx.x; i < t_vecs; i += kThreads) {
    float v[8];
    load_vec<BF16>(src, v0 + i, v);
    if (sm.s) apply_smooth(v, sm, c0 + (uint32_t)i);
    const Stats s = stats_of<K>(v);
    merge<K>(st, s);
  }
  for (int o = 1; o < 64; o <<= 1) {
    merge_xor<K>(st, o);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = st.amax;
    red[1][w] = st.lo;
    red[2][w] = st.hi;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    merge<K>(st, Stats{red[0][i], red[1][i], red[2][i]});
  }
  const Params p = make_params<K>(st);
  for (int64_t i = threadIdx.x; i < t_vecs; i += kThreads) {
    float v[8];
    load_vec<BF16>(src, v0 + i, v);
    if (sm.s) apply_smooth(v, sm, c0 + (uint32_t)i);
    quantize_store<K>(v, p, codes, v0 + i);
  }
  if (threadIdx.x == 0) store_params<K>(p, scales, zeros, g);
}

// --------------------------------------------------------------- dequant

template <int FMT, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const void* __restrict__ codes,
                                                           const void* __restrict__ scales,
                                                           const void* __restrict__ zeros,
                                                           int64_t total_vecs, int64_t t_vecs,
                                                           void* __restrict__ dst) {
  const int64_t vec = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (vec >= total_vecs) return;
  const int64_t g = vec / t_vecs;
  float out[8];
  if constexpr (FMT == QG_INT4_SYM || FMT == QG_INT4_ASYM) {
    const float s = f16_bits_to_f32(reinterpret_cast<const uint16_t*>(scales)[g]);
    const float z =
        (FMT == QG_INT4_ASYM) ? f16_bits_to_f32(reinterpret_cast<const uint16_t*>(zeros)[g]) : 0.f;
    const uint32_t word = reinterpret_cast<const uint32_t*>(codes)[vec];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int q = (int)((word >> (4 * i)) & 0xFu);
      if (FMT == QG_INT4_SYM) q = (q ^ 8) - 8;        // two's-complement nibble
      out[i] = s * ((float)q - z);
    }
  } else if constexpr (FMT == QG_MXFP4) {
    const int e = (int)reinterpret_cast<const uint8_t*>(scales)[g] - 127;
    const uint32_t word = reinterpret_cast<const uint32_t*>(codes)[vec];
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = __builtin_ldexpf(e2m1_decode(word >> (4 * i)), e);
  } else {
    const float s = reinterpret_cast<const float*>(scales)[g];
    const float z = (FMT == QG_INT8_ASYM) ? reinterpret_cast<const float*>(zeros)[g] : 0.f;
    const uint2 w = reinterpret_cast<const uint2*>(codes)[vec];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = ((i < 4 ? w.x : w.y) >> (8 * (i & 3))) & 0xFFu;
      if constexpr (FMT == QG_FP8_E4M3) {
        out[i] = s * e4m3_decode(b);
      } else if constexpr (FMT == QG_INT8_SYM) {
        out[i] = s * ((float)(int)(int8_t)b - z);
      } else {
        out[i] = s * ((float)(int)b - z);
      }
    }
  }
  if constexpr (OUT_BF16) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(out[2 * i], out[2 * i + 1]);
    reinterpret_cast<u32x4*>(dst)[vec] = o;
  } else {
    f32x4* p = reinterpret_cast<f32x4*>(dst) + 2 * vec;
    p[0] = f32x4{out[0], out[1], out[2], out[3]};
    p[1] = f32x4{out[4], out[5], out[6], out[7]};
  }
}

// ---------------------------------------------------------------- MXFP4

// One lane per 8 elements, 4 lanes per 32-element block; a wave covers 64 *
// kVpl consecutive vecs (lane l: vecs l + 64 i), all loads issued first.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void mx_quant_kernel(const void* __restrict__ src,
                                                            int64_t total_vecs,
                                                            void* __restrict__ codes,
                                                            void* __restrict__ e8m0) {
  const int lane = threadIdx.x & 63;
  const int64_t base = ((int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * 64 * kVpl;
  float v[kVpl][8];
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const int64_t vec = base + 64 * i + lane;
    if (vec < total_vecs) {
      load_vec<BF16>(src, vec, v[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < kVpl; ++i) {
    const int64_t vec = base + 64 * i + lane;
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[i][e]));
    m = __builtin_fmaxf(m, shfl_xor(m, 1));
    m = __builtin_fmaxf(m, shfl_xor(m, 2));
    if (vec < total_vecs) {
      const int e = mx_shared_exponent(m);
      // x / 2^e (exact) is within [-6, 6]; the gfx950 conversion (scale 1)
      // rounds to the nearest E2M1 value, ties to the even code, element 2 j
      // into the low nibble of byte j
      float t[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = __builtin_ldexpf(v[i][k], -e);
      uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, t[0], t[1], 1.0f, 0);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, t[2], t[3], 1.0f, 1);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, t[4], t[5], 1.0f, 2);
      word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, t[6], t[7], 1.0f, 3);
      reinterpret_cast<uint32_t*>(codes)[vec] = word;
      if ((vec & 3) == 0) reinterpret_cast<uint8_t*>(e8m0)[vec >> 2] = (uint8_t)(e + 127);
    }
  }
}

inline unsigned blocks_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }
// workgroups for kernels whose waves each cover 64 * kVpl vecs
inline unsigned blocks_for_vpl(int64_t n) {
  return (unsigned)((n + kThreads * kVpl - 1) / (kThreads * kVpl));
}

template <int K, bool BF16>
void launch_quant_t(const void* src, int64_t rows, int64_t Kdim, int64_t group, void* codes,
                    void* scales, void* zeros, const Smooth& sm, hipStream_t stream) {
  const int64_t t_vecs = group / 8;
  const int64_t total = rows * Kdim / 8;
  if (t_vecs <= 64 && (t_vecs & (t_vecs - 1)) == 0) {
    int t_log2 = 0;
    while ((1LL << t_log2) < t_vecs) ++t_log2;
    hipLaunchKernelGGL((quant_wave_kernel<K, BF16>), dim3(blocks_for_vpl(total)), dim3(kThreads),
                       0, stream, src, total, t_log2, codes, scales, zeros, sm);
  } else if (t_vecs % 64 == 0 && t_vecs <= 64 * 16) {
    // groups of 512, 1024, 2048, 4096 or 8192 elements: one wave per group
    // (other multiples of 512 take the workgroup kernel below)
    const int64_t groups = rows * (Kdim / group);
    const unsigned blocks = (unsigned)((groups + kThreads / 64 - 1) / (kThreads / 64));
    switch (t_vecs / 64) {
      case 1:
        hipLaunchKernelGGL((quant_rowwave_kernel<K, BF16, 1>), dim3(blocks), dim3(kThreads), 0,
                           stream, src, groups, codes, scales, zeros, sm);
        break;
      case 2:
        hipLaunchKernelGGL((quant_rowwave_kernel<K, BF16, 2>), dim3(blocks), dim3(kThreads), 0,
                           stream, src, groups, codes, scales, zeros, sm);
        break;
      case 4:
        hipLaunchKernelGGL((quant_rowwave_kernel<K, BF16, 4>), dim3(blocks), dim3(kThreads), 0,
                           stream, src, groups, codes, scales, zeros, sm);
        break;
      case 8:
        hipLaunchKernelGGL((quant_rowwave_kernel<K, BF16, 8>), dim3(blocks), dim3(kThreads), 0,
                           stream, src, groups, codes, scales, zeros, sm);
        break;
      case 16:
        hipLaunchKernelGGL((quant_rowwave_kernel<K, BF16, 16>), dim3(blocks), dim3(kThreads), 0,
                           stream, src, groups, codes, scales, zeros, sm);
        break;
      default:
        hipLaunchKernelGGL((quant_block_kernel<K, BF16>), dim3((unsigned)groups), dim3(kThreads),
                           0, stream, src, t_vecs, codes, scales, zeros, sm);
        break;
    }
  } else {
    const int64_t groups = rows * (Kdim / group);
    hipLaunchKernelGGL((quant_block_kernel<K, BF16>), dim3((unsigned)groups), dim3(kThreads), 0,
                       stream, src, t_vecs, codes, scales, zeros, sm);
  }
}

template <bool BF16>
void launch_quant_fmt(qg_format fmt, const void* src, int64_t rows, int64_t Kdim, int64_t group,
                      void* codes, void* scales, void* zeros, const Smooth& sm,
                      hipStream_t stream) {
  switch (fmt) {
    case QG_INT4_SYM:
      return launch_quant_t<K_INT4_SYM, BF16>(src, rows, Kdim, group, codes, scales, zeros, sm, stream);
    case QG_INT4_ASYM:
      return launch_quant_t<K_INT4_ASYM, BF16>(src, rows, Kdim, group, codes, scales, zeros, sm, stream);
    case QG_INT8_SYM:
      return launch_quant_t<K_INT8_SYM, BF16>(src, rows, Kdim, group, codes, scales, zeros, sm, stream);
    case QG_INT8_ASYM:
      return launch_quant_t<K_INT8_ASYM, BF16>(src, rows, Kdim, group, codes, scales, zeros, sm, stream);
    default:
      return launch_quant_t<K_FP8, BF16>(src, rows, Kdim, group, codes, scales, zeros, sm, stream);
  }
}

template <int FMT>
void launch_dequant_t(const void* codes, const void* scales, const void* zeros, int64_t total,
                      int64_t t_vecs, void* dst, qg_dtype dt, hipStream_t stream) {
  if (dt == QG_BF16)
    hipLaunchKernelGGL((dequant_kernel<FMT, true>), dim3(blocks_for(total)), dim3(kThreads), 0,
                       stream, codes, scales, zeros, total, t_vecs, dst);
  else
    hipLaunchKernelGGL((dequant_kernel<FMT, false>), dim3(blocks_for(total)), dim3(kThreads), 0,
                       stream, codes, scales, zeros, total, t_vecs, dst);
}

// --------------------------------------------------------------- fused norm + quant

// LayerNorm or RMSNorm of one row followed by its per-row dynamic
// quantization, written once (《推理优化与量化算子深度技术调研》 section 4.4:
// statistics, normalization and the quantization scale of a row in one
// kernel, codes and scale written once).  One workgroup per row; thread t
// holds vecs t + kThreads i (i < VPT) of the row in registers.  The row
// statistics are summed in fp64 (sum of x, then of (x - mean)^2; or sum of
// x^2), mean and r = 1 / sqrt(var + eps) are rounded once to fp32, and the
// normalized value is formed in fp32 with one rounding per operation and no
// fused multiply-add: t = x - mean, u = t * r, y = u * gamma (+ beta).  The
// codes are then those of the per-row quantizer above, or (K_MX) those of
// the MXFP4 quantizer: a 32-element block is 4 consecutive vecs, held by 4
// consecutive threads, so its maximum is two xor-shuffles away and the row
// needs no further reduction.
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();   // the previous use of red is over
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) t += red[i];
  return t;
}

template <int K, bool BF16, bool RMS, int VPT>
__global__ __launch_bounds__(kThreads) void norm_quant_kernel(const void* __restrict__ src,
                                                              int64_t kvecs,
                                                              const float* __restrict__ gamma,
                                                              const float* __restrict__ beta,
                                                              float eps, void* __restrict__ codes,
                                                              void* __restrict__ scales,
                                                              void* __restrict__ zeros) {
  __shared__ double redd[kThreads / 64];
  __shared__ float red[3][kThreads / 64];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t v0 = row * kvecs;
  float v[VPT][8];
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t vec = tid + (int64_t)kThreads * i;
    if (vec < kvecs) {
      load_vec<BF16>(src, v0 + vec, v[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = 0.f;   // contributes nothing to the sums
    }
  }
  const double kd = (double)(kvecs * 8);
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < VPT; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double d = (double)v[i][e];
      acc += RMS ? d * d : d;
    }
  const double s1 = block_sum_f64(acc, redd);
  const double mean64 = RMS ? 0.0 : s1 / kd;
  double var64 = s1 / kd;
  if constexpr (!RMS) {
    double acc2 = 0.0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      if (tid + (int64_t)kThreads * i >= kvecs) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        // converted again here: reusing the first pass's fp64 values would
        // keep all of them live (two registers per element) across the
        // reduction, halving the waves that fit on a SIMD
        float f = v[i][e];
        asm volatile("" : "+v"(f));
        const double d = (double)f - mean64;
        acc2 += d * d;
      }
    }
    var64 = block_sum_f64(acc2, redd) / kd;
  }
  const float mean32 = (float)mean64;
  const float r32 = (float)(1.0 / __builtin_sqrt(var64 + (double)eps));

  Stats st{0.f, __builtin_inff(), -__builtin_inff()};
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t vec = tid + (int64_t)kThreads * i;
    if (vec >= kvecs) continue;
    const f32x4* gp = reinterpret_cast<const f32x4*>(gamma) + 2 * vec;
    const f32x4 g0 = gp[0], g1 = gp[1];
    f32x4 b0 = {0.f, 0.f, 0.f, 0.f}, b1 = b0;
    if constexpr (!RMS) {
      const f32x4* bp = reinterpret_cast<const f32x4*>(beta) + 2 * vec;
      b0 = bp[0];
      b1 = bp[1];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float g = e < 4 ? g0[e] : g1[e - 4];
      const float t = RMS ? v[i][e] : v[i][e] - mean32;
      float y = (t * r32) * g;
      // the product is rounded before beta is added: the empty asm keeps the
      // compiler from fusing the two into one multiply-add (which
      // -ffp-contract=fast would do regardless of a contract pragma)
      asm volatile("" : "+v"(y));
      if constexpr (!RMS) y = y + (e < 4 ? b0[e] : b1[e - 4]);
      v[i][e] = y;
    }
    if constexpr (K != K_MX) {
      const Stats s = stats_of<K>(v[i]);
      merge<K>(st, s);
    }
  }
  if constexpr (K == K_MX) {
    // K % 32 == 0, so the 4 threads of a block are all inside or all past
    // the row; every thread takes part in the shuffles
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int64_t vec = tid + (int64_t)kThreads * i;
      float m = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[i][e]));
      m = __builtin_fmaxf(m, shfl_xor(m, 1));
      m = __builtin_fmaxf(m, shfl_xor(m, 2));
      if (vec < kvecs) {
        const int ex = mx_shared_exponent(m);
        // y / 2^e (exact) lies in [-6, 6]; the gfx950 conversion (scale 1)
        // rounds to the nearest E2M1 value, ties to the even code, element
        // 2 j into the low nibble of byte j
        float t[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) t[k] = __builtin_ldexpf(v[i][k], -ex);
        uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, t[0], t[1], 1.0f, 0);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, t[2], t[3], 1.0f, 1);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, t[4], t[5], 1.0f, 2);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, t[6], t[7], 1.0f, 3);
        reinterpret_cast<uint32_t*>(codes)[v0 + vec] = word;
        if ((vec & 3) == 0) reinterpret_cast<uint8_t*>(scales)[(v0 + vec) >> 2] = (uint8_t)(ex + 127);
      }
    }
    return;
  } else {
  for (int o = 1; o < 64; o <<= 1) {
    merge_xor<K>(st, o);
  }
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    red[0][w] = st.amax;
    red[1][w] = st.lo;
    red[2][w] = st.hi;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    merge<K>(st, Stats{red[0][i], red[1][i], red[2][i]});
  }
  const Params p = make_params<K>(st);
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const int64_t vec = tid + (int64_t)kThreads * i;
    if (vec < kvecs) quantize_store<K>(v[i], p, codes, v0 + vec);
  }
  if (tid == 0) store_params<K>(p, scales, zeros, row);
  }
}

template <int K, bool BF16, bool RMS>
void launch_norm_quant_t(const void* src, int64_t rows, int64_t kvecs, const float* gamma,
                         const float* beta, float eps, void* codes, void* scales, void* zeros,
                         hipStream_t stream) {
  const dim3 grid((unsigned)rows), block(kThreads);
  if (kvecs <= kThreads)
    hipLaunchKernelGGL((norm_quant_kernel<K, BF16, RMS, 1>), grid, block, 0, stream, src, kvecs,
                       gamma, beta, eps, codes, scales, zeros);
  else if (kvecs <= 2 * kThreads)
    hipLaunchKernelGGL((norm_quant_kernel<K, BF16, RMS, 2>), grid, block, 0, stream, src, kvecs,
                       gamma, beta, eps, codes, scales, zeros);
  else if (kvecs <= 4 * kThreads)
    hipLaunchKernelGGL((norm_quant_kernel<K, BF16, RMS, 4>), grid, block, 0, stream, src, kvecs,
                       gamma, beta, eps, codes, scales, zeros);
  else
    hipLaunchKernelGGL((norm_quant_kernel<K, BF16, RMS, 8>), grid, block, 0, stream, src, kvecs,
                       gamma, beta, eps, codes, scales, zeros);
}

template <bool BF16, bool RMS>
void launch_norm_quant_fmt(qg_format fmt, const void* src, int64_t rows, int64_t kvecs,
                           const float* gamma, const float* beta, float eps, void* codes,
                           void* scales, void* zeros, hipStream_t stream) {
  if (fmt == QG_INT8_SYM)
    launch_norm_quant_t<K_INT8_SYM, BF16, RMS>(src, rows, kvecs, gamma, beta, eps, codes, scales,
                                              zeros, stream);
  else if (fmt == QG_INT8_ASYM)
    launch_norm_quant_t<K_INT8_ASYM, BF16, RMS>(src, rows, kvecs, gamma, beta, eps, codes,
                                               scales, zeros, stream);
  else if (fmt == QG_MXFP4)
    launch_norm_quant_t<K_MX, BF16, RMS>(src, rows, kvecs, gamma, beta, eps, codes, scales,
                                        zeros, stream);
  else
    launch_norm_quant_t<K_FP8, BF16, RMS>(src, rows, kvecs, gamma, beta, eps, codes, scales,
                                         zeros, stream);
}

}  // namespace

hipError_t launch_norm_quant(bool rms, qg_format fmt, const void* src, qg_dtype src_dtype,
                             const void* gamma, const void* beta, float eps, int64_t rows,
                             int64_t K, void* codes, void* scales, void* zeros,
                             hipStream_t stream) {
  const int64_t kvecs = K / 8;
  const float* g = (const float*)gamma;
  const float* b = (const float*)beta;
  if (src_dtype == QG_BF16) {
    if (rms)
      launch_norm_quant_fmt<true, true>(fmt, src, rows, kvecs, g, b, eps, codes, scales, zeros, stream);
    else
      launch_norm_quant_fmt<true, false>(fmt, src, rows, kvecs, g, b, eps, codes, scales, zeros, stream);
  } else {
    if (rms)
      launch_norm_quant_fmt<false, true>(fmt, src, rows, kvecs, g, b, eps, codes, scales, zeros, stream);
    else
      launch_norm_quant_fmt<false, false>(fmt, src, rows, kvecs, g, b, eps, codes, scales, zeros, stream);
  }
  return hipGetLastError();
}

namespace {
}  // namespace

hipError_t launch_quantize(qg_format fmt, const void* src, qg_dtype src_dtype, int64_t rows,
                           int64_t K, int64_t group, void* codes, void* scales, void* zeros,
                           const float* smooth, bool divide, hipStream_t stream) {
  const Smooth sm{smooth, K / 8, divide ? 1 : 0};
  if (src_dtype == QG_BF16)
    launch_quant_fmt<true>(fmt, src, rows, K, group, codes, scales, zeros, sm, stream);
  else
    launch_quant_fmt<false>(fmt, src, rows, K, group, codes, scales, zeros, sm, stream);
  return hipGetLastError();
}

hipError_t launch_dequant(qg_format fmt, const void* codes, const void* scales,
                          const void* zeros, int64_t rows, int64_t K, int64_t group, void* dst,
                          qg_dtype dst_dtype, hipStream_t stream) {
  const int64_t total = rows * K / 8;
  const int64_t t_vecs = group / 8;
  switch (fmt) {
    case QG_INT4_SYM:
      launch_dequant_t<QG_INT4_SYM>(codes, scales, zeros, total, t_vecs, dst, dst_dtype, stream);
      break;
    case QG_INT4_ASYM:
      launch_dequant_t<QG_INT4_ASYM>(codes, scales, zeros, total, t_vecs, dst, dst_dtype, stream);
      break;
    case QG_INT8_SYM:
      launch_dequant_t<QG_INT8_SYM>(codes, scales, zeros, total, t_vecs, dst, dst_dtype, stream);
      break;
    case QG_INT8_ASYM:
      launch_dequant_t<QG_INT8_ASYM>(codes, scales, zeros, total, t_vecs, dst, dst_dtype, stream);
      break;
    case QG_FP8_E4M3:
      launch_dequant_t<QG_FP8_E4M3>(codes, scales, zeros, total, t_vecs, dst, dst_dtype, stream);
      break;
    default:
      launch_dequant_t<QG_MXFP4>(codes, scales, zeros, total, t_vecs, dst, dst_dtype, stream);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_mx_quant(const void* src, qg_dtype src_dtype, int64_t rows, int64_t K,
                           void* codes, void* e8m0, hipStream_t stream) {
  const int64_t total = rows * K / 8;
  if (src_dtype == QG_BF16)
    hipLaunchKernelGGL((mx_quant_kernel<true>), dim3(blocks_for_vpl(total)), dim3(kThreads), 0,
                       stream, src, total, codes, e8m0);
  else
    hipLaunchKernelGGL((mx_quant_kernel<false>), dim3(blocks_for_vpl(total)), dim3(kThreads), 0,
                       stream, src, total, codes, e8m0);
  return hipGetLastError();
}

}  // namespace qg
