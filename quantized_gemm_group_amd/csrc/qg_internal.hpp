// Internal launch interface between the C ABI (qg_api.hip) and the kernel
// translation units.  Arguments reaching these functions are already
// validated; each function only enqueues kernels on `stream` and returns the
// hipGetLastError() of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qgemm.h"

namespace qg {

// smooth: per-column factors [K] folded into the operand before the group
// statistics (x * s_j, or x / s_j when divide), or null.
hipError_t launch_quantize(qg_format fmt, const void* src, qg_dtype src_dtype, int64_t rows,
                           int64_t K, int64_t group, void* codes, void* scales, void* zeros,
                           const float* smooth, bool divide, hipStream_t stream);

hipError_t launch_channel_absmax(const void* src, qg_dtype src_dtype, int64_t rows, int64_t K,
                                 bool accumulate, float* out, hipStream_t stream);

hipError_t launch_smooth_scales(const float* act_absmax, const float* w_absmax, float alpha,
                                int64_t K, float* smooth, hipStream_t stream);

hipError_t launch_channel_scales(const float* absmax, int64_t n, float qmax, float* scales,
                                 hipStream_t stream);

hipError_t launch_kv_cache_store(const void* x, qg_dtype x_dtype, int64_t tokens, int64_t heads,
                                 int64_t head_dim, const int64_t* slot_mapping, int64_t num_slots,
                                 const float* channel_scales, void* cache_codes,
                                 float* cache_scales, hipStream_t stream);

hipError_t launch_dequant(qg_format fmt, const void* codes, const void* scales,
                          const void* zeros, int64_t rows, int64_t K, int64_t group, void* dst,
                          qg_dtype dst_dtype, hipStream_t stream);

hipError_t launch_norm_quant(bool rms, qg_format fmt, const void* src, qg_dtype src_dtype,
                             const void* gamma, const void* beta, float eps, int64_t rows,
                             int64_t K, void* codes, void* scales, void* zeros,
                             hipStream_t stream);

hipError_t launch_mx_quant(const void* src, qg_dtype src_dtype, int64_t rows, int64_t K,
                           void* codes, void* e8m0, hipStream_t stream);

// tiled: wcodes in the GEMV tile layout written by launch_tile_gemv_codes.
hipError_t launch_qgemv(bool asym, bool tiled, const void* x, int64_t M, const void* wcodes,
                        const void* wscales, const void* wzeros, int64_t N, int64_t K, void* y,
                        hipStream_t stream);

// W4A16 product for group sizes other than 128 (32, 64 or a multiple of 128
// dividing K, K a multiple of 128), any M, canonical or tiled codes.
bool w4a16_group_supported(int64_t K, int64_t group);
hipError_t launch_w4a16_groups(bool asym, bool tiled, const void* x, int64_t M,
                               const void* wcodes, const void* wscales, const void* wzeros,
                               int64_t N, int64_t K, int64_t group, void* y, hipStream_t stream);

// SwiGLU decode GEMV over [W_gate; W_up] (N2 = 2I rows) into h [M][I];
// qgemv_swiglu_supported tells which (M, K) the kernels cover.
bool qgemv_swiglu_supported(int64_t M, int64_t K);
hipError_t launch_qgemv_swiglu(bool asym, bool tiled, const void* x, int64_t M,
                               const void* wcodes, const void* wscales, const void* wzeros,
                               int64_t N2, int64_t K, void* h, hipStream_t stream);

hipError_t launch_tile_gemv_codes(const void* codes, int64_t N, int64_t K, void* tiled,
                                  hipStream_t stream);

hipError_t launch_gemm_w4a16(bool asym, const void* x, int64_t M, const void* wcodes,
                             const void* wscales, const void* wzeros, int64_t N, int64_t K,
                             void* y, hipStream_t stream);

hipError_t launch_gemm_w4a16_swiglu(bool asym, const void* x, int64_t M, const void* wcodes,
                                    const void* wscales, const void* wzeros, int64_t N2,
                                    int64_t K, void* h, hipStream_t stream);

hipError_t launch_gemm_fp8(const void* a, const void* a_scales, int64_t M, const void* w,
                           const void* w_scales, int64_t N, int64_t K, void* y,
                           hipStream_t stream);

// FP8 W8A8 GEMM over [W_gate; W_up] (N2 = 2I rows) with the SwiGLU epilogue
// into h [M][I].
hipError_t launch_gemm_fp8_swiglu(const void* a, const void* a_scales, int64_t M, const void* w,
                                  const void* w_scales, int64_t N2, int64_t K, void* h,
                                  hipStream_t stream);

hipError_t launch_gemm_int8(bool a_asym, bool w_asym, const void* a, const void* a_scales,
                            const void* a_zeros, int64_t M, const void* w, const void* w_scales,
                            const void* w_zeros, int64_t N, int64_t K, void* y,
                            hipStream_t stream);

hipError_t launch_mx_gemm(const void* a_codes, const void* a_e8m0, int64_t M,
                          const void* b_codes, const void* b_e8m0, int64_t N, int64_t K, void* y,
                          hipStream_t stream);

// Roofline calibration (measurement only): a read-only stream of `bytes`
// (a multiple of 64 KiB) and an MFMA-only loop of `waves` waves (a multiple
// of 4) x `iters` iterations of 8 instructions.
hipError_t launch_calib_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                                    hipStream_t stream);

hipError_t launch_calib_mfma(int kind, int64_t waves, int64_t iters, float* sink,
                             hipStream_t stream);

#ifdef QG_DEBUG_FP32
// Debug library: point every translation unit's fp32 output recorder at p.
hipError_t debug_set_gemv(float* p);
hipError_t debug_set_f8f4(float* p);
hipError_t debug_set_int8(float* p);
hipError_t debug_set_w4a16(float* p);
#endif

}  // namespace qg
