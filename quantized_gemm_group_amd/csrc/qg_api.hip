// C ABI of the quantized linear layer library (declared in include/qgemm.h).
//
// Every entry point validates its arguments completely before the first HIP
// call, so an invalid call enqueues nothing and touches no device state.  The
// library allocates nothing and never synchronizes.

#include <cstdint>
#include <cstdio>
#include <cstring>

#include "qg_internal.hpp"

namespace {

thread_local char g_last_error[256] = "";

qg_status fail(qg_status st, const char* what) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s", what);
  return st;
}

qg_status ok() {
  g_last_error[0] = '\0';
  return QG_OK;
}

qg_status from_hip(hipError_t e) {
  if (e == hipSuccess) return ok();
  std::snprintf(g_last_error, sizeof(g_last_error), "HIP launch error: %s", hipGetErrorString(e));
  return QG_ERR_HIP;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool aligned_to(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool is_quant_fmt(qg_format f) {
  return f == QG_INT4_SYM || f == QG_INT4_ASYM || f == QG_INT8_SYM || f == QG_INT8_ASYM ||
         f == QG_FP8_E4M3;
}

bool is_asym(qg_format f) { return f == QG_INT4_ASYM || f == QG_INT8_ASYM; }

bool is_int4(qg_format f) { return f == QG_INT4_SYM || f == QG_INT4_ASYM; }

bool is_int8(qg_format f) { return f == QG_INT8_SYM || f == QG_INT8_ASYM; }

// Shared checks of a quantized [rows][K] operand with groups along K.
qg_status check_quant_operand(qg_format fmt, int64_t rows, int64_t K, int64_t group,
                              const void* codes, const void* scales, const void* zeros) {
  if (rows < 1 || K < 1) return fail(QG_ERR_GEOMETRY, "rows and K must be positive");
  if (group <= 0 || K % group != 0) return fail(QG_ERR_GEOMETRY, "group must divide K");
  if (group % 8 != 0) return fail(QG_ERR_GEOMETRY, "group must be a multiple of 8");
  if (!codes || !scales) return fail(QG_ERR_NULL, "codes and scales are required");
  if (is_asym(fmt) && !zeros) return fail(QG_ERR_NULL, "asymmetric formats need zeros");
  if (!is_asym(fmt) && zeros) return fail(QG_ERR_NULL, "zeros must be NULL for this format");
  if (!aligned16(codes) || !aligned16(scales) || (zeros && !aligned16(zeros)))
    return fail(QG_ERR_ALIGN, "pointers must be 16-byte aligned");
  return QG_OK;
}

// The GEMM and GEMV kernels address every operand with 32-bit byte offsets
// inside a buffer resource of at most 0x7ffff000 bytes; tiles may run up to
// 256 rows past the end of an operand.
bool fits_offsets(int64_t rows, int64_t row_bytes) {
  return (rows + 256) * row_bytes <= 0x7ffff000LL;
}

qg_status qgemv_common(bool tiled, qg_format wfmt, const void* x, int64_t M, const void* wcodes,
                       const void* wscales, const void* wzeros, int64_t N, int64_t K,
                       int64_t group, void* y, void* stream) {
  if (!is_int4(wfmt)) return fail(QG_ERR_FORMAT, "qgemv: weights must be INT4_SYM or INT4_ASYM");
  if (M < 1 || M > 16) return fail(QG_ERR_GEOMETRY, "qgemv: M must be in 1..16");
  if (N < 1 || N > (int64_t)1 << 30) return fail(QG_ERR_GEOMETRY, "qgemv: N out of range");
  qg_status st = check_quant_operand(wfmt, N, K, group, wcodes, wscales, wzeros);
  if (st != QG_OK) return st;
  if (group != 128 && !qg::w4a16_group_supported(K, group))
    return fail(QG_ERR_UNSUPPORTED, "qgemv: groups of 32, 64 or a multiple of 128 (K a "
                                    "multiple of 128) are implemented");
  if (K > 65536) return fail(QG_ERR_UNSUPPORTED, "qgemv: K above 65536 is not implemented");
  if (!fits_offsets(N, K / 2) || !fits_offsets(M, K * 2))
    return fail(QG_ERR_UNSUPPORTED, "qgemv: operand larger than 2 GiB");
  if (!x || !y) return fail(QG_ERR_NULL, "qgemv: x and y are required");
  if (!aligned16(x) || !aligned16(y)) return fail(QG_ERR_ALIGN, "qgemv: x, y must be 16-byte aligned");
  if (group != 128)
    return from_hip(qg::launch_w4a16_groups(wfmt == QG_INT4_ASYM, tiled, x, M, wcodes, wscales,
                                            wzeros, N, K, group, y, (hipStream_t)stream));
  return from_hip(qg::launch_qgemv(wfmt == QG_INT4_ASYM, tiled, x, M, wcodes, wscales, wzeros, N,
                                   K, y, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int qg_abi_version(void) { return QG_ABI_VERSION; }

const char* qg_last_error(void) { return g_last_error; }

const char* qg_status_str(qg_status s) {
  switch (s) {
    case QG_OK: return "ok";
    case QG_ERR_GEOMETRY: return "invalid quantization geometry";
    case QG_ERR_ALIGN: return "misaligned pointer";
    case QG_ERR_FORMAT: return "unsupported format";
    case QG_ERR_NULL: return "null pointer";
    case QG_ERR_HIP: return "HIP error";
    case QG_ERR_UNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

qg_status qg_quantize_pack(qg_format fmt, const void* src, qg_dtype src_dtype, int64_t rows,
                           int64_t K, int64_t group, void* codes, void* scales, void* zeros,
                           void* stream) {
  if (!is_quant_fmt(fmt)) return fail(QG_ERR_FORMAT, "quantize_pack: unknown format");
  if (src_dtype != QG_BF16 && src_dtype != QG_F32)
    return fail(QG_ERR_FORMAT, "quantize_pack: source dtype must be bf16 or f32");
  qg_status st = check_quant_operand(fmt, rows, K, group, codes, scales, zeros);
  if (st != QG_OK) return st;
  if (!src) return fail(QG_ERR_NULL, "quantize_pack: src is NULL");
  if (!aligned16(src)) return fail(QG_ERR_ALIGN, "quantize_pack: src must be 16-byte aligned");
  return from_hip(qg::launch_quantize(fmt, src, src_dtype, rows, K, group, codes, scales, zeros,
                                      nullptr, false, (hipStream_t)stream));
}

qg_status qg_quantize_pack_smooth(qg_format fmt, const void* src, qg_dtype src_dtype,
                                  int64_t rows, int64_t K, int64_t group, const float* smooth,
                                  int divide, void* codes, void* scales, void* zeros,
                                  void* stream) {
  if (!is_quant_fmt(fmt)) return fail(QG_ERR_FORMAT, "quantize_pack_smooth: unknown format");
  if (src_dtype != QG_BF16 && src_dtype != QG_F32)
    return fail(QG_ERR_FORMAT, "quantize_pack_smooth: source dtype must be bf16 or f32");
  if (divide != 0 && divide != 1)
    return fail(QG_ERR_GEOMETRY, "quantize_pack_smooth: divide must be 0 or 1");
  qg_status st = check_quant_operand(fmt, rows, K, group, codes, scales, zeros);
  if (st != QG_OK) return st;
  if (K % 8 != 0) return fail(QG_ERR_GEOMETRY, "quantize_pack_smooth: K must be a multiple of 8");
  if (K / 8 > 0x7fffff00LL) return fail(QG_ERR_UNSUPPORTED, "quantize_pack_smooth: K too large");
  if (!src || !smooth) return fail(QG_ERR_NULL, "quantize_pack_smooth: src and smooth are required");
  if (!aligned16(src) || !aligned16(smooth))
    return fail(QG_ERR_ALIGN, "quantize_pack_smooth: src and smooth must be 16-byte aligned");
  return from_hip(qg::launch_quantize(fmt, src, src_dtype, rows, K, group, codes, scales, zeros,
                                      smooth, divide == 1, (hipStream_t)stream));
}

qg_status qg_channel_absmax(const void* src, qg_dtype src_dtype, int64_t rows, int64_t K,
                            int accumulate, float* absmax, void* stream) {
  if (src_dtype != QG_BF16 && src_dtype != QG_F32)
    return fail(QG_ERR_FORMAT, "channel_absmax: source dtype must be bf16 or f32");
  if (rows < 1 || K < 8 || K % 8 != 0)
    return fail(QG_ERR_GEOMETRY, "channel_absmax: rows >= 1 and K a positive multiple of 8");
  if (accumulate != 0 && accumulate != 1)
    return fail(QG_ERR_GEOMETRY, "channel_absmax: accumulate must be 0 or 1");
  if (K / 8 > 64LL * 0x7fffffffLL)
    return fail(QG_ERR_UNSUPPORTED, "channel_absmax: K too large");
  if (!src || !absmax) return fail(QG_ERR_NULL, "channel_absmax: src and absmax are required");
  if (!aligned16(src) || !aligned16(absmax))
    return fail(QG_ERR_ALIGN, "channel_absmax: pointers must be 16-byte aligned");
  return from_hip(qg::launch_channel_absmax(src, src_dtype, rows, K, accumulate == 1, absmax,
                                            (hipStream_t)stream));
}

qg_status qg_smooth_scales(const float* act_absmax, const float* w_absmax, float alpha, int64_t K,
                           float* smooth, void* stream) {
  if (K < 1) return fail(QG_ERR_GEOMETRY, "smooth_scales: K must be positive");
  if (!(alpha >= 0.f && alpha <= 1.f))
    return fail(QG_ERR_GEOMETRY, "smooth_scales: alpha must lie in [0, 1]");
  if (!act_absmax || !w_absmax || !smooth)
    return fail(QG_ERR_NULL, "smooth_scales: act_absmax, w_absmax and smooth are required");
  if (!aligned16(act_absmax) || !aligned16(w_absmax) || !aligned16(smooth))
    return fail(QG_ERR_ALIGN, "smooth_scales: pointers must be 16-byte aligned");
  return from_hip(qg::launch_smooth_scales(act_absmax, w_absmax, alpha, K, smooth,
                                           (hipStream_t)stream));
}

qg_status qg_channel_scales(const float* absmax, int64_t n, float qmax, float* scales,
                            void* stream) {
  if (n < 1) return fail(QG_ERR_GEOMETRY, "channel_scales: n must be positive");
  if (!(qmax > 0.f && qmax <= 3.4e38f))
    return fail(QG_ERR_GEOMETRY, "channel_scales: qmax must be positive and finite");
  if (!absmax || !scales) return fail(QG_ERR_NULL, "channel_scales: absmax and scales are required");
  if (!aligned16(absmax) || !aligned16(scales))
    return fail(QG_ERR_ALIGN, "channel_scales: pointers must be 16-byte aligned");
  return from_hip(qg::launch_channel_scales(absmax, n, qmax, scales, (hipStream_t)stream));
}

qg_status qg_kv_cache_store(const void* x, qg_dtype x_dtype, int64_t tokens, int64_t heads,
                            int64_t head_dim, const int64_t* slot_mapping, int64_t num_slots,
                            const float* channel_scales, void* cache_codes, float* cache_scales,
                            void* stream) {
  if (x_dtype != QG_BF16 && x_dtype != QG_F32)
    return fail(QG_ERR_FORMAT, "kv_cache_store: source dtype must be bf16 or f32");
  if (tokens < 0 || heads < 1 || num_slots < 1)
    return fail(QG_ERR_GEOMETRY, "kv_cache_store: tokens >= 0, heads >= 1 and num_slots >= 1");
  if (head_dim < 8 || head_dim > 512 || head_dim % 8 != 0)
    return fail(QG_ERR_GEOMETRY, "kv_cache_store: head_dim a multiple of 8 in [8, 512]");
  if (tokens * heads > 0x7fffffffLL - 4096 || heads > 0x7fffffffLL / head_dim)
    return fail(QG_ERR_UNSUPPORTED, "kv_cache_store: tokens * heads must stay below 2^31");
  if (num_slots > INT64_MAX / (heads * head_dim))
    return fail(QG_ERR_UNSUPPORTED, "kv_cache_store: cache too large");
  if (!cache_codes) return fail(QG_ERR_NULL, "kv_cache_store: cache_codes is required");
  if (tokens > 0 && !slot_mapping) return fail(QG_ERR_NULL, "kv_cache_store: slot_mapping is NULL");
  if (!channel_scales && !cache_scales)
    return fail(QG_ERR_NULL, "kv_cache_store: per-token mode needs cache_scales");
  if (channel_scales && cache_scales)
    return fail(QG_ERR_NULL, "kv_cache_store: cache_scales must be NULL with channel_scales");
  if (tokens > 0 && !x) return fail(QG_ERR_NULL, "kv_cache_store: x is NULL");
  if ((x && !aligned16(x)) || (channel_scales && !aligned16(channel_scales)) ||
      !aligned_to(cache_codes, 8) || (slot_mapping && !aligned_to(slot_mapping, 8)) ||
      (cache_scales && !aligned_to(cache_scales, 4)))
    return fail(QG_ERR_ALIGN, "kv_cache_store: x and channel_scales 16-byte, cache_codes and "
                              "slot_mapping 8-byte, cache_scales 4-byte aligned");
  if (tokens == 0) return ok();
  return from_hip(qg::launch_kv_cache_store(x, x_dtype, tokens, heads, head_dim, slot_mapping,
                                            num_slots, channel_scales, cache_codes, cache_scales,
                                            (hipStream_t)stream));
}

qg_status qg_norm_quant(qg_norm norm, qg_format fmt, const void* src, qg_dtype src_dtype,
                        const float* gamma, const float* beta, float eps, int64_t rows,
                        int64_t K, void* codes, void* scales, void* zeros, void* stream) {
  if (norm != QG_NORM_LAYER && norm != QG_NORM_RMS)
    return fail(QG_ERR_FORMAT, "norm_quant: unknown normalization");
  if (fmt != QG_FP8_E4M3 && fmt != QG_INT8_SYM && fmt != QG_INT8_ASYM && fmt != QG_MXFP4)
    return fail(QG_ERR_FORMAT,
                "norm_quant: format must be FP8_E4M3, INT8_SYM, INT8_ASYM or MXFP4");
  if (src_dtype != QG_BF16 && src_dtype != QG_F32)
    return fail(QG_ERR_FORMAT, "norm_quant: source dtype must be bf16 or f32");
  if (rows < 1 || rows > 0x7fffffffLL || K < 8 || K % 8 != 0)
    return fail(QG_ERR_GEOMETRY, "norm_quant: rows >= 1 and K a positive multiple of 8");
  if (!(eps >= 0.f) || !(eps <= 3.4e38f))
    return fail(QG_ERR_GEOMETRY, "norm_quant: eps must be finite and >= 0");
  if (fmt == QG_MXFP4 && K % 32 != 0)
    return fail(QG_ERR_GEOMETRY, "norm_quant: MXFP4 needs K a multiple of 32");
  qg_status st = check_quant_operand(fmt, rows, K, fmt == QG_MXFP4 ? 32 : K, codes, scales, zeros);
  if (st != QG_OK) return st;
  if (!src || !gamma) return fail(QG_ERR_NULL, "norm_quant: src and gamma are required");
  if (norm == QG_NORM_LAYER && !beta) return fail(QG_ERR_NULL, "norm_quant: LayerNorm needs beta");
  if (norm == QG_NORM_RMS && beta) return fail(QG_ERR_NULL, "norm_quant: beta must be NULL for RMSNorm");
  if (!aligned16(src) || !aligned16(gamma) || (beta && !aligned16(beta)))
    return fail(QG_ERR_ALIGN, "norm_quant: pointers must be 16-byte aligned");
  if (K > 16384) return fail(QG_ERR_UNSUPPORTED, "norm_quant: K above 16384 is not implemented");
  return from_hip(qg::launch_norm_quant(norm == QG_NORM_RMS, fmt, src, src_dtype, gamma, beta,
                                        eps, rows, K, codes, scales, zeros,
                                        (hipStream_t)stream));
}

qg_status qg_dequant(qg_format fmt, const void* codes, const void* scales, const void* zeros,
                     int64_t rows, int64_t K, int64_t group, void* dst, qg_dtype dst_dtype,
                     void* stream) {
  if (!is_quant_fmt(fmt) && fmt != QG_MXFP4) return fail(QG_ERR_FORMAT, "dequant: unknown format");
  if (dst_dtype != QG_BF16 && dst_dtype != QG_F32)
    return fail(QG_ERR_FORMAT, "dequant: destination dtype must be bf16 or f32");
  if (fmt == QG_MXFP4 && group != 32)
    return fail(QG_ERR_GEOMETRY, "dequant: MXFP4 blocks are 32 elements");
  qg_status st = check_quant_operand(fmt, rows, K, group, codes, scales, zeros);
  if (st != QG_OK) return st;
  if (!dst) return fail(QG_ERR_NULL, "dequant: dst is NULL");
  if (!aligned16(dst)) return fail(QG_ERR_ALIGN, "dequant: dst must be 16-byte aligned");
  return from_hip(qg::launch_dequant(fmt, codes, scales, zeros, rows, K, group, dst, dst_dtype,
                                     (hipStream_t)stream));
}

qg_status qg_qgemv(qg_format wfmt, const void* x, int64_t M, const void* wcodes,
                   const void* wscales, const void* wzeros, int64_t N, int64_t K, int64_t group,
                   void* y, void* stream) {
  return qgemv_common(false, wfmt, x, M, wcodes, wscales, wzeros, N, K, group, y, stream);
}

qg_status qg_qgemv_tiled(qg_format wfmt, const void* x, int64_t M, const void* tiled_codes,
                         const void* wscales, const void* wzeros, int64_t N, int64_t K,
                         int64_t group, void* y, void* stream) {
  return qgemv_common(true, wfmt, x, M, tiled_codes, wscales, wzeros, N, K, group, y, stream);
}

qg_status qg_qgemv_swiglu(qg_format wfmt, const void* x, int64_t M, const void* wcodes,
                          const void* wscales, const void* wzeros, int64_t N2, int64_t K,
                          int64_t group, int tiled, void* h, void* stream) {
  if (!is_int4(wfmt))
    return fail(QG_ERR_FORMAT, "qgemv_swiglu: weights must be INT4_SYM or INT4_ASYM");
  if (M < 1 || M > 16) return fail(QG_ERR_GEOMETRY, "qgemv_swiglu: M must be in 1..16");
  if (N2 < 2 || N2 % 2 != 0 || N2 > (int64_t)1 << 30)
    return fail(QG_ERR_GEOMETRY, "qgemv_swiglu: N2 = 2 I must be even and positive");
  if (tiled != 0 && tiled != 1) return fail(QG_ERR_GEOMETRY, "qgemv_swiglu: tiled must be 0 or 1");
  qg_status st = check_quant_operand(wfmt, N2, K, group, wcodes, wscales, wzeros);
  if (st != QG_OK) return st;
  if (group != 128) return fail(QG_ERR_UNSUPPORTED, "qgemv_swiglu: only group 128 is implemented");
  if (!qg::qgemv_swiglu_supported(M, K))
    return fail(QG_ERR_UNSUPPORTED, "qgemv_swiglu: K must be a multiple of 512, at most 32768 "
                                    "(M = 1), 16384 (M = 2..4) or 8192 (M = 5..16)");
  if (!fits_offsets(N2, K / 2) || !fits_offsets(M, K * 2))
    return fail(QG_ERR_UNSUPPORTED, "qgemv_swiglu: operand larger than 2 GiB");
  if (!x || !h) return fail(QG_ERR_NULL, "qgemv_swiglu: x and h are required");
  if (!aligned16(x) || !aligned16(h))
    return fail(QG_ERR_ALIGN, "qgemv_swiglu: x, h must be 16-byte aligned");
  return from_hip(qg::launch_qgemv_swiglu(wfmt == QG_INT4_ASYM, tiled == 1, x, M, wcodes,
                                          wscales, wzeros, N2, K, h, (hipStream_t)stream));
}

qg_status qg_tile_gemv_weights(const void* codes, int64_t N, int64_t K, void* tiled_codes,
                               void* stream) {
  if (N < 1 || N > (int64_t)1 << 30 || K < 128 || K % 128 != 0)
    return fail(QG_ERR_GEOMETRY, "tile_gemv_weights: N >= 1 and K a positive multiple of 128");
  if (K > 65536) return fail(QG_ERR_UNSUPPORTED, "tile_gemv_weights: K above 65536");
  if (!fits_offsets(N, K / 2))
    return fail(QG_ERR_UNSUPPORTED, "tile_gemv_weights: codes larger than 2 GiB");
  if (!codes || !tiled_codes) return fail(QG_ERR_NULL, "tile_gemv_weights: NULL pointer");
  if (!aligned16(codes) || !aligned16(tiled_codes))
    return fail(QG_ERR_ALIGN, "tile_gemv_weights: pointers must be 16-byte aligned");
  if (codes == tiled_codes) return fail(QG_ERR_UNSUPPORTED, "tile_gemv_weights: not in place");
  return from_hip(qg::launch_tile_gemv_codes(codes, N, K, tiled_codes, (hipStream_t)stream));
}

qg_status qg_qgemm(qg_format wfmt, qg_format afmt, const void* a, const void* a_scales,
                   const void* a_zeros, int64_t M, const void* wcodes, const void* wscales,
                   const void* wzeros, int64_t N, int64_t K, int64_t group, void* y,
                   void* stream) {
  if (M < 1 || N < 1 || K < 1) return fail(QG_ERR_GEOMETRY, "qgemm: M, N, K must be positive");
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30)
    return fail(QG_ERR_GEOMETRY, "qgemm: size out of range");
  if (!a || !y) return fail(QG_ERR_NULL, "qgemm: a and y are required");
  if (!aligned16(a) || !aligned16(y)) return fail(QG_ERR_ALIGN, "qgemm: a, y must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  {
    const int64_t wrow = is_int4(wfmt) ? K / 2 : K;
    const int64_t arow = afmt == QG_BF16_ACT ? K * 2 : K;
    if (!fits_offsets(N, wrow) || !fits_offsets(M, arow))
      return fail(QG_ERR_UNSUPPORTED, "qgemm: operand larger than 2 GiB");
  }
  if (is_int4(wfmt) && afmt == QG_BF16_ACT) {
    qg_status st = check_quant_operand(wfmt, N, K, group, wcodes, wscales, wzeros);
    if (st != QG_OK) return st;
    if (group != 128 && !qg::w4a16_group_supported(K, group))
      return fail(QG_ERR_UNSUPPORTED, "qgemm W4A16: groups of 32, 64 or a multiple of 128 (K a "
                                      "multiple of 128) are implemented");
    if (a_scales || a_zeros) return fail(QG_ERR_NULL, "qgemm W4A16: a_scales/a_zeros must be NULL");
    if (group != 128 && M > 16 * 65535)
      return fail(QG_ERR_UNSUPPORTED, "qgemm W4A16: M above 1048560 with a group other than 128");
    if (group != 128)
      return from_hip(qg::launch_w4a16_groups(wfmt == QG_INT4_ASYM, false, a, M, wcodes, wscales,
                                              wzeros, N, K, group, y, s));
    return from_hip(qg::launch_gemm_w4a16(wfmt == QG_INT4_ASYM, a, M, wcodes, wscales, wzeros, N,
                                          K, y, s));
  }
  if (wfmt == QG_FP8_E4M3 && afmt == QG_FP8_E4M3) {
    if (group != K) return fail(QG_ERR_UNSUPPORTED, "qgemm FP8: per-row scales only (group == K)");
    if (K % 16 != 0) return fail(QG_ERR_GEOMETRY, "qgemm FP8: K must be a multiple of 16");
    qg_status st = check_quant_operand(wfmt, N, K, group, wcodes, wscales, wzeros);
    if (st != QG_OK) return st;
    st = check_quant_operand(afmt, M, K, group, a, a_scales, a_zeros);
    if (st != QG_OK) return st;
    return from_hip(qg::launch_gemm_fp8(a, a_scales, M, wcodes, wscales, N, K, y, s));
  }
  if (is_int8(wfmt) && is_int8(afmt)) {
    if (group != K) return fail(QG_ERR_UNSUPPORTED, "qgemm INT8: per-row scales only (group == K)");
    if (K % 16 != 0) return fail(QG_ERR_GEOMETRY, "qgemm INT8: K must be a multiple of 16");
    qg_status st = check_quant_operand(wfmt, N, K, group, wcodes, wscales, wzeros);
    if (st != QG_OK) return st;
    st = check_quant_operand(afmt, M, K, group, a, a_scales, a_zeros);
    if (st != QG_OK) return st;
    return from_hip(qg::launch_gemm_int8(afmt == QG_INT8_ASYM, wfmt == QG_INT8_ASYM, a, a_scales,
                                         a_zeros, M, wcodes, wscales, wzeros, N, K, y, s));
  }
  return fail(QG_ERR_FORMAT, "qgemm: unsupported format pair");
}

qg_status qg_qgemm_swiglu(qg_format wfmt, qg_format afmt, const void* a, int64_t M,
                          const void* wcodes, const void* wscales, const void* wzeros,
                          int64_t N2, int64_t K, int64_t group, void* h, void* stream) {
  if (!is_int4(wfmt) || afmt != QG_BF16_ACT)
    return fail(QG_ERR_FORMAT, "qgemm_swiglu: weights INT4_SYM / INT4_ASYM with BF16_ACT activations");
  if (M < 1 || N2 < 2 || K < 1 || N2 % 2 != 0)
    return fail(QG_ERR_GEOMETRY, "qgemm_swiglu: M, K positive and N2 = 2 I even");
  if (M > (int64_t)1 << 30 || N2 > (int64_t)1 << 30 || K > (int64_t)1 << 30)
    return fail(QG_ERR_GEOMETRY, "qgemm_swiglu: size out of range");
  if (!a || !h) return fail(QG_ERR_NULL, "qgemm_swiglu: a and h are required");
  if (!aligned16(a) || !aligned16(h))
    return fail(QG_ERR_ALIGN, "qgemm_swiglu: a, h must be 16-byte aligned");
  qg_status st = check_quant_operand(wfmt, N2, K, group, wcodes, wscales, wzeros);
  if (st != QG_OK) return st;
  if (group != 128) return fail(QG_ERR_UNSUPPORTED, "qgemm_swiglu: only group 128 is implemented");
  if (!fits_offsets(N2, K / 2) || !fits_offsets(M, K * 2))
    return fail(QG_ERR_UNSUPPORTED, "qgemm_swiglu: operand larger than 2 GiB");
  return from_hip(qg::launch_gemm_w4a16_swiglu(wfmt == QG_INT4_ASYM, a, M, wcodes, wscales, wzeros,
                                               N2, K, h, (hipStream_t)stream));
}

qg_status qg_qgemm_swiglu_fp8(const void* a, const void* a_scales, int64_t M, const void* wcodes,
                              const void* wscales, int64_t N2, int64_t K, void* h, void* stream) {
  if (M < 1 || N2 < 2 || K < 1 || N2 % 2 != 0)
    return fail(QG_ERR_GEOMETRY, "qgemm_swiglu_fp8: M, K positive and N2 = 2 I even");
  if (M > (int64_t)1 << 30 || N2 > (int64_t)1 << 30 || K > (int64_t)1 << 30)
    return fail(QG_ERR_GEOMETRY, "qgemm_swiglu_fp8: size out of range");
  if (K % 16 != 0) return fail(QG_ERR_GEOMETRY, "qgemm_swiglu_fp8: K must be a multiple of 16");
  qg_status st = check_quant_operand(QG_FP8_E4M3, N2, K, K, wcodes, wscales, nullptr);
  if (st != QG_OK) return st;
  st = check_quant_operand(QG_FP8_E4M3, M, K, K, a, a_scales, nullptr);
  if (st != QG_OK) return st;
  if (!h) return fail(QG_ERR_NULL, "qgemm_swiglu_fp8: h is required");
  if (!aligned16(h)) return fail(QG_ERR_ALIGN, "qgemm_swiglu_fp8: h must be 16-byte aligned");
  if (!fits_offsets(N2, K) || !fits_offsets(M, K))
    return fail(QG_ERR_UNSUPPORTED, "qgemm_swiglu_fp8: operand larger than 2 GiB");
  return from_hip(qg::launch_gemm_fp8_swiglu(a, a_scales, M, wcodes, wscales, N2, K, h,
                                             (hipStream_t)stream));
}

qg_status qg_mx_quant(const void* src, qg_dtype src_dtype, int64_t rows, int64_t K, void* codes,
                      void* e8m0, void* stream) {
  if (src_dtype != QG_BF16 && src_dtype != QG_F32)
    return fail(QG_ERR_FORMAT, "mx_quant: source dtype must be bf16 or f32");
  if (rows < 1 || K < 32 || K % 32 != 0)
    return fail(QG_ERR_GEOMETRY, "mx_quant: rows >= 1 and K a positive multiple of 32");
  if (!src || !codes || !e8m0) return fail(QG_ERR_NULL, "mx_quant: NULL pointer");
  if (!aligned16(src) || !aligned16(codes) || !aligned16(e8m0))
    return fail(QG_ERR_ALIGN, "mx_quant: pointers must be 16-byte aligned");
  return from_hip(qg::launch_mx_quant(src, src_dtype, rows, K, codes, e8m0, (hipStream_t)stream));
}

qg_status qg_mx_gemm(const void* a_codes, const void* a_e8m0, int64_t M, const void* b_codes,
                     const void* b_e8m0, int64_t N, int64_t K, void* y, void* stream) {
  if (M < 1 || N < 1 || K < 32 || K % 32 != 0)
    return fail(QG_ERR_GEOMETRY, "mx_gemm: M, N >= 1 and K a positive multiple of 32");
  if (M > (int64_t)1 << 30 || N > (int64_t)1 << 30 || K > (int64_t)1 << 30)
    return fail(QG_ERR_GEOMETRY, "mx_gemm: size out of range");
  if (!fits_offsets(M, K / 2) || !fits_offsets(N, K / 2))
    return fail(QG_ERR_UNSUPPORTED, "mx_gemm: operand larger than 2 GiB");
  if (!a_codes || !a_e8m0 || !b_codes || !b_e8m0 || !y) return fail(QG_ERR_NULL, "mx_gemm: NULL pointer");
  if (!aligned16(a_codes) || !aligned16(a_e8m0) || !aligned16(b_codes) || !aligned16(b_e8m0) ||
      !aligned16(y))
    return fail(QG_ERR_ALIGN, "mx_gemm: pointers must be 16-byte aligned");
  return from_hip(qg::launch_mx_gemm(a_codes, a_e8m0, M, b_codes, b_e8m0, N, K, y,
                                     (hipStream_t)stream));
}

qg_status qg_calib_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (bytes < 65536 || bytes % 65536 != 0 || bytes > ((int64_t)1 << 40))
    return fail(QG_ERR_GEOMETRY, "calib_stream_read: bytes a positive multiple of 65536");
  if (!src || !sink) return fail(QG_ERR_NULL, "calib_stream_read: src and sink are required");
  if (!aligned16(src) || !aligned_to(sink, 4))
    return fail(QG_ERR_ALIGN, "calib_stream_read: src 16-byte, sink 4-byte aligned");
  return from_hip(qg::launch_calib_stream_read(src, bytes, sink, (hipStream_t)stream));
}

qg_status qg_calib_mfma(qg_calib_kind kind, int64_t waves, int64_t iters, float* sink,
                        void* stream) {
  if (kind != QG_CALIB_BF16 && kind != QG_CALIB_FP8 && kind != QG_CALIB_FP4 &&
      kind != QG_CALIB_INT8)
    return fail(QG_ERR_FORMAT, "calib_mfma: unknown kind");
  if (waves < 4 || waves % 4 != 0 || waves > ((int64_t)1 << 20) || iters < 1 ||
      iters > ((int64_t)1 << 24))
    return fail(QG_ERR_GEOMETRY, "calib_mfma: waves a positive multiple of 4, iters 1 .. 2^24");
  if (!sink) return fail(QG_ERR_NULL, "calib_mfma: sink is required");
  if (!aligned_to(sink, 4)) return fail(QG_ERR_ALIGN, "calib_mfma: sink must be 4-byte aligned");
  return from_hip(qg::launch_calib_mfma((int)kind, waves, iters, sink, (hipStream_t)stream));
}

qg_status qg_debug_fp32_output(float* out, void* stream) {
  (void)stream;
#ifdef QG_DEBUG_FP32
  if (out && !aligned_to(out, 4)) return fail(QG_ERR_ALIGN, "debug_fp32_output: 4-byte aligned");
  hipError_t e = qg::debug_set_gemv(out);
  if (e == hipSuccess) e = qg::debug_set_f8f4(out);
  if (e == hipSuccess) e = qg::debug_set_int8(out);
  if (e == hipSuccess) e = qg::debug_set_w4a16(out);
  return from_hip(e);
#else
  (void)out;
  return fail(QG_ERR_UNSUPPORTED, "debug_fp32_output: this library was built without "
                                  "QG_DEBUG_FP32 (use libqgemm_debug.so)");
#endif
}

int qg_debug_build(void) {
#ifdef QG_DEBUG_FP32
  return 1;
#else
  return 0;
#endif
}

}  // extern "C"
