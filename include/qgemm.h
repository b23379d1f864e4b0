/*
 * qgemm.h -- C ABI of the quantized linear layer library for AMD Instinct
 * MI355X (gfx950).
 *
 * Y = X * W^T.  W is stored [N][K] row-major (row n = output channel), X is
 * [M][K] and Y is [M][N], both row-major.  Quantization groups and MX blocks
 * run along K.
 *
 * Sources of the operations (page titles, with the section used):
 *   [Q&A]  《量化与加速》: format table (E4M3 +-448, E5M2 +-57344, INT8, INT4
 *          [-8,7]), float formula, "INT8 量化原理" affine equations
 *          x_q = clip(round(x/s) + z), x_hat = s (x_q - z).
 *   [SRV]  《推理优化与量化算子深度技术调研》 section 1.2 (INT8 symmetric scale
 *          max|x|/127 with clip +-127, asymmetric scale (max-min)/255 with
 *          zero point round(-min/s) and clip [0,255]; dequantization fused
 *          into the GEMM), 1.3 (group-wise INT4, group 128, W4A16 decode is
 *          HBM bound), 1.4 (FP8 E4M3 with an fp32 scale tensor), 1.5
 *          (SmoothQuant factor and folding), 1.6 (FP8 KV-cache
 *          quantization, per token or per channel), 4.4 (normalization +
 *          quantization fusion), 4.6 (GEMM + activation fusion).
 *   [L6]   《第 6 课：量化源码走读》 section 2 (eight INT4 codes per int32;
 *          W4A16 dequantizes inside the GEMM; W8A8/FP8 quantizes activations
 *          dynamically; figure 6-2 Out = acc * scale_x * scale_w; micro-block
 *          scaling), section 3 (the asymmetric cross term must be kept; the
 *          MX block must divide K), practice exercise (a zero block uses
 *          scale 1; invalid geometry is an error).
 *   [MX]   《大模型量化推理引擎全景大复盘》 section 2 eq. 3 (32 four-bit
 *          elements share one E8M0 exponent), section 3 code (shared scale
 *          2^ceil(log2(max|x|/6))).
 *   [CH1]  《第 1 章：推理加速全景》 section 1.5 (the roofline: attainable
 *          throughput = min(bandwidth x intensity, peak); calibration
 *          probes), section 4.1 (uniform quantization math),
 *          section 4.3 (SmoothQuant: X W = (X diag(s)^-1)(diag(s) W),
 *          s_j = max|X_j|^alpha / max|W_j|^(1-alpha)).
 *   [Q&A] also its KV-cache section (keys per channel, values per token).
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronizes; each call only enqueues work on
 *     `stream` (a hipStream_t; NULL = the default stream) and returns.
 *   - Arguments are validated before any HIP call; on an error nothing is
 *     enqueued and a status other than QG_OK is returned.  QG_ERR_HIP reports
 *     a failed kernel launch (hipGetLastError after the launch).
 *   - Every data pointer must be 16-byte aligned (QG_ERR_ALIGN otherwise);
 *     128-bit loads and stores are used throughout.  (qg_kv_cache_store
 *     states its own, smaller requirements for its cache-side pointers.)
 *   - round() is round-half-to-even; x/s is one IEEE fp32 division by the
 *     scale as stored; a scale that is zero (an all-zero group) is stored as 1.
 *   - Calls are stateless and re-entrant; calls on different streams may run
 *     concurrently (they share no state).
 *
 * Storage formats (bit-exact, and what the kernels read):
 *   INT4_SYM   codes int32 [rows][K/8]: element k = 8j+i in bits 4i..4i+3 of
 *              word j (LSB first), two's-complement nibble; q in [-8,7];
 *              scales fp16 [rows][K/group] = fp16(max|x|/7) (saturating).
 *   INT4_ASYM  same packing, unsigned nibble q in [0,15]; scales fp16 =
 *              fp16((max-min)/15); zeros fp16 [rows][K/group], integer
 *              values round(-min/s), not clamped.
 *   INT8_SYM   codes int8 [rows][K], q in [-127,127]; scales fp32 =
 *              max|x|/127 [rows][K/group].
 *   INT8_ASYM  codes uint8 [rows][K], q in [0,255]; scales fp32 = (max-min)/255;
 *              zeros fp32 [rows][K/group].
 *   FP8_E4M3   codes uint8 [rows][K], OCP E4M3FN bits, nearest value with ties
 *              to even, saturating at +-448 (never NaN), sign kept;
 *              scales fp32 [rows][K/group] = max|x|/448.
 *   MXFP4      codes uint8 [rows][K/2], E2M1 sign-magnitude nibbles, element
 *              2j in the low nibble of byte j; E8M0 uint8 [rows][K/32] = e+127
 *              with e the smallest integer such that max|x| <= 6*2^e over the
 *              32-element block (0 for an all-zero block), clamped to
 *              [-127,127].
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QG_ABI_VERSION 1

typedef enum {
    QG_OK = 0,
    QG_ERR_GEOMETRY = 1,     /* sizes: non-positive, group does not divide K, ... */
    QG_ERR_ALIGN = 2,        /* a pointer is not 16-byte aligned */
    QG_ERR_FORMAT = 3,       /* unknown format or unsupported format pair */
    QG_ERR_NULL = 4,         /* a required pointer is NULL */
    QG_ERR_HIP = 5,          /* the HIP runtime reported an error at launch */
    QG_ERR_UNSUPPORTED = 6   /* valid but not implemented (e.g. GEMV group != 128) */
} qg_status;

typedef enum {
    QG_BF16 = 0,
    QG_F32 = 1
} qg_dtype;

typedef enum {
    QG_INT4_SYM = 0,
    QG_INT4_ASYM = 1,
    QG_INT8_SYM = 2,
    QG_INT8_ASYM = 3,
    QG_FP8_E4M3 = 4,
    QG_BF16_ACT = 5,   /* unquantized bf16 activations (the A side of W4A16) */
    QG_MXFP4 = 6
} qg_format;

/*
 * qg_quantize_pack -- quantize `rows` x `K` values along K in groups of
 * `group` (group == K: one scale per row, i.e. per output channel for
 * weights or per token for activations).  [Q&A] "INT8 量化原理"; [SRV] 1.2,
 * 1.3, 1.4; [L6] section 2 (dynamic per-token activation quantization,
 * eight INT4 codes per int32) and the practice exercise (zero block -> 1).
 *   fmt        QG_INT4_SYM | QG_INT4_ASYM | QG_INT8_SYM | QG_INT8_ASYM |
 *              QG_FP8_E4M3.
 *   src        [rows][K] of src_dtype (QG_BF16 or QG_F32), row-major.
 *   group      > 0, divides K, and a multiple of 8 (every format).
 *   codes, scales, zeros   outputs in the storage format above; zeros is
 *              required for *_ASYM and must be NULL otherwise.
 * Errors: QG_ERR_GEOMETRY (rows < 1, K < 1, bad group), QG_ERR_FORMAT,
 * QG_ERR_NULL, QG_ERR_ALIGN, QG_ERR_HIP.
 */
qg_status qg_quantize_pack(qg_format fmt, const void* src, qg_dtype src_dtype,
                           int64_t rows, int64_t K, int64_t group,
                           void* codes, void* scales, void* zeros, void* stream);

/*
 * qg_dequant -- x_hat = s * (q - z) per group ([Q&A] "INT8 量化原理"; [SRV]
 * 1.2), or 2^(e8m0-127) * e2m1(q) per 32-block for QG_MXFP4 ([MX]).
 *   fmt        any quantized format (QG_MXFP4: scales = E8M0 bytes, group
 *              must be 32, zeros NULL).
 *   dst        [rows][K] of dst_dtype.  QG_F32 is the value s*(q-z) rounded
 *              once to fp32; QG_BF16 is that fp32 value rounded to bf16 (RNE).
 * Errors as for qg_quantize_pack.
 */
qg_status qg_dequant(qg_format fmt, const void* codes, const void* scales, const void* zeros,
                     int64_t rows, int64_t K, int64_t group,
                     void* dst, qg_dtype dst_dtype, void* stream);

/*
 * qg_qgemv -- W4A16 decode product Y = X * dequant(W)^T for 1 <= M <= 16
 * ([SRV] 1.3: the small-batch W4A16 GEMV is HBM bound; [L6] section 2:
 * dequantization happens inside the kernel; section 3: the zero-point cross
 * term).  Computes
 *   y[m][n] = bf16( sum_g s[n][g] * sum_{k in g} x[m][k] * (q[n][k] - z[n][g]) )
 * with fp32 accumulation and one round-to-nearest-even conversion to bf16.
 *   wfmt       QG_INT4_SYM (wzeros NULL) or QG_INT4_ASYM.
 *   x          bf16 [M][K];  wcodes int32 [N][K/8];  wscales/wzeros fp16
 *              [N][K/group];  y bf16 [M][N].
 *   group      128 (the tuned kernels), or 32, 64 or a multiple of 128
 *              dividing K ([CH1] section 4.1: per-group granularity from 32
 *              to 128) on a general kernel that flushes each group's
 *              partial sum with its own scale; K % 128 == 0 in every case.
 * Errors: QG_ERR_GEOMETRY (M outside 1..16, N < 1, K not a multiple of
 * group), QG_ERR_UNSUPPORTED (another group size, K > 65536, or codes / x
 * padded by 256 rows larger than 2 GiB - 4 KiB), QG_ERR_FORMAT,
 * QG_ERR_NULL, QG_ERR_ALIGN, QG_ERR_HIP.
 */
qg_status qg_qgemv(qg_format wfmt, const void* x, int64_t M,
                   const void* wcodes, const void* wscales, const void* wzeros,
                   int64_t N, int64_t K, int64_t group, void* y, void* stream);

/*
 * qg_tile_gemv_weights -- the one-time relayout of INT4 codes for the decode
 * GEMV ([L6] section 2: weights are re-laid-out for the kernel's access
 * pattern after loading, process_weights_after_loading; [SRV] 1.3: Marlin's
 * interleaved weight layout is the NVIDIA prior art).  Tiled layout: tile t
 * (rows 16t .. 16t+15), group g (128 codes = 64 bytes per row) is one
 * contiguous 1 KiB block at byte (t * K/128 + g) * 1024, holding the 16 rows'
 * 64-byte group segments a quarter at a time: bytes 16q .. 16q+15 of the
 * segment of row r (0..15) at block offset 256 q + 16 r, each exactly as in
 * the canonical packing (same nibble order); rows past N in the last tile
 * are zero.  The
 * nibbles only move, so INT4_SYM and INT4_ASYM tile alike, and the scales
 * and zero points keep their canonical [N][K/group] layout.
 *   codes        int32 [N][K/8], the canonical packing of qg_quantize_pack.
 *   tiled_codes  ceil(N/16) * 16 * K/2 bytes (caller-owned, not `codes`).
 * Errors: QG_ERR_GEOMETRY (N < 1, K not a positive multiple of 128),
 * QG_ERR_UNSUPPORTED (K > 65536, codes larger than 2 GiB - 4 KiB, in place),
 * QG_ERR_NULL, QG_ERR_ALIGN, QG_ERR_HIP.
 */
qg_status qg_tile_gemv_weights(const void* codes, int64_t N, int64_t K, void* tiled_codes,
                               void* stream);

/*
 * qg_qgemv_tiled -- qg_qgemv on codes in the tiled layout of
 * qg_tile_gemv_weights (same arguments, results bit-identical to qg_qgemv on
 * the canonical codes).  Every 16-byte code load then covers whole cache
 * lines and is issued with the non-temporal hint, which streams HBM faster
 * than the canonical layout's half-line loads.
 */
qg_status qg_qgemv_tiled(qg_format wfmt, const void* x, int64_t M, const void* tiled_codes,
                         const void* wscales, const void* wzeros, int64_t N, int64_t K,
                         int64_t group, void* y, void* stream);

/*
 * qg_qgemv_swiglu -- fused SwiGLU projection of W4A16 decode:
 * H = SiLU(X W_gate^T) * (X W_up^T) for 1 <= M <= 16 rows of X ([SRV]
 * section 4.6: the gate and up projections as one product over the
 * concatenation [W_gate; W_up], SiLU and the product formed in registers, H
 * written once; SiLU(g) = g / (1 + e^-g)).  Each of g and u is the qg_qgemv
 * sum in fp32; h = bf16(SiLU(g) * u), one rounding.
 *   wfmt       QG_INT4_SYM (wzeros NULL) or QG_INT4_ASYM; group 128.
 *   x          bf16 [M][K].
 *   wcodes, wscales, wzeros   the quantized [N2][K] concatenation: rows
 *              0 .. N2/2 - 1 are W_gate, rows N2/2 .. N2 - 1 are W_up;
 *              codes canonical (tiled = 0, qg_quantize_pack) or in the tile
 *              layout of qg_tile_gemv_weights over all N2 rows (tiled = 1);
 *              scales and zeros fp16 [N2][K/group] either way.
 *   N2         2 I, even.
 *   h          bf16 [M][I].
 * Limits: K a multiple of 512 and at most 32768 (M = 1), 16384 (M = 2..4)
 * or 8192 (M = 5..16), QG_ERR_UNSUPPORTED otherwise.
 * Errors: QG_ERR_GEOMETRY (M outside 1..16, N2 odd or < 2, group not
 * dividing K, tiled not 0/1), QG_ERR_FORMAT, QG_ERR_UNSUPPORTED, QG_ERR_NULL,
 * QG_ERR_ALIGN, QG_ERR_HIP.
 */
qg_status qg_qgemv_swiglu(qg_format wfmt, const void* x, int64_t M, const void* wcodes,
                          const void* wscales, const void* wzeros, int64_t N2, int64_t K,
                          int64_t group, int tiled, void* h, void* stream);

/*
 * qg_qgemm -- quantized GEMM Y = dequant(A) * dequant(W)^T, fp32
 * accumulation, bf16 output (round to nearest even).  Format pairs:
 *   W INT4_SYM|INT4_ASYM, A BF16_ACT : W4A16 prefill ([SRV] 1.3; [L6] sec. 2);
 *       a = bf16 [M][K], a_scales/a_zeros NULL; group 128 (the MFMA prefill
 *       kernel), or 32, 64 or a multiple of 128 dividing K (the general
 *       kernel of qg_qgemv, over blocks of 16 rows; M <= 1048560).
 *   W FP8_E4M3, A FP8_E4M3 : FP8 W8A8 ([L6] figure 6-2: the product of the
 *       codes is rescaled by s_x[m] * s_w[n]); per-row scales only
 *       (group == K): a_scales fp32 [M], wscales fp32 [N].
 *   W INT8_SYM|INT8_ASYM, A INT8_SYM|INT8_ASYM : INT8 W8A8 ([SRV] 1.2;
 *       [L6] section 3 cross terms); per-row scales/zeros (group == K).
 *       The integer sums are exact for every accepted K (int32 runs of
 *       at most 65536 elements folded into fp64).
 *   y          bf16 [M][N].
 * Errors: QG_ERR_GEOMETRY (M, N, K < 1; K % 128 for W4A16; K % 16 for the
 * 8-bit formats; group), QG_ERR_FORMAT, QG_ERR_UNSUPPORTED (also when an
 * operand, padded by 256 rows, exceeds 2 GiB - 4 KiB: the kernels address
 * each array with 32-bit byte offsets), QG_ERR_NULL, QG_ERR_ALIGN,
 * QG_ERR_HIP.
 */
qg_status qg_qgemm(qg_format wfmt, qg_format afmt,
                   const void* a, const void* a_scales, const void* a_zeros, int64_t M,
                   const void* wcodes, const void* wscales, const void* wzeros,
                   int64_t N, int64_t K, int64_t group, void* y, void* stream);

/*
 * qg_qgemm_swiglu -- fused SwiGLU projection of W4A16 prefill:
 * H = SiLU(X W_gate^T) * (X W_up^T) ([SRV] section 4.6: the gate and up
 * projections as one GEMM over the concatenation [W_gate; W_up], SiLU and the
 * product formed in registers, H written once; SiLU(g) = g / (1 + e^-g)).
 *   wfmt       QG_INT4_SYM | QG_INT4_ASYM; afmt QG_BF16_ACT; group 128.
 *   a          bf16 [M][K].
 *   wcodes, wscales, wzeros   the quantized [N2][K] concatenation: rows
 *              0 .. N2/2 - 1 are W_gate, rows N2/2 .. N2 - 1 are W_up (the
 *              storage format of qg_quantize_pack).
 *   N2         2 I, even.
 *   h          bf16 [M][I]; each value is the fp32 SiLU(gate) * up rounded
 *              once (RNE).
 * Errors as for qg_qgemm; QG_ERR_GEOMETRY for an odd N2.
 */
qg_status qg_qgemm_swiglu(qg_format wfmt, qg_format afmt, const void* a, int64_t M,
                          const void* wcodes, const void* wscales, const void* wzeros,
                          int64_t N2, int64_t K, int64_t group, void* h, void* stream);

/*
 * qg_qgemm_swiglu_fp8 -- fused SwiGLU projection of FP8 W8A8 prefill:
 * H = SiLU(G) * U with G, U the rescaled code products of qg_qgemm's FP8
 * pair ([L6] figure 6-2: acc * s_x[m] * s_w[n]) over the gate and up rows of
 * the concatenation [W_gate; W_up] ([SRV] section 4.6: the W8A8 GEMM with
 * dequantization and activation fused, H written once).  Per output,
 * g = acc_g * (s_x * s_g) and u = acc_u * (s_x * s_u) in fp32, then
 * h = bf16(g / (1 + e^-g) * u), one rounding.
 *   a, a_scales   FP8 E4M3 activation codes uint8 [M][K] and their per-token
 *                 fp32 scales [M] (qg_quantize_pack, group == K).
 *   wcodes, wscales   the per-row FP8 quantized [N2][K] concatenation: rows
 *                 0 .. N2/2 - 1 gate, rows N2/2 .. N2 - 1 up; scales fp32 [N2].
 *   h             bf16 [M][N2/2].
 * Errors: QG_ERR_GEOMETRY (M, K < 1, K % 16, N2 odd or < 2), QG_ERR_NULL,
 * QG_ERR_ALIGN, QG_ERR_UNSUPPORTED (an operand, padded by 256 rows, larger
 * than 2 GiB - 4 KiB), QG_ERR_HIP.
 */
qg_status qg_qgemm_swiglu_fp8(const void* a, const void* a_scales, int64_t M, const void* wcodes,
                              const void* wscales, int64_t N2, int64_t K, void* h, void* stream);

/*
 * qg_channel_absmax -- per-channel statistics for calibration ([CH1]
 * section 4.3; [SRV] 1.5 per_channel_max): absmax[k] = max over rows of
 * |src[r][k]|, exact.
 *   src         [rows][K] of src_dtype (QG_BF16 or QG_F32); K % 8 == 0.
 *   accumulate  0: absmax is overwritten; 1: absmax holds a running maximum
 *               (non-negative floats, e.g. of earlier calibration batches)
 *               and is raised where this batch is larger.
 *   absmax      fp32 [K].
 * A NaN in a column gives a NaN maximum.  Overlapping calls on one absmax
 * race only in order, not in result (the update is an atomic max).
 * Errors: QG_ERR_GEOMETRY, QG_ERR_FORMAT, QG_ERR_NULL, QG_ERR_ALIGN,
 * QG_ERR_HIP.
 */
qg_status qg_channel_absmax(const void* src, qg_dtype src_dtype, int64_t rows, int64_t K,
                            int accumulate, float* absmax, void* stream);

/*
 * qg_smooth_scales -- SmoothQuant factors ([CH1] section 4.3; [SRV] 1.5):
 * smooth[j] = act_absmax[j]^alpha / w_absmax[j]^(1 - alpha), evaluated in
 * fp64 and rounded once to fp32; 1 where a statistic is zero (or NaN) or the
 * factor is not a positive normal fp32 value.
 *   act_absmax  fp32 [K], channel maxima of calibration activations.
 *   w_absmax    fp32 [K], channel maxima of the weights (column maxima of
 *               W [N][K]).
 *   alpha       migration strength in [0, 1] (QG_ERR_GEOMETRY otherwise).
 *   smooth      fp32 [K].
 */
qg_status qg_smooth_scales(const float* act_absmax, const float* w_absmax, float alpha, int64_t K,
                           float* smooth, void* stream);

/*
 * qg_quantize_pack_smooth -- qg_quantize_pack of the smoothed operand
 * ([CH1] section 4.3; [SRV] 1.5: W_hat = W * s offline, X_hat = X / s).
 * Element (r, k) is first multiplied by smooth[k] (divide = 0: weights,
 * W diag(s)) or divided by it (divide = 1: activations, X diag(s)^-1), one
 * fp32 rounding, then quantized exactly as qg_quantize_pack does (same
 * formats, groups, outputs and errors).  The smoothed operand is never
 * written.  smooth: fp32 [K], positive and finite; the smoothed values must
 * stay finite.
 */
qg_status qg_quantize_pack_smooth(qg_format fmt, const void* src, qg_dtype src_dtype,
                                  int64_t rows, int64_t K, int64_t group, const float* smooth,
                                  int divide, void* codes, void* scales, void* zeros,
                                  void* stream);

/*
 * qg_channel_scales -- static per-channel scales from calibration maxima
 * ([SRV] 1.6 per-channel granularity): scales[i] = absmax[i] / qmax (one
 * fp32 division), 1 where that is zero.  For FP8 E4M3 KV channels qmax is
 * 448.  Errors: QG_ERR_GEOMETRY (n < 1, qmax not positive and finite),
 * QG_ERR_NULL, QG_ERR_ALIGN, QG_ERR_HIP.
 */
qg_status qg_channel_scales(const float* absmax, int64_t n, float qmax, float* scales,
                            void* stream);

/*
 * qg_kv_cache_store -- FP8 E4M3 quantization of new keys or values into a
 * paged cache ([SRV] 1.6; [Q&A] KV-cache section).
 *   x            [tokens][heads][head_dim] of x_dtype (QG_BF16 or QG_F32),
 *                16-byte aligned; tokens may be 0 (nothing is enqueued).
 *   head_dim     a multiple of 8 in [8, 512].
 *   slot_mapping int64 [tokens], 8-byte aligned: token t is written to slot
 *                slot_mapping[t]; a slot outside [0, num_slots) (negative
 *                marks padding) is skipped.  The slots of one call must be
 *                distinct.
 *   channel_scales  NULL: per token and head, scale = max_d |x[t][h][d]| /
 *                448 (1 when zero), written to cache_scales.  Otherwise fp32
 *                [heads][head_dim] static scales (16-byte aligned, e.g. from
 *                qg_channel_absmax and qg_channel_scales over calibration
 *                keys); codes of values beyond the calibrated range saturate
 *                at +-448, and cache_scales must be NULL.
 *   cache_codes  uint8 [num_slots][heads][head_dim], 8-byte aligned; E4M3
 *                codes of x / scale (one fp32 division), ties to even.
 *   cache_scales fp32 [num_slots][heads], 4-byte aligned (per-token mode).
 * Inputs must be finite.  Errors: QG_ERR_GEOMETRY, QG_ERR_FORMAT,
 * QG_ERR_UNSUPPORTED (tokens * heads >= 2^31 - 4096), QG_ERR_NULL,
 * QG_ERR_ALIGN, QG_ERR_HIP.
 */
qg_status qg_kv_cache_store(const void* x, qg_dtype x_dtype, int64_t tokens, int64_t heads,
                            int64_t head_dim, const int64_t* slot_mapping, int64_t num_slots,
                            const float* channel_scales, void* cache_codes, float* cache_scales,
                            void* stream);

/*
 * qg_mx_quant -- OCP MXFP4 quantization of [rows][K] along K ([MX]; [L6]
 * section 2 micro-block scaling).  K must be a multiple of 32 ([L6]
 * section 3), else QG_ERR_GEOMETRY.
 *   src        [rows][K] of src_dtype (QG_BF16 or QG_F32).
 *   codes      uint8 [rows][K/2];  e8m0  uint8 [rows][K/32].
 */
qg_status qg_mx_quant(const void* src, qg_dtype src_dtype, int64_t rows, int64_t K,
                      void* codes, void* e8m0, void* stream);

typedef enum {
    QG_NORM_LAYER = 0,   /* (x - mean) / sqrt(var + eps) * gamma + beta */
    QG_NORM_RMS = 1      /* x / sqrt(mean(x^2) + eps) * gamma */
} qg_norm;

/*
 * qg_norm_quant -- fused LayerNorm / RMSNorm of each row followed by its
 * per-row dynamic quantization, written once ([SRV] section 4.4: the row's
 * statistics, the normalization and the quantization scale in one kernel,
 * codes and scale written once; RMSNorm + quantization as the same kind of
 * fusion).  The result equals the normalized rows passed to
 * qg_quantize_pack with group == K, or for QG_MXFP4 to qg_mx_quant (the
 * same fusion with the block-scaled format of [MX] section 2 eq. 3: one
 * E8M0 exponent per 32 elements instead of a row scale).
 *   norm       QG_NORM_LAYER or QG_NORM_RMS.
 *   fmt        QG_FP8_E4M3 | QG_INT8_SYM | QG_INT8_ASYM | QG_MXFP4.
 *   src        [rows][K] of src_dtype (QG_BF16 or QG_F32), row-major.
 *   gamma      fp32 [K]; beta fp32 [K] for QG_NORM_LAYER, NULL for
 *              QG_NORM_RMS.
 *   eps        >= 0 and finite.
 *   codes      [rows][K] (int8 / uint8 / E4M3 bytes); scales fp32 [rows];
 *              zeros fp32 [rows] for QG_INT8_ASYM, NULL otherwise.
 *              QG_MXFP4: codes uint8 [rows][K/2], scales = E8M0 uint8
 *              [rows][K/32] (the layout of qg_mx_quant), zeros NULL, K a
 *              multiple of 32.
 * Arithmetic (bit-exact reference): the row sums (of x and of (x - mean)^2,
 * or of x^2) are accumulated in fp64 and the variance is the biased one
 * (divide by K); mean and r = 1 / sqrt(var + eps) are rounded once to fp32;
 * then t = x - mean, u = t * r, y = u * gamma, y = y + beta, each one fp32
 * operation rounded to nearest even (no fused multiply-add); y is quantized
 * as by qg_quantize_pack (qg_mx_quant for QG_MXFP4).
 * Limits: K a multiple of 8, 8 <= K <= 16384 (QG_ERR_GEOMETRY when not a
 * multiple of 8, QG_ERR_UNSUPPORTED above 16384); rows <= 2^31 - 1.
 * Errors: QG_ERR_GEOMETRY, QG_ERR_FORMAT, QG_ERR_NULL, QG_ERR_ALIGN,
 * QG_ERR_UNSUPPORTED, QG_ERR_HIP.
 */
qg_status qg_norm_quant(qg_norm norm, qg_format fmt, const void* src, qg_dtype src_dtype,
                        const float* gamma, const float* beta, float eps, int64_t rows,
                        int64_t K, void* codes, void* scales, void* zeros, void* stream);

/*
 * qg_mx_gemm -- block-scaled MXFP4 product
 *   y[m][n] = bf16( sum_b 2^(ea[m][b] + eb[n][b] - 254) *
 *                   sum_{k in b} e2m1(a[m][k]) * e2m1(b[n][k]) )
 * on the gfx950 scaled matrix cores, fp32 accumulation ([MX]; [L6] sec. 2).
 *   a_codes uint8 [M][K/2], a_e8m0 uint8 [M][K/32]; b_codes uint8 [N][K/2],
 *   b_e8m0 uint8 [N][K/32] (the layout qg_mx_quant writes); y bf16 [M][N].
 * Errors: QG_ERR_GEOMETRY (M, N < 1; K < 32 or K % 32 != 0), QG_ERR_NULL,
 * QG_ERR_ALIGN, QG_ERR_UNSUPPORTED (an operand, padded by 256 rows, larger
 * than 2 GiB - 4 KiB), QG_ERR_HIP.
 */
qg_status qg_mx_gemm(const void* a_codes, const void* a_e8m0, int64_t M,
                     const void* b_codes, const void* b_e8m0, int64_t N, int64_t K,
                     void* y, void* stream);

/*
 * Roofline calibration (measurement only, not a step of the method): the two
 * roofs of [CH1] section 1.5 (attainable = min(bandwidth x intensity, peak))
 * as measured on this GPU, reported beside the published peaks.
 *
 * qg_calib_stream_read -- reads `bytes` of device memory once: workgroup c
 * reads the contiguous 64 KiB chunk c with 16-byte non-temporal loads, all
 * in flight at once, and writes the XOR of the chunk's 32-bit words to
 * sink[c].
 *   src        device memory, 16-byte aligned, `bytes` long.
 *   bytes      a positive multiple of 65536, at most 2^40.
 *   sink       uint32 [bytes / 65536], 4-byte aligned (owned by the caller).
 * Errors: QG_ERR_GEOMETRY, QG_ERR_NULL, QG_ERR_ALIGN, QG_ERR_HIP.
 *
 * qg_calib_mfma -- `waves` waves each issue `iters` x 8 back-to-back 32x32
 * matrix instructions (four independent accumulators, no memory traffic in
 * the loop) on pseudo-random finite operands whose mantissa bits change
 * every iteration; lane l of the grid writes the sum of its accumulators to
 * sink[l].  Work per launch: waves x iters x 8 x 2 x 32 x 32 x Kc operations
 * with Kc = 16 (QG_CALIB_BF16), 64 (QG_CALIB_FP8, QG_CALIB_FP4 on the scaled
 * f8f6f4 instruction with per-lane unit-range scales) or 32 (QG_CALIB_INT8).
 *   waves      a positive multiple of 4, at most 2^20; iters 1 .. 2^24.
 *   sink       fp32 [waves x 64], 4-byte aligned.
 * Errors: QG_ERR_FORMAT (kind), QG_ERR_GEOMETRY, QG_ERR_NULL, QG_ERR_ALIGN,
 * QG_ERR_HIP.
 */
typedef enum {
    QG_CALIB_BF16 = 0,
    QG_CALIB_FP8 = 1,
    QG_CALIB_FP4 = 2,
    QG_CALIB_INT8 = 3
} qg_calib_kind;

qg_status qg_calib_stream_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

qg_status qg_calib_mfma(qg_calib_kind kind, int64_t waves, int64_t iters, float* sink,
                        void* stream);

/*
 * Debug outputs (a localisation aid, not part of the method): the debug
 * library libqgemm_debug.so is the same source built with QG_DEBUG_FP32.  In
 * it, every kernel that rounds an output to bf16 (the GEMV, GEMM and SwiGLU
 * entry points) also stores the fp32 value it rounds, at the same index of
 * an fp32 buffer shaped like that output ([M][N], or [M][I] for SwiGLU), so
 * a parity failure can be told apart from the final rounding.
 *
 * qg_debug_fp32_output -- set (out != NULL) or clear (out == NULL) that
 * buffer for every later launch, process-wide (library state; not for
 * concurrent use).  The caller sizes the buffer for the next call's output.
 *   out        fp32, 4-byte aligned, or NULL.
 * Errors: QG_ERR_UNSUPPORTED in the product library, QG_ERR_ALIGN,
 * QG_ERR_HIP.
 *
 * qg_debug_build -- 1 in the debug library, 0 in the product library.
 */
qg_status qg_debug_fp32_output(float* out, void* stream);

int qg_debug_build(void);

/* Human-readable name of a status code (static storage). */
const char* qg_status_str(qg_status status);

/* Detail of the last error returned on the calling thread (static or
 * thread-local storage; empty string if none). */
const char* qg_last_error(void);

/* QG_ABI_VERSION of the built library. */
int qg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
