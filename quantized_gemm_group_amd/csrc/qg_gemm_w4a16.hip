// W4A16 prefill GEMM: Y[M][N] = X[M][K] (bf16) * dequant(W)^T with INT4
// weights in groups of 128 along K (《推理优化与量化算子深度技术调研》 section
// 1.3; 《第 6 课：量化源码走读》 section 2: the weights are dequantized inside
// the GEMM; section 3: the asymmetric zero-point cross term is kept).
//
// The matrix cores multiply exact integers: each nibble u becomes the bf16
// value 128 + u in registers (a byte permute and one bitop per pair of
// codes) and meets the bf16 activations in v_mfma_f32_32x32x16_bf16.  With
// c = 136 for symmetric codes (u = q + 8) and c = 128 + z for asymmetric ones
//     y = sum_g s_g * (acc_g - c_g * sum_x_g),
// where acc_g is the group's fp32 accumulator.  The two terms are kept apart:
//   * s_g * acc_g is one fused multiply-add per output and group;
//   * the cross term -sum_g (s_g c_g) sum_x_g is a rank-G product that the
//     fp32 matrix instruction v_mfma_f32_32x32x2_f32 adds straight into the
//     output accumulators, two groups per instruction, with the row sums
//     sum_x_g computed from the activation tile in LDS (bf16 dot products
//     against 1.0, each row's sum split over the four waves sharing it).
// Rounding dequantized weights to bf16 before the matrix cores is avoided on
// purpose: its error is of the size of the bf16 output rounding itself.
//
// The activations are the first MFMA operand and the codes the second, so
// lane (l % 32, l / 32) of a 32x32 tile accumulates D[m][n = l % 32]: one
// weight row per lane, hence one scale per lane and tile.
//
// Tiling: 512-thread workgroup (two waves per SIMD, so one wave's unpacking
// and scaling overlaps the other's matrix instructions), 128 (tokens) x 256
// (channels) output tile; one k-step = one group.  Each of the 8 waves owns
// 128 x 32 (4 x 1 tiles of 32x32): a wave unpacks only its own 32 weight
// rows' codes and uses each unpacked code for four MFMAs.  The operands
// travel HBM -> LDS with buffer loads that write LDS directly, into a ring of
// 3 stages: X (128 rows x 256 bytes, 16-byte chunks XOR-swizzled by row bits
// 0..3), the codes (256 rows x 64 bytes, swizzled by row bits 2..3) and the
// fp16 scales and zero points (one 2-byte load per row and group, or, for an
// even group count, one dword load per row for two groups).  The loads of
// k-step k + 2 go out after the barrier of k-step k; the compiler does not
// track loads that write LDS, so the waits are explicit.  Within a group,
// lane half h and MFMA j cover k = 64 h + 8 j .. + 7 in natural order, so a
// lane's codes of the group are 32 contiguous bytes and its X pieces 128.
// Tiles are ordered XCD by XCD (contiguous ranges in column groups of 4 tile
// rows), and a last, mostly empty wave of tiles runs in 32-token quarters.
//
// SwiGLU variant (《推理优化与量化算子深度技术调研》 section 4.6: the gate and
// up projections as one GEMM over [W_gate; W_up], SiLU(gate) * up formed in
// registers and written once): the weight rows are the 2I rows of the
// concatenation and the output is H[M][I].  A workgroup covers 128
// intermediate channels: wave w's 32 weight rows are gate rows n0 + 16 w ..
// + 15 and the up rows I + n0 + 16 w .. + 15, so lane l32 < 16 and lane
// l32 + 16 hold gate[n] and up[n] of the same channel and token rows, and one
// lane exchange per value pairs them in the epilogue.

#include <atomic>

#include "qg_gemm_common.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int kThreads = 512;
constexpr int XROW = BK * 2;              // bytes of one X row per k-step
constexpr int WROW = BK / 2;              // bytes of one code row per k-step
constexpr int kStages = 3;
constexpr int kXBytes = BM * XROW;        // 32 KiB
constexpr int kWBytes = BN * WROW;        // 16 KiB
constexpr int kSBytes = BN * 4;           // one dword per row (zero-extended fp16)
constexpr int kStageBytes = kXBytes + kWBytes + 2 * kSBytes;
constexpr int kSumBytes = BM * 16;        // four partial sums per X row
constexpr int kSumBufs = 3;
constexpr int kLdsBytes = kStages * kStageBytes + kSumBufs * kSumBytes;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

// Codes of one 32-bit word (elements 8 w .. 8 w + 7, element i in bits
// 4 i .. 4 i + 3) as four bf16 pairs (128 + u_{2d}, 128 + u_{2d+1}): byte d
// of w and byte d of w >> 4 are moved to the two halves, the mask keeps their
// low nibbles and the xor adds the bf16 exponent of 128.  For symmetric
// (two's-complement) codes the xor also flips bit 3 of each nibble, which
// gives u = q + 8.  Mask and constant arrive as kernel arguments so that the
// compiler selects one v_bitop3 per pair.
__device__ __forceinline__ u32x4 unpack_word(uint32_t w, uint32_t mask, uint32_t c) {
  const uint32_t t = w >> 4;
  u32x4 r;
  r[0] = (__builtin_amdgcn_perm(t, w, 0x0C040C00u) & mask) ^ c;
  r[1] = (__builtin_amdgcn_perm(t, w, 0x0C050C01u) & mask) ^ c;
  r[2] = (__builtin_amdgcn_perm(t, w, 0x0C060C02u) & mask) ^ c;
  r[3] = (__builtin_amdgcn_perm(t, w, 0x0C070C03u) & mask) ^ c;
  return r;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Byte offsets within a stage: X chunk c (16 bytes) of row r, code chunk c of
// row r.
__device__ __forceinline__ int x_off(int r, int c) { return r * XROW + ((c ^ (r & 15)) << 4); }
__device__ __forceinline__ int w_off(int r, int c) {
  return kXBytes + r * WROW + ((c ^ ((r >> 2) & 3)) << 4);
}

template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int V>
struct Parity {
  static constexpr int value = V;
};

// SUB = 4: each workgroup covers one 32-token quarter of a 128 x 256 tile
// (the tiles of a last, partly filled wave of workgroups, spread over every
// CU); the four quarters of a tile run on one XCD so its codes come from
// that XCD's L2.  lin0: linear index of the launch's first tile.
// PAIRS (an even number of groups G): the scales (and zero points) of two
// groups, one dword per row, come in one load at every even k-step, into
// slot (g / 2) % 3 of the three stages' scale areas, instead of one 2-byte
// load per group: half the scale loads and half their cache-line requests.
template <bool ASYM, bool SWIGLU, int SUB = 1, bool PAIRS = false>
__global__ __launch_bounds__(kThreads) void gemm_w4a16_kernel(
    const uint16_t* __restrict__ X, int M, const uint32_t* __restrict__ Wc,
    const uint16_t* __restrict__ S, const uint16_t* __restrict__ Z, int N, int K,
    uint16_t* __restrict__ Y, uint32_t mask, uint32_t cmag, int lin0) {
  static_assert(SUB == 1 || SUB == 4, "whole tiles or quarters");
  constexpr int BMS = BM / SUB;                    // token rows of the workgroup
  constexpr int kXL = BMS / 32;                    // X loads (4 rows each) per wave and k-step
  constexpr int kGroupLoads = kXL + 2 + 1;         // loads per wave per k-step
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLdsBytes];
  uint8_t* const sums = smem + kStages * kStageBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lh = lane >> 5;
  // Wave tile: 128 tokens x 32 weight rows (4 x 1 tiles of 32x32), so every
  // wave unpacks codes no other wave unpacks and uses each unpacked code for
  // four MFMAs.  SWIGLU: the 32 rows are 16 gate and the same 16 up channels.
  constexpr int MT = BMS / 32, NT = 1;
  const int mrow0 = 0;                             // first X row of the wave tile
  const int nrow0 = 32 * wave;                     // first LDS code row

  // SWIGLU: N = 2 I weight rows, 128 intermediate channels per tile
  const int NI = SWIGLU ? N / 2 : N;                 // output columns
  const int TN = SWIGLU ? BN / 2 : BN;               // output columns per tile
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (NI + TN - 1) / TN;
  int tm, tn, lin = lin0 + (int)blockIdx.x, quarter = 0;
  if constexpr (SUB == 1) {
    // workgroups go round-robin over the 8 XCDs: XCD x takes the contiguous
    // tile range x * nb / 8 .., walked in column groups of 4 tile rows, so
    // the tiles running together on one XCD share code columns and X rows
    // in its L2 (Qwen2.5-72B up 1011 -> 987 us, down 973 -> 954 us against
    // round-robin tiles in groups of 8 rows; outputs bit-identical)
    const int nb = (int)gridDim.x;
    if (nb % 8 == 0) lin = lin0 + ((int)blockIdx.x % 8) * (nb / 8) + (int)blockIdx.x / 8;
  } else {
    // unit u = SUB * (tile - lin0) + quarter; XCD x (blocks x, x + 8, ...)
    // takes a contiguous range of units when the count divides by 8
    const int units = (int)gridDim.x;
    const int u = units % 8 == 0 ? ((int)blockIdx.x % 8) * (units / 8) + (int)blockIdx.x / 8
                                 : (int)blockIdx.x;
    lin = lin0 + u / SUB;
    quarter = u % SUB;
  }
  tile_coords(lin, tiles_m, tiles_n, 4, &tm, &tn);
  const int m0 = tm * BM + quarter * BMS, n0 = tn * TN;
  // weight row of LDS tile row r (0..255); SWIGLU: rows 32 w .. 32 w + 15
  // are gate channels n0 + 16 w .., rows 32 w + 16 .. their up channels
  auto wrow = [&](int r) {
    return SWIGLU ? ((r >> 4) & 1) * NI + n0 + 16 * (r >> 5) + (r & 15) : n0 + r;
  };
  const int G = K / BK;

  // rows past M (N) fall outside the buffers' byte ranges and read as zero
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X, (int64_t)M * K * 2);
  const __amdgpu_buffer_rsrc_t rwc = make_rsrc(Wc, (int64_t)N * K / 2);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(S, (int64_t)N * G * 2);
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(Z, ASYM ? (int64_t)N * G * 2 : 0);

  // Load map.  X: wave w brings rows 16 w .. 16 w + 15 in 4 loads of 4 rows x
  // 256 bytes; lane i -> row 16 w + 4 q + i / 16, LDS position i % 16 holding
  // chunk (i % 16) ^ (row & 15).  Codes: 2 loads of 16 rows x 64 bytes; lane
  // i -> row 32 w + 16 q + i / 4, position i % 4 holding chunk
  // (i % 4) ^ ((row >> 2) & 3).  Scales: waves 0..3 bring s of rows
  // 64 (w % 4) + i, waves 4..7 the zero points (symmetric: a load of nothing,
  // which keeps the counts equal).
  uint32_t vx[4], vw[2];
#pragma unroll
  for (int q = 0; q < kXL; ++q) {
    const int r = 4 * kXL * wave + 4 * q + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    vx[q] = (uint32_t)(m0 + r) * (uint32_t)(K * 2) + c * 16;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int r = 32 * wave + 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    vw[q] = (uint32_t)wrow(r) * (uint32_t)(K / 2) + c * 16;
  }
  const int srow = 64 * (wave & 3) + lane;
  const bool zwave = wave >= 4;
  const uint32_t vs = (zwave && !ASYM) ? kOutOfRange : (uint32_t)wrow(srow) * (uint32_t)(G * 2);

  // Loads of group g into stage g % 3.  Past the last group the last group is
  // loaded again (into a stage nobody reads), so every k-step issues the same
  // number of loads and the wait counts stay uniform.
  auto issue = [&](int g, int stage) {
    uint8_t* st = smem + stage * kStageBytes;
    const int gl = g < G ? g : G - 1;
#pragma unroll
    for (int q = 0; q < kXL; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (lds_void*)(st + (4 * kXL * wave + 4 * q) * XROW),
                                               16, vx[q], gl * XROW, 0, 0);
#pragma unroll
    for (int q = 0; q < 2; ++q)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rwc, (lds_void*)(st + kXBytes + (32 * wave + 16 * q) * WROW), 16, vw[q], gl * WROW, 0, 0);
    if constexpr (PAIRS) {
      // groups g, g + 1 (g even; past the end the last pair again, into a
      // slot nobody reads) into slot (g / 2) % 3; odd g: no scale load
      if ((g & 1) == 0) {
        const int gp = g < G ? g : G - 2;
        uint8_t* slot = smem + ((g >> 1) % 3) * kStageBytes + kXBytes + kWBytes;
        lds_void* sd = (lds_void*)(slot + (zwave ? kSBytes : 0) + 256 * (wave & 3));
        if (zwave)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, sd, 4, vs, gp * 2, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, sd, 4, vs, gp * 2, 0, 0);
      }
    } else {
      lds_void* sd = (lds_void*)(st + kXBytes + kWBytes + (zwave ? kSBytes : 0) + 256 * (wave & 3));
      if (zwave)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, sd, 2, vs, gl * 2, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, sd, 2, vs, gl * 2, 0, 0);
    }
  };

  const f32x16 zero16 = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                         0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // (bounds fixed at the largest MT: bounds that depend on the template
  // arguments left the host compilation pass without the launch stub)
  static_assert(MT <= 4 && NT == 1, "array bounds below");
  f32x16 yacc[4][1];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) yacc[mt][nt] = zero16;
  // s_g * c_g of this lane's channels for the last two groups, by parity
  float scp[2][NT];
#pragma unroll
  for (int p2 = 0; p2 < 2; ++p2)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) scp[p2][nt] = 0.f;
  const bf16x2_t ones2 = __builtin_bit_cast(bf16x2_t, 0x3F803F80u);

  // Cross term of groups g0 (even) and g0 + 1: lane half h supplies group
  // g0 + h (sum_x of the lane's row as the first operand, -(s c) of its
  // channel as the second); without `pair` group g0 + 1 does not exist.
  auto cross = [&](int g0, bool pair) {
    const uint8_t* sb = sums + ((g0 + lh) % kSumBufs) * kSumBytes;
    float sx[4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 p = *reinterpret_cast<const u32x4*>(sb + (mrow0 + 32 * mt + l32) * 16);
      sx[mt] = (__uint_as_float(p[0]) + __uint_as_float(p[1])) +
               (__uint_as_float(p[2]) + __uint_as_float(p[3]));
      if (!pair && lh) sx[mt] = 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float b = -(lh ? scp[1][nt] : scp[0][nt]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        yacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x2f32(sx[mt], b, yacc[mt][nt], 0, 0, 0);
    }
  };

  // One k-step over group g (P = g % 2).  SC = g % 3 when known at compile
  // time (the main loop is unrolled by 6), else -1: with a constant stage
  // every LDS address is a per-lane offset plus an immediate.
  auto step = [&](int g, auto parity, auto stage_c) {
    constexpr int P = decltype(parity)::value;
    constexpr int SC = decltype(stage_c)::value;
    const int sg = SC >= 0 ? SC : g % kStages;        // stage of g (also its row-sum buffer)
    // group g has landed for every wave; stage (g - 1) % 3 is free and the
    // row sums of the groups before g are in LDS
    // PAIRS: step g - 1 issued its scale load iff it was even, i.e. iff P = 1
    wait_vm_barrier<PAIRS ? kXL + 2 + P : kGroupLoads>();
    issue(g + 2, SC >= 0 ? (SC + 2) % kStages : (g + 2) % kStages);
    const uint8_t* st = smem + sg * kStageBytes;
    if (P == 0 && g >= 2) cross(g - 2, true);

    // this wave's share of the row sums of group g: rows 16 w .. 16 w + 15,
    // four lanes a row, each one of four partial sums of 32 k (a quarter
    // tile: the first two waves)
    if (SUB == 1 || wave < BMS / 16) {
      const int r = 16 * wave + (lane >> 2);
      const int part = lane & 3;
      const int c0 = 4 * part;
      float ps = 0.f;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(st + x_off(r, c0 + h));
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          // (a bit cast of a vector element itself would read element 0)
          const uint32_t e = v[d];
          ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, e), ones2, ps, false);
        }
      }
      *reinterpret_cast<float*>(sums + sg * kSumBytes + r * 16 + part * 4) = ps;
    }

    // codes: 32 contiguous bytes of the lane's row (words 8 lh .. 8 lh + 7)
    u32x4 cw[NT][2];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = nrow0 + nt * 32 + l32;
      cw[nt][0] = *reinterpret_cast<const u32x4*>(st + w_off(r, 2 * lh));
      cw[nt][1] = *reinterpret_cast<const u32x4*>(st + w_off(r, 2 * lh + 1));
    }
    float sv[NT];
    // PAIRS: slot (g / 2) % 3, known at compile time inside the unrolled
    // loop (position i of the six steps: i % 2 = P, i % 3 = SC); the dword
    // holds group g - P in its low half and group g - P + 1 in its high half
    constexpr int kSlot = SC >= 0 ? ((3 * P + 4 * SC) % 6) / 2 : -1;
    const int slot = kSlot >= 0 ? kSlot : (g >> 1) % 3;
    const uint32_t* sl = reinterpret_cast<const uint32_t*>(
        (PAIRS ? smem + slot * kStageBytes : st) + kXBytes + kWBytes);
    constexpr int kHalf = PAIRS ? 16 * P : 0;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int r = nrow0 + nt * 32 + l32;
      sv[nt] = f16_bits_to_f32((uint16_t)(sl[r] >> kHalf));
      const float c = ASYM ? 128.f + f16_bits_to_f32((uint16_t)(sl[BN + r] >> kHalf)) : 136.f;
      scp[P][nt] = sv[nt] * c;
    }

    f32x16 gacc[4][1];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16x8 a[4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = mrow0 + mt * 32 + l32;
        a[mt] = as_bf16x8(*reinterpret_cast<const u32x4*>(st + x_off(r, 8 * lh + j)));
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const bf16x8 b = as_bf16x8(unpack_word(cw[nt][j >> 2][j & 3], mask, cmag));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          gacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mt], b, j ? gacc[mt][nt] : zero16,
                                                                 0, 0, 0);
      }
    }
    // y += s * acc: lane (l32, lh) register r holds m = 8 (r / 4) + 4 lh + r % 4
    // of its m-tile and n = l32 of its n-tile
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          yacc[mt][nt][r] = __builtin_fmaf(sv[nt], gacc[mt][nt][r], yacc[mt][nt][r]);
  };

  static_assert(kSumBufs == kStages, "row-sum buffers rotate with the stages");
  issue(0, 0);
  issue(1, 1);
  int g = 0;
  for (; g + 5 < G; g += 6) {
    step(g, Parity<0>{}, Parity<0>{});
    step(g + 1, Parity<1>{}, Parity<1>{});
    step(g + 2, Parity<0>{}, Parity<2>{});
    step(g + 3, Parity<1>{}, Parity<0>{});
    step(g + 4, Parity<0>{}, Parity<1>{});
    step(g + 5, Parity<1>{}, Parity<2>{});
  }
  for (; g + 1 < G; g += 2) {
    step(g, Parity<0>{}, Parity<-1>{});
    step(g + 1, Parity<1>{}, Parity<-1>{});
  }
  if (g < G) step(g, Parity<0>{}, Parity<-1>{});
  // Every wave's trailing loads (a repeat of the last group) have landed and
  // every wave is past its last k-step: the row sums of the last groups are
  // in LDS and the operand stages are free for the epilogue.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // cross terms not yet added: groups (G - 2, G - 1) for even G, G - 1 alone
  // for odd G
  if (G & 1)
    cross(G - 1, false);
  else
    cross(G - 2, true);

  // Epilogue through LDS (the operand stages, not the row-sum buffers): each
  // wave writes its bf16 values at [m][n] with a 528-byte row pitch, then
  // every thread moves 16-byte pieces of whole output rows to memory.  SWIGLU
  // writes
  // h = SiLU(gate) * up = gate / (1 + exp(-gate)) * up (fp32, one bf16
  // rounding) for its 128 channels, the plain GEMM its 256.
  constexpr int kPitch = 528;
  uint16_t* const so = reinterpret_cast<uint16_t*>(smem);
  if constexpr (SWIGLU) {
    // lane l32 < 16 holds gate channel n0 + 16 w + l32 and lane l32 + 16 the
    // same channel's up value for the same token rows
    const int nl = 16 * wave + (l32 & 15);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ml = mrow0 + mt * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const float g = yacc[mt][0][r];
        const float u = __shfl_xor(g, 16, 64);
        if (l32 < 16) {
          const float hv = g / (1.f + __expf(-g)) * u;
          if (m0 + ml < M && n0 + nl < NI) QG_DEBUG_STORE((int64_t)(m0 + ml) * NI + n0 + nl, hv);
          so[ml * (kPitch / 2) + nl] = (uint16_t)cvt_bf16x2(hv, 0.f);
        }
      }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int nl = nrow0 + nt * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ml = mrow0 + mt * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (m0 + ml < M && n0 + nl < NI)
            QG_DEBUG_STORE((int64_t)(m0 + ml) * NI + n0 + nl, yacc[mt][nt][r]);
          so[ml * (kPitch / 2) + nl] = (uint16_t)cvt_bf16x2(yacc[mt][nt][r], 0.f);
        }
      }
  }
  __syncthreads();
  constexpr int kChunks = (SWIGLU ? BN / 2 : BN) / 8;   // 16-byte pieces per row
  const bool vec_ok = (NI & 7) == 0;
#pragma unroll 4
  for (int c = tid; c < BMS * kChunks; c += kThreads) {
    const int ml = c / kChunks, cn = c - ml * kChunks;
    const int m = m0 + ml, n = n0 + cn * 8;
    if (m >= M || n >= NI) continue;
    const u32x4 o = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(so) +
                                                    ml * kPitch + cn * 16);
    uint16_t* py = Y + (int64_t)m * NI + n;
    if (vec_ok && n + 7 < NI) {
      // nontemporal: the output is not read again by this kernel
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(py));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (n + j < NI) py[j] = (uint16_t)(o[j >> 1] >> (16 * (j & 1)));
    }
  }
}

// Compute units of the current device (cached per device id; host threads
// may race to fill an entry, all with the same value).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Whole tiles [0, full), then tiles [full, tiles) as quarters.
template <bool ASYM, bool SWIGLU, bool PAIRS>
void launch_tiles(const void* x, int64_t M, const void* wcodes, const void* wscales,
                  const void* wzeros, int64_t N, int64_t K, void* y, int full, int tiles,
                  uint32_t cmag, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_w4a16_kernel<ASYM, SWIGLU, 1, PAIRS>), dim3(full), dim3(kThreads), 0,
                     stream, (const uint16_t*)x, (int)M, (const uint32_t*)wcodes,
                     (const uint16_t*)wscales, (const uint16_t*)wzeros, (int)N, (int)K,
                     (uint16_t*)y, 0x000F000Fu, cmag, 0);
  if (full < tiles)
    hipLaunchKernelGGL((gemm_w4a16_kernel<ASYM, SWIGLU, 4, PAIRS>), dim3(4 * (tiles - full)),
                       dim3(kThreads), 0, stream, (const uint16_t*)x, (int)M,
                       (const uint32_t*)wcodes, (const uint16_t*)wscales,
                       (const uint16_t*)wzeros, (int)N, (int)K, (uint16_t*)y, 0x000F000Fu, cmag,
                       full);
}

// One workgroup per CU at a time (the LDS holds one), so the tiles run in
// waves of `cus`.  When the last wave would fill at most a quarter of the
// CUs, its tiles go to a second launch in 32-token quarters, four per tile
// (each quarter unpacks the tile's codes again for a quarter of the matrix
// work, but all CUs take part).  Qwen2.5-72B up projection (1856 tiles, 7.25
// waves): 1055 -> 1034 us, the SwiGLU gate+up 1086 -> 1056 us (medians of
// three A/B pairs on one box); outputs bit-identical.
template <bool ASYM, bool SWIGLU>
void launch_t(const void* x, int64_t M, const void* wcodes, const void* wscales,
              const void* wzeros, int64_t N, int64_t K, void* y, hipStream_t stream) {
  const int64_t tn = SWIGLU ? (N / 2 + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  const int tiles = (int)(((M + BM - 1) / BM) * tn);
  const int cus = device_cus();
  const int rest = cus > 0 ? tiles % cus : 0;
  const int full = (rest > 0 && tiles > cus && 4 * rest <= cus) ? tiles - rest : tiles;
  const uint32_t cmag = ASYM ? 0x43004300u : 0x43084308u;
  if ((K / BK) % 2 == 0)
    launch_tiles<ASYM, SWIGLU, true>(x, M, wcodes, wscales, wzeros, N, K, y, full, tiles, cmag,
                                     stream);
  else
    launch_tiles<ASYM, SWIGLU, false>(x, M, wcodes, wscales, wzeros, N, K, y, full, tiles, cmag,
                                      stream);
}

}  // namespace

QG_DEBUG_TU_SETTER(debug_set_w4a16)

hipError_t launch_gemm_w4a16(bool asym, const void* x, int64_t M, const void* wcodes,
                             const void* wscales, const void* wzeros, int64_t N, int64_t K,
                             void* y, hipStream_t stream) {
  if (asym)
    launch_t<true, false>(x, M, wcodes, wscales, wzeros, N, K, y, stream);
  else
    launch_t<false, false>(x, M, wcodes, wscales, wzeros, N, K, y, stream);
  return hipGetLastError();
}

hipError_t launch_gemm_w4a16_swiglu(bool asym, const void* x, int64_t M, const void* wcodes,
                                    const void* wscales, const void* wzeros, int64_t N2,
                                    int64_t K, void* h, hipStream_t stream) {
  if (asym)
    launch_t<true, true>(x, M, wcodes, wscales, wzeros, N2, K, h, stream);
  else
    launch_t<false, true>(x, M, wcodes, wscales, wzeros, N2, K, h, stream);
  return hipGetLastError();
}

}  // namespace qg
