// FP8 E4M3 W8A8 GEMM and MXFP4 block-scaled GEMM on the gfx950 scaled
// matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// FP8 (《第 6 课：量化源码走读》 section 2 and figure 6-2): the matrix cores
// multiply the E4M3 codes exactly and accumulate in fp32; the epilogue
// rescales by s_x[m] * s_w[n] (per-token activation scale, per-channel weight
// scale) and rounds once to bf16.  The MFMA's own block scales are off: the
// unscaled form of the instruction, which multiplies as block scales of 2^0
// would.
//
// MXFP4 (《大模型量化推理引擎全景大复盘》 section 2 eq. 3; 《第 6 课：量化源码走读》
// section 2): each lane of the MFMA holds 32 E2M1 codes of one row that form
// exactly one 32-element block, and passes that block's E8M0 byte as its
// scale, so 2^(ea + eb) is applied inside the matrix core and the epilogue
// only rounds.
//
// Tiling: a workgroup owns a 256x256 output tile.  MXFP4 (and FP8 with a
// K tail): 8 waves of 128 (tokens) x 64 (channels) each (2x4 tiles of
// v_mfma_scale_f32_32x32x64_f8f6f4, 128 fp32 accumulators per lane), two
// waves per SIMD so that one wave's fragment reads and barrier waits hide
// behind the other's matrix work.  FP8 with whole k-steps: 4 waves of 128 x
// 128 (4x4 tiles, 256 accumulators per lane in AGPRs), one per SIMD: each
// A fragment read from LDS feeds four matrix instructions instead of two,
// which takes a third off the LDS reads per k-step.
//
// Operand pipeline: a k-step covers 64 bytes of every operand row (64 FP8 or
// 128 FP4 codes).  Operand tiles go from HBM straight into LDS with buffer
// loads that write LDS (no VGPR round trip), into a ring of 4 stages kept
// as 2 double stages: the pair of k-steps (2 p, 2 p + 1) is one 128-byte
// row per operand row, so every load covers 8 rows' whole cache lines.  The
// loads of the pair (k + 3, k + 4) go out together at odd k.  One barrier
// per k-step: it certifies that stage k + 1 has landed and that every wave
// has finished reading the stages of k - 1 and k (whose fragments are
// already in registers), which may then be refilled.  During k-step k
// the matrix cores work on fragments already in registers while the
// fragments of k-step k + 1 are read from LDS.  The compiler does not track
// the LDS writes of these loads, so the waits for them are explicit.
// Within a 128-byte row the eight 16-byte chunks are stored XOR-swizzled by
// bits 1..3 of the row, so the 16 rows read by 16 lanes cover all banks.
// Workgroups are dispatched round-robin over the 8 XCDs; each XCD is given a
// contiguous range of tiles walked in column groups, so concurrently running
// workgroups of one XCD share operand panels in its L2.

#include <type_traits>

#include "qg_gemm_common.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 256, BN = 256;   // workgroup tile
constexpr int BK = 64;              // bytes of each operand row per k-step
constexpr int kStages = 4;
// Two wave layouts of the 256x256 tile: 8 waves of 128 (tokens) x 64
// (channels), two per SIMD, or (W4) 4 waves of 128 x 128, one per SIMD,
// with their 256 accumulators in AGPRs: each fragment read from LDS then
// feeds twice the matrix instructions.
template <bool W4> struct Layout {
  static constexpr int kWaves = W4 ? 4 : 8;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kRW = 256 / kWaves;        // tile rows each wave loads per operand
  static constexpr int kNP = kRW / 8;             // 1 KiB operand pieces per wave and pair
  static constexpr int NT = W4 ? 4 : 2;           // 32-channel W tiles per wave
  static constexpr int kWN = 32 * NT;             // channels per wave
  static constexpr int kEpiPitch = kWN * 2 + 16;  // bf16 staging row pitch (bytes)
  static constexpr int kEpiBytes = kWaves * 128 * kEpiPitch;
  static constexpr int kExpPieces = 512 / 16 / kWaves;   // 16-row exponent chunks per wave
};
constexpr int kOpBytes = BM * BK;   // one operand, one stage: 16 KiB
constexpr int kStageBytes = 2 * kOpBytes;
// The ring holds pairs of k-steps (even, odd) as double stages: each operand
// row's 128 bytes of the pair form one row of 8 16-byte chunks, chunk c of
// row r stored at position c ^ ((r >> 1) & 7).
constexpr int kPRow = 2 * BK;             // 128 bytes per row and pair
constexpr int kDOpBytes = BM * kPRow;     // one operand, one pair: 32 KiB
constexpr int kDStageBytes = 2 * kDOpBytes;
// epilogue: each wave's 128 (m) x 64 (n) (W4: 128 x 128) bf16 piece with a
// 144- (272-) byte row pitch (8-byte LDS writes of 32 rows spread over the
// banks, 16-byte aligned reads)

// Tile of workgroup `bid`: XCD-contiguous ranges (when the tile count divides
// evenly over the XCDs), then column groups of 4 tile rows.
__device__ __forceinline__ void xcd_tile(int bid, int tiles_m, int tiles_n, int* tm, int* tn) {
  constexpr int kXcd = 8;
  const int tiles = tiles_m * tiles_n;
  int lin = bid;
  if (tiles % kXcd == 0) lin = (bid % kXcd) * (tiles / kXcd) + bid / kXcd;
  tile_coords(lin, tiles_m, tiles_n, 4, tm, tn);
}


template <bool MX, int NT> struct Frags;
template <int NT> struct Frags<false, NT> {
  i32x8 a[4], w[NT];                      // [A tile], [W tile]: 32 codes each
};
template <int NT> struct Frags<true, NT> {
  i32x4 a[2][4], w[2][NT];                // [sub-step][tile]: 32 codes each
  uint32_t as[4], ws[NT];                 // exponent dword of each row, >> 8 lh
};

// Wait until at most N vector-memory loads of this wave are outstanding and
// its LDS operations are done, then meet the other waves.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// The epilogue's staging pieces are private to their wave (each wave reads
// back only rows it wrote), so between its LDS writes and reads a wave only
// waits for its own LDS operations, which complete in order; no barrier.
// (Against a workgroup barrier there: MXFP4 129.9 -> 128.9 us, FP8 unchanged,
// outputs bit-identical.)
__device__ __forceinline__ void wait_own_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// SALIGN (MX only): every row's exponents of a k-step are one aligned dword
// (K a multiple of 128); otherwise its 4 bytes are loaded one by one.
// KFULL: K fills whole k-steps, so no load needs a K-tail check (loads past
// the last k-step fill stages that are never read).
// SWIGLU (FP8 only; 《推理优化与量化算子深度技术调研》 section 4.6, the W8A8 GEMM
// with dequantization and activation fused): W is the [N][K] concatenation
// [W_gate; W_up] (N = 2I) and a workgroup's 256 weight rows are 128 gate
// channels and the same 128 up channels: tile rows 32 q .. 32 q + 31 are the
// gate (q even) or up (q odd) rows of channels c0 + 32 (q / 2) ..; so the W
// tiles u = 2 p and u = 2 p + 1 of a wave hold gate and up of the same 32
// channels and each lane forms h = SiLU(s_x s_g g) * (s_x s_u u) of its own
// accumulators.  Y is then h [M][I].
template <bool MX, bool SALIGN, bool KFULL, bool SWIGLU = false, bool W4 = false>
__global__ __launch_bounds__(W4 ? 256 : 512) void gemm_f8f4_kernel(const uint8_t* __restrict__ A,
                                                             const void* __restrict__ a_aux, int M,
                                                             const uint8_t* __restrict__ W,
                                                             const void* __restrict__ w_aux, int N,
                                                             int K, uint16_t* __restrict__ Y) {
  // Exponent staging.  Grouped (SALIGN): the dwords of 4 k-steps (a group)
  // of all 512 tile rows in one of 3 slots, see issue_exp.  Otherwise per
  // row and k-step 4 bytes loaded one by one beside the operands, each
  // landing zero-extended in a dword of its own, in every ring stage.
  using LY = Layout<W4>;
  static_assert(LY::kThreads == (W4 ? 256 : 512), "launch bound of the layout");
  constexpr int kWaves = LY::kWaves, kRW = LY::kRW, kNP = LY::kNP, NT = LY::NT, kWN = LY::kWN;
  constexpr int kEpiPitch = LY::kEpiPitch, kEpiBytes = LY::kEpiBytes;
  static_assert(!W4 || KFULL, "the 4-wave layout takes whole k-steps");
  static_assert(!W4 || !MX || SALIGN, "the 4-wave layout takes grouped exponents");
  constexpr bool kGrouped = MX && SALIGN;
  constexpr int kSWords = (MX && !SALIGN) ? 4 : 0;
  constexpr int kScaleStage = (BM + BN) * 4 * kSWords;
  constexpr int kChunk = 320;                   // 16 rows x 4 k-steps + 64 bytes of skew
  constexpr int kExpSlot = kGrouped ? (BM + BN) / 16 * kChunk : 0;
  constexpr int kRing = kStages * (kStageBytes + kScaleStage) + 3 * kExpSlot;
  // FP8: the tile's s_x (256 rows) and s_w (256 channels) above the ring,
  // loaded with the first operands and read back before the epilogue
  constexpr int kEpiScales = MX ? 0 : 2 * 1024;
  static_assert(MX || kRing + kEpiScales <= kEpiBytes, "epilogue scales within the staging area");
  constexpr int kLds = kRing + kEpiScales > kEpiBytes ? kRing + kEpiScales : kEpiBytes;
  // loads per wave per k-step beside the grouped exponent loads: kNP operand
  // blocks of 1 KiB + per-k-step exponent loads
  constexpr int kGroup = kNP + kSWords;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  uint8_t* const sscale = smem + kStages * kStageBytes;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;     // A rows 128 wm.., W rows kWN wn..
  const int l32 = lane & 31, lh = lane >> 5;

  static_assert(!(SWIGLU && MX), "the SwiGLU epilogue is for the FP8 product");
  const int I = N / 2;                          // SwiGLU: channels of h
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = SWIGLU ? (I + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  int tm, tn;
  xcd_tile(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int c0 = tn * (BN / 2);                 // SwiGLU: first channel of the tile

  const int kbytes = MX ? K / 2 : K;           // bytes per operand row
  const int nk = (kbytes + BK - 1) / BK;
  const int kblocks = K / 32;                  // MX exponents per row
  // rows past M (N) fall outside the buffer's byte range and read as zero
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (int64_t)M * kbytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W, (int64_t)N * kbytes);

  // Operand loads, one pair of k-steps at a time: wave w brings rows kRW w
  // .. kRW w + kRW - 1 (kRW = 32, or 64 in the 4-wave layout) of both operand
  // tiles in kNP loads each (piece j: rows kRW w + 8 j .. + 7, whole 128-byte
  // lines); lane i brings row kRW w + 8 j + i / 8,
  // chunk (i & 7) ^ ((row >> 1) & 7) = (i & 7) ^ (4 (j & 1) + (i >> 4)),
  // which lands at LDS position i of the piece.  Piece j's row offset goes
  // into the scalar offset, so two voffsets per operand (by j & 1) suffice.
  // W4: a wave's 64 rows are two runs of 32 (h = j / 4), each addressed from
  // its own base (the SwiGLU row map is not linear across them).
  // Local arrays are sized for the larger layout (the 8-wave one leaves the
  // rest untouched): bounds that depend on the template arguments left the
  // host compilation pass without the kernel's launch stub.
  static_assert(kRW <= 64 && NT <= 4, "array bounds below");
  int pchunk[2];
  uint32_t voa[4], vow[4];                        // [2 h + jp]
#pragma unroll
  for (int h = 0; h < kRW / 32; ++h)
#pragma unroll
    for (int jp = 0; jp < 2; ++jp) {
      pchunk[jp] = (lane & 7) ^ (4 * jp + (lane >> 4));
      const int r = kRW * wave + 32 * h + (lane >> 3);
      // SwiGLU: tile rows 32 q .. 32 q + 31 are the gate (q even) or up (q
      // odd) rows of channels c0 + 32 (q / 2) + 0..31; gate rows past I read
      // up rows and up rows past N read zero, both for channels that are
      // never stored
      const int q = r >> 5;
      const int wrow = SWIGLU ? (q & 1) * I + c0 + 32 * (q >> 1) + (r & 31) : n0 + r;
      voa[2 * h + jp] = (uint32_t)(m0 + r) * kbytes + pchunk[jp] * 16;
      vow[2 * h + jp] = (uint32_t)wrow * kbytes + pchunk[jp] * 16;
    }
  // Exponent loads (MX): wave w brings the exponents of tile rows 2 kRW w ..
  // (rows 0..255 of A, then 256..511 of W).  Grouped: lane l reads dword
  // l / 16 (k-step) of row l % 16 of a 16-row chunk, so one load touches 16
  // rows' cache lines instead of 64; otherwise one load per k-step and byte
  // with lane l on row l.
  __amdgpu_buffer_rsrc_t rsx = make_rsrc(a_aux, 0);
  uint32_t vos = 0;
  if constexpr (MX) {
    const bool wop = wave >= kWaves / 2;
    rsx = make_rsrc(wop ? w_aux : a_aux, (int64_t)(wop ? N : M) * kblocks);
    const int grow = (wop ? n0 : m0) + 2 * kRW * (wave % (kWaves / 2)) +
                     (kGrouped ? (lane & 15) : lane);
    vos = (uint32_t)grow * kblocks + (kGrouped ? 4 * (lane >> 4) : 0);
  }

  // One load of the pair group (the pair holding k-step k): d < 4 -> operand
  // piece j = 2 (d >> 1) + (k & 1) of A (d even) or W (d odd), so the 8
  // operand loads of the two k-steps cover both operands' 4 pieces; then the
  // per-k-step exponent loads (MX, K not a multiple of 128).
  auto issue_piece = [&](int k, int d) {
    if (d < kNP) {
      const int pk = k >> 1;
      uint8_t* sD = smem + (pk & 1) * kDStageBytes + (d & 1) * kDOpBytes;
      const int j = 2 * (d >> 1) + (k & 1);
      const int jp = j & 1, h = j >> 2;
      const bool kin = KFULL || pk * kPRow + pchunk[jp] * 16 < kbytes;   // K tail: whole chunks
      const int soff = pk * kPRow + 8 * (j & 3) * kbytes;
      lds_void* dst = (lds_void*)(sD + (kRW * wave + 8 * j) * kPRow);
      if (d & 1)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, dst, 16, kin ? vow[2 * h + jp] : kOutOfRange, soff,
                                                 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, kin ? voa[2 * h + jp] : kOutOfRange, soff,
                                                 0, 0);
    } else if constexpr (MX && !SALIGN) {
      const int st = k & (kStages - 1);
      const int j = d - kNP;
      uint8_t* ss = sscale + st * kScaleStage;
      lds_void* dst = (lds_void*)(ss + (j * 512 + 64 * wave) * 4);
      const uint32_t vo = k * 4 + j < kblocks ? vos + j : kOutOfRange;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, dst, 1, vo, k * 4, 0, 0);
    }
  };

  // Grouped exponents of k-steps 4 G .. 4 G + 3 go to slot G % 3 as 32 chunks
  // of 16 rows, chunk q at q * kChunk: dword 16 j + r' of a chunk holds k-step
  // j of row 16 q + r', so one k-step of 32 consecutive rows spans 32 banks
  // (the 64-byte skew per chunk shifts the second 16 rows by 16 banks).
  // Piece p (0 .. kExpPieces - 1) of a group is chunk kExpPieces w + p of
  // wave w.  The pieces of group g + 2 go out half per odd step at steps
  // 4 g + 1 and 4 g + 3; its slot
  // last held group g - 1, whose reads ended before the barrier of step
  // 4 g - 1.  They are waited for by the barrier of step 4 g + 5 at the
  // latest, before the reads of k-step 4 g + 8.
  auto issue_exp = [&](int G, int p) {
    if constexpr (kGrouped) {
      uint8_t* dst = sscale + (G % 3) * kExpSlot + (LY::kExpPieces * wave + p) * kChunk;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsx, (lds_void*)dst, 4, vos,
                                               p * 16 * kblocks + G * 16, 0, 0);
    }
  };
  // lane's offset within a group slot for rows r0 + l32 (r0 a multiple of 32)
  const int eoff = (l32 >> 4) * kChunk + (l32 & 15) * 4;

  // LDS read offsets within a double stage: the lane's row in the first
  // 32-row tile of its A rows (wm) and W rows (wn), for k-step parity h and
  // fragment half c (FP8: chunk 4 h + 2 lh + c, MX: chunk 4 h + 2 c + lh).
  // The other tiles lie 32 rows (4 KiB) further, and the row swizzle
  // (r >> 1) & 7 depends only on l32 because every tile starts at a multiple
  // of 32 rows; so each read is one of these offsets plus a constant.
  int offA[2][2], offW[2][2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int ch = (4 * h + (MX ? 2 * c + lh : 2 * lh + c)) ^ ((l32 >> 1) & 7);
      offA[h][c] = (wm * 128 + l32) * kPRow + (ch << 4);
      offW[h][c] = kDOpBytes + (wn * kWN + l32) * kPRow + (ch << 4);
    }

  typedef Frags<MX, NT> frags_t;
  // Fragment reads of k-step k, in the order the MFMAs consume them: entry
  // e of kOrd is A tile e (e < 4) or W tile e - 4 (the first 4 + NT entries).
  constexpr int kOrd[8] = {4, 0, 1, 2, 3, 5, 6, 7};
  constexpr int kTiles = 4 + NT;                    // fragment tiles per k-step
  constexpr int kEWords = kGrouped ? 1 : kSWords;   // exponent reads per row and k-step
  constexpr int kReads = MX ? 2 * kTiles + kTiles * kEWords : 2 * kTiles;
  auto read_piece = [&](int k, frags_t& f, int p, auto hpar) {
    constexpr int H = decltype(hpar)::value;   // k & 1
    const int st = k & (kStages - 1);
    const uint8_t* sA = smem + ((k >> 1) & 1) * kDStageBytes;
    if constexpr (!MX) {
      // the lane holds bytes 32 * lh .. +32 of the k-step's 64 for its row
      // (half h = 16 of them); both operands use the same byte -> k map
      const int e = kOrd[p >> 1], h = p & 1;
      const bool isw = e >= 4;
      const u32x4 v = *reinterpret_cast<const u32x4*>(
          sA + (isw ? offW[H][h] + (e - 4) * 32 * kPRow : offA[H][h] + e * 32 * kPRow));
      i32x8& dst = isw ? f.w[e - 4] : f.a[e];
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[4 * h + i] = (int)v[i];
    } else {
      if (p < kTiles * kEWords) {
        // exponents first: row entry p / kEWords (A rows 0..3, W rows 4..)
        const int e = p / kEWords, j = p % kEWords;
        const bool isw = e >= 4;
        const int r0 = isw ? 256 + wn * kWN + (e - 4) * 32 : wm * 128 + e * 32;
        uint32_t& dst = isw ? f.ws[e - 4] : f.as[e];
        uint32_t v;
        if constexpr (kGrouped) {
          const uint8_t* se = sscale + ((k >> 2) % 3) * kExpSlot + (r0 >> 4) * kChunk + (k & 3) * 64;
          v = *reinterpret_cast<const uint32_t*>(se + eoff);
        } else {
          const uint32_t* ss = reinterpret_cast<const uint32_t*>(sscale + st * kScaleStage);
          v = ss[j * 512 + r0 + l32];
        }
        if (j == 0)
          dst = v;
        else
          dst |= v << (8 * j);
        // the lane's block in sub-step s is byte 2 s + lh: shifted to byte 2 s
        if (j == kEWords - 1) dst >>= 8 * lh;
      } else {
        // sub-step s: the lane holds block 2 s + lh of the k-step (16 bytes)
        const int q = p - kTiles * kEWords;
        const int sub = q / kTiles, e = kOrd[q % kTiles];
        const bool isw = e >= 4;
        const i32x4 v = *reinterpret_cast<const i32x4*>(
            sA + (isw ? offW[H][sub] + (e - 4) * 32 * kPRow : offA[H][sub] + e * 32 * kPRow));
        if (isw)
          f.w[sub][e - 4] = v;
        else
          f.a[sub][e] = v;
      }
    }
  };

  // NT x 4 tiles of 32x32 per wave (32 NT channels x 128 rows), D[n][m] in
  // 16 fp32 per lane
  f32x16 acc[4][4];                               // [u < NT][t]
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // MFMA i of k-step k: tile (u, t) = ((i / 4) % NT, i % 4); MX sub-step
  // i / (4 NT)
  constexpr int kMfma = (MX ? 2 : 1) * 4 * NT;
  auto mma_piece = [&](const frags_t& f, int k, int i) {
    const int u = (i >> 2) % NT, t = i & 3;
    if constexpr (!MX) {
      // constant zero scale operands: the compiler selects the unscaled
      // v_mfma_f32_32x32x64_f8f6f4 (8-byte encoding, no scale prefix), whose
      // products equal those of scale bytes 127 (2^0) bit for bit
      acc[u][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[u], f.a[t], acc[u][t], 0, 0,
                                                                  0, 0, 0, 0);
    } else {
      // the scale operands are the exponent dwords with byte 2 s selected;
      // blocks past K (last k-step, K not a multiple of 128) have zero codes
      // and zero exponent bytes, so their products are zero
      const int sub = i / (4 * NT);
      const i32x8 wf = i32x8{f.w[sub][u][0], f.w[sub][u][1], f.w[sub][u][2], f.w[sub][u][3], 0, 0, 0, 0};
      const i32x8 af = i32x8{f.a[sub][t][0], f.a[sub][t][1], f.a[sub][t][2], f.a[sub][t][3], 0, 0, 0, 0};
      if (sub == 0)
        acc[u][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf, af, acc[u][t], 4, 4, 0,
                                                                    (int)f.ws[u], 0, (int)f.as[t]);
      else
        acc[u][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf, af, acc[u][t], 4, 4, 2,
                                                                    (int)f.ws[u], 2, (int)f.as[t]);
    }
  };

  // k-step k: stage k + 1 has landed and stage k (and k - 1) are free.  The
  // loads go out in pairs of k-steps (k + 3, k + 4) at odd k, interleaved so
  // that the two 64-byte halves of every 128-byte row segment are requested
  // back to back and each cache line crosses from L2 once.  Meanwhile the
  // MFMAs of k-step k (in cur) run, each followed by its share of the
  // fragment reads of k + 1 (all issued in the first three quarters of the
  // k-step, so they have landed by the next barrier) and of the loads.
  // Loads past the last k-step read zeros and keep the wait counts uniform.
  // At the barrier of an even step the pair (k + 2, k + 3) may still be in
  // flight; at an odd step the pair holding k + 1 is waited for entirely.
  // Grouped exponents: every odd step also issues two exponent pieces after
  // its operand loads, so an even step lets those 10 loads stay in flight.
  constexpr int kExpPer = kGrouped ? LY::kExpPieces / 2 : 0;
  constexpr int kReadsPer = (kReads + (3 * kMfma / 4) - 1) / (3 * kMfma / 4);
  constexpr int kLoadsPer = (2 * kGroup + kExpPer + kMfma - 1) / kMfma;
  auto step = [&](int k, frags_t& cur, frags_t& nxt, auto odd_t) {
    constexpr bool odd = decltype(odd_t)::value;
    wait_vm_barrier<odd ? 0 : 2 * kGroup + kExpPer>();
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      mma_piece(cur, k, i);
#pragma unroll
      for (int r = 0; r < kReadsPer; ++r)
        if (i * kReadsPer + r < kReads)
          read_piece(k + 1, nxt, i * kReadsPer + r, std::integral_constant<int, odd ? 0 : 1>{});
      if constexpr (odd) {
#pragma unroll
        for (int r = 0; r < kLoadsPer; ++r) {
          const int x = i * kLoadsPer + r;     // x / 2 = piece, x % 2 = which k-step
          if (x < 2 * kGroup)
            issue_piece(k + 3 + (x & 1), x >> 1);
          else if (x < 2 * kGroup + kExpPer)   // group (k - 1) / 4 + 2, pieces 2 ((k >> 1) & 1) + 0, 1
            issue_exp(((k - 1) >> 2) + 2, kExpPer * ((k >> 1) & 1) + (x - 2 * kGroup));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // FP8: the epilogue's scales go first (they retire before the operands
  // the first wait is for).  The first half of the waves bring s_x of the
  // 256 tile rows, the second half s_w of the 256 tile channels (SwiGLU:
  // gate channels c0 .., then the same channels' up rows), 64 dwords per
  // load; out of range reads 0.
  float* const sepi = reinterpret_cast<float*>(smem + kRing);
  if constexpr (!MX) {
    constexpr int kSL = 512 / 64 / kWaves;          // 64-dword loads per wave
    const bool wsc = wave >= kWaves / 2;
    const __amdgpu_buffer_rsrc_t rsc =
        make_rsrc(wsc ? w_aux : a_aux, (int64_t)(wsc ? N : M) * 4);
#pragma unroll
    for (int h = 0; h < kSL; ++h) {
      const int q0 = 64 * (kSL * (wave % (kWaves / 2)) + h);
      const int q = q0 + lane;
      int row;
      if (!wsc)
        row = m0 + q;
      else if constexpr (SWIGLU)
        row = (q >> 7) * I + c0 + (q & 127);
      else
        row = n0 + q;
      const bool ok = SWIGLU && wsc ? c0 + (q & 127) < I : true;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (lds_void*)(sepi + 256 * wsc + q0), 4,
                                               ok ? (uint32_t)row * 4 : kOutOfRange, 0, 0, 0);
    }
  }
  // prologue: k-steps 0..3 in two interleaved pairs (grouped exponents:
  // group 0 before them, group 1 after); stage 0 (all of the first pair)
  // must land before its fragments are read
  if constexpr (kGrouped) {
#pragma unroll
    for (int p = 0; p < LY::kExpPieces; ++p) issue_exp(0, p);
  }
#pragma unroll
  for (int k0 = 0; k0 < 4; k0 += 2)
#pragma unroll
    for (int x = 0; x < 2 * kGroup; ++x) issue_piece(k0 + (x & 1), x >> 1);
  if constexpr (kGrouped) {
#pragma unroll
    for (int p = 0; p < LY::kExpPieces; ++p) issue_exp(1, p);
  }
  wait_vm_barrier<2 * kGroup + (kGrouped ? LY::kExpPieces : 0)>();
  frags_t f0, f1;
#pragma unroll
  for (int p = 0; p < kReads; ++p) read_piece(0, f0, p, std::integral_constant<int, 0>{});
  int k = 0;
  for (; k + 1 < nk; k += 2) {
    step(k, f0, f1, std::false_type{});
    step(k + 1, f1, f0, std::true_type{});
  }
  if (k < nk) step(k, f0, f1, std::false_type{});
  // the trailing loads (zeros) must land before the LDS is reused
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue.  The lane holds D[n = 8 * (r / 4) + 4 * lh + r % 4][m = l32] of
  // each 32x32 tile.  FP8 rescales by s_x[m] * s_w[n] (from LDS, where the
  // prologue put them; out-of-range rows and channels read as zero).
  // The bf16 results go through LDS so that each row of the tile leaves in
  // 16-byte pieces that fill whole cache lines (stores straight from the
  // accumulators, 32 bytes of 32 rows per instruction, measured 15 % slower
  // for the FP8 and 37 % for the MXFP4 product).
  f32x4 swv[4][4];                                // [u < NT][b]
  float sxv[4];
  if constexpr (!MX) {
#pragma unroll
    for (int t = 0; t < 4; ++t) sxv[t] = sepi[wm * 128 + t * 32 + l32];
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        // SwiGLU: W tile u holds the gate (u even) or up (u odd) rows of
        // channels wn kWN / 2 + 32 (u / 2) .. of the tile
        const int q = SWIGLU ? (u & 1) * 128 + wn * (kWN / 2) + 32 * (u >> 1) + 8 * b + 4 * lh
                             : wn * kWN + u * 32 + 8 * b + 4 * lh;
        swv[u][b] = *reinterpret_cast<const f32x4*>(sepi + 256 + q);
      }
  }
  __syncthreads();   // every wave is done with the operand buffers
  if constexpr (SWIGLU) {
    // h = SiLU(g) * u per lane (fp32, e^-g from the hardware exponential),
    // staged as the wave's 128 (m) x kWN / 2 (channel) bf16 piece with a
    // 16-byte pad per row, then whole rows per store instruction (kLR lanes
    // x 16 bytes a row)
    constexpr int kHC = kWN / 2;                    // channels of h per wave
    constexpr int kHPitch = kHC * 2 + 16;
    constexpr int kLR = kHC / 8;                    // lanes per staged row
    uint8_t* sh = smem + wave * (128 * kHPitch);
#pragma unroll
    for (int pp = 0; pp < NT / 2; ++pp)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float g = acc[2 * pp][t][4 * b + r] * (sxv[t] * swv[2 * pp][b][r]);
            const float u = acc[2 * pp + 1][t][4 * b + r] * (sxv[t] * swv[2 * pp + 1][b][r]);
            v[r] = g / (1.f + __expf(-g)) * u;
          }
          const int ml = t * 32 + l32, nl = 32 * pp + 8 * b + 4 * lh;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * 128 + ml, c = c0 + wn * kHC + nl + r;
            if (m < M && c < I) QG_DEBUG_STORE((int64_t)m * I + c, v[r]);
          }
          *reinterpret_cast<uint2*>(sh + ml * kHPitch + nl * 2) =
              make_uint2(cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3]));
        }
    wait_own_lds();
    const int cbase = c0 + wn * kHC + (lane % kLR) * 8;
    const bool full_c = cbase + 7 < I && (I & 7) == 0;
#pragma unroll 4
    for (int i = 0; i < 128 * kLR / 64; ++i) {
      const int ml = (64 / kLR) * i + lane / kLR;
      const int m = m0 + wm * 128 + ml;
      const u32x4 o = *reinterpret_cast<const u32x4*>(sh + ml * kHPitch + (lane % kLR) * 16);
      if (m < M) {
        uint16_t* ph = Y + (int64_t)m * I + cbase;
        if (full_c) {
          __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(ph));
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (cbase + j < I) ph[j] = (uint16_t)(o[j >> 1] >> (16 * (j & 1)));
        }
      }
    }
    return;
  }
  uint8_t* so = smem + wave * (128 * kEpiPitch);
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = acc[u][t][4 * b + r];
          if constexpr (!MX) v[r] *= sxv[t] * swv[u][b][r];
        }
        const int ml = t * 32 + l32, nl = u * 32 + 8 * b + 4 * lh;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * 128 + ml, n = n0 + wn * kWN + nl + r;
          if (m < M && n < N) QG_DEBUG_STORE((int64_t)m * N + n, v[r]);
        }
        *reinterpret_cast<uint2*>(so + ml * kEpiPitch + nl * 2) =
            make_uint2(cvt_bf16x2(v[0], v[1]), cvt_bf16x2(v[2], v[3]));
      }
  wait_own_lds();
  // kLR lanes x 8 outputs per row (8 or 16), 64 / kLR rows per instruction
  constexpr int kLR = kWN / 8;
  const int nbase = n0 + wn * kWN + (lane % kLR) * 8;
  const bool full_n = nbase + 7 < N && (N & 7) == 0;
#pragma unroll 4
  for (int i = 0; i < 128 * kLR / 64; ++i) {
    const int ml = (64 / kLR) * i + lane / kLR;
    const int m = m0 + wm * 128 + ml;
    const u32x4 o = *reinterpret_cast<const u32x4*>(so + ml * kEpiPitch + (lane % kLR) * 16);
    if (m < M) {
      uint16_t* py = Y + (int64_t)m * N + nbase;
      if (full_n) {
        // nontemporal: the output is not read again by this kernel
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(py));
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (nbase + j < N) py[j] = (uint16_t)(o[j >> 1] >> (16 * (j & 1)));
      }
    }
  }
}

template <bool MX, bool SALIGN, bool KFULL, bool SWIGLU = false, bool W4 = false>
hipError_t launch(const void* a, const void* a_aux, int64_t M, const void* w, const void* w_aux,
                  int64_t N, int64_t K, void* y, hipStream_t stream) {
  const int64_t tn = SWIGLU ? (N / 2 + BN / 2 - 1) / (BN / 2) : (N + BN - 1) / BN;
  const int tiles = (int)(((M + BM - 1) / BM) * tn);
  hipLaunchKernelGGL((gemm_f8f4_kernel<MX, SALIGN, KFULL, SWIGLU, W4>), dim3(tiles),
                     dim3(Layout<W4>::kThreads), 0, stream,
                     (const uint8_t*)a, a_aux, (int)M, (const uint8_t*)w, w_aux, (int)N, (int)K,
                     (uint16_t*)y);
  return hipGetLastError();
}

}  // namespace

QG_DEBUG_TU_SETTER(debug_set_f8f4)

// FP8 with whole k-steps runs the 4-wave layout (8192^3 on MI355X: 375 ->
// 369 us and 387 -> 381 us in A/Bs on two boxes); MXFP4 keeps 8 waves (the
// 4-wave layout measured 131 -> 132.5 us).
hipError_t launch_gemm_fp8(const void* a, const void* a_scales, int64_t M, const void* w,
                           const void* w_scales, int64_t N, int64_t K, void* y,
                           hipStream_t stream) {
  if (K % BK == 0)
    return launch<false, true, true, false, true>(a, a_scales, M, w, w_scales, N, K, y, stream);
  return launch<false, true, false>(a, a_scales, M, w, w_scales, N, K, y, stream);
}

hipError_t launch_gemm_fp8_swiglu(const void* a, const void* a_scales, int64_t M, const void* w,
                                  const void* w_scales, int64_t N2, int64_t K, void* h,
                                  hipStream_t stream) {
  if (K % BK == 0)
    return launch<false, true, true, true, true>(a, a_scales, M, w, w_scales, N2, K, h, stream);
  return launch<false, true, false, true>(a, a_scales, M, w, w_scales, N2, K, h, stream);
}

hipError_t launch_mx_gemm(const void* a_codes, const void* a_e8m0, int64_t M,
                          const void* b_codes, const void* b_e8m0, int64_t N, int64_t K, void* y,
                          hipStream_t stream) {
  // one aligned exponent dword per row and k-step, and whole k-steps of 128
  // codes, when K is a multiple of 128
  if (K % 128 == 0)
    return launch<true, true, true>(a_codes, a_e8m0, M, b_codes, b_e8m0, N, K, y, stream);
  return launch<true, false, false>(a_codes, a_e8m0, M, b_codes, b_e8m0, N, K, y, stream);
}

}  // namespace qg
