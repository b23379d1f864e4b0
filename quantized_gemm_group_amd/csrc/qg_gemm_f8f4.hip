// FP8 E4M3 W8A8 GEMM and MXFP4 block-scaled GEMM on the gfx950 scaled
// matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4).
//
// FP8 (《第 6 课：量化源码走读》 section 2 and figure 6-2): the matrix cores
// multiply the E4M3 codes exactly and accumulate in fp32; the epilogue
// rescales by s_x[m] * s_w[n] (per-token activation scale, per-channel weight
// scale) and rounds once to bf16.  The MFMA's own block scales are set to
// 2^0 (E8M0 byte 127).
//
// MXFP4 (《大模型量化推理引擎全景大复盘》 section 2 eq. 3; 《第 6 课：量化源码走读》
// section 2): each lane of the MFMA holds 32 E2M1 codes of one row that form
// exactly one 32-element block, and passes that block's E8M0 byte as its
// scale, so 2^(ea + eb) is applied inside the matrix core and the epilogue
// only rounds.
//
// Tiling: a 256-thread workgroup owns a 256x256 output tile and its 4 waves a
// 128x128 quarter each (4x4 tiles of v_mfma_scale_f32_32x32x64_f8f6f4, 256
// fp32 accumulators per lane), which halves the LDS bytes read per MFMA
// compared with 64x64 quarters; the 64-deep K of the 32x32 shape keeps the
// operand registers of one sub-step small.
// Each k-step stages 128 bytes per row of both operands (128 FP8 or 256 FP4
// codes) into one of two LDS buffers through registers: the next k-step's
// global loads are issued first, the current buffer is multiplied, then the
// registers are written to the other buffer -- one barrier per k-step.
// Workgroups are dispatched round-robin over the 8 XCDs; each XCD is given a
// contiguous range of tiles walked in column groups, so concurrently running
// workgroups of one XCD share operand panels in its L2.

#include "qg_gemm_common.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

constexpr int BM = 256, BN = 256, BKB = 128;   // tile rows and bytes per row per k-step
constexpr int kStageBytes = (BM + BN) * BKB;   // 64 KiB per buffer

// Tile of workgroup `bid`: XCD-contiguous ranges (when the tile count divides
// evenly over the XCDs), then column groups of `group_m` tile rows.
__device__ __forceinline__ void xcd_tile(int bid, int tiles_m, int tiles_n, int* tm, int* tn) {
  constexpr int kXcd = 8;
  const int tiles = tiles_m * tiles_n;
  int lin = bid;
  if (tiles % kXcd == 0) lin = (bid % kXcd) * (tiles / kXcd) + bid / kXcd;
  tile_coords(lin, tiles_m, tiles_n, 4, tm, tn);
}

template <bool MX> struct FragT { typedef i32x8 type; };
template <> struct FragT<true> { typedef i32x4 type; };

template <bool MX, bool SVEC>
__global__ __launch_bounds__(256) void gemm_f8f4_kernel(const uint8_t* __restrict__ A,
                                                        const void* __restrict__ a_aux, int M,
                                                        const uint8_t* __restrict__ W,
                                                        const void* __restrict__ w_aux, int N,
                                                        int K, uint16_t* __restrict__ Y) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kStageBytes];
  __shared__ __attribute__((aligned(16))) uint8_t sscale[MX ? 2 * (BM + BN) * 8 : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int l32 = lane & 31, lh = lane >> 5;

  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  xcd_tile(blockIdx.x, tiles_m, tiles_n, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const int kbytes = MX ? K / 2 : K;           // bytes per operand row
  const int nk = (kbytes + BKB - 1) / BKB;
  // rows past M (N) fall outside the buffer's byte range and read as zero
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (int64_t)M * kbytes);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W, (int64_t)N * kbytes);

  // staging map: chunk q = tid + 256 i (i < 8) of each operand tile sits at
  // row (tid >> 3) + 32 i, 16-byte chunk tid & 7
  const int srow = tid >> 3, scol = (tid & 7) * 16;
  const uint32_t va0 = (uint32_t)(m0 + srow) * kbytes + scol;
  const uint32_t vw0 = (uint32_t)(n0 + srow) * kbytes + scol;
  const uint32_t rstep = 32u * (uint32_t)kbytes;
  // MX scales: thread t stages the 8 block exponents of A row t and W row t
  const int kblocks = K / 32;
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(a_aux, MX ? (int64_t)M * kblocks : 0);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(w_aux, MX ? (int64_t)N * kblocks : 0);
  const bool sa_ok = m0 + tid < M, sw_ok = n0 + tid < N;

  u32x4 rar[8], rwr[8];
  uint32_t sa_lo = 0, sa_hi = 0, sw_lo = 0, sw_hi = 0;

  // global -> registers for k-step kb; a k-step past the end reads zeros
  auto gload = [&](int kb) {
    const bool kin = kb * BKB + scol < kbytes;     // K tail: mask whole chunks
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      rar[i] = buf_load16(ra, kin ? va0 + i * rstep : kOutOfRange, kb * BKB);
      rwr[i] = buf_load16(rw, kin ? vw0 + i * rstep : kOutOfRange, kb * BKB);
    }
    if constexpr (MX && SVEC) {
      // a row's 8 exponents of this k-step are 8 aligned bytes
      const bool bin = kb * 8 < kblocks;
      const uint32_t oa = (sa_ok && bin) ? (uint32_t)(m0 + tid) * kblocks + kb * 8 : kOutOfRange;
      const uint32_t ow = (sw_ok && bin) ? (uint32_t)(n0 + tid) * kblocks + kb * 8 : kOutOfRange;
      const uint2 a8 = buf_load8(rsa, oa, 0), w8 = buf_load8(rsw, ow, 0);
      sa_lo = a8.x;
      sa_hi = a8.y;
      sw_lo = w8.x;
      sw_hi = w8.y;
    } else if constexpr (MX) {
      sa_lo = sa_hi = sw_lo = sw_hi = 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int blk = kb * 8 + j;
        const bool bin = blk < kblocks;
        const uint32_t oa = (sa_ok && bin) ? (uint32_t)(m0 + tid) * kblocks + blk : kOutOfRange;
        const uint32_t ow = (sw_ok && bin) ? (uint32_t)(n0 + tid) * kblocks + blk : kOutOfRange;
        const uint32_t ba = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsa, oa, 0, 0);
        const uint32_t bw = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rsw, ow, 0, 0);
        if (j < 4) {
          sa_lo |= ba << (8 * j);
          sw_lo |= bw << (8 * j);
        } else {
          sa_hi |= ba << (8 * (j - 4));
          sw_hi |= bw << (8 * (j - 4));
        }
      }
    }
  };
  // registers -> LDS buffer `buf`; exponents are stored per row as the dword
  // of the even blocks (0, 2, 4, 6) followed by the dword of the odd blocks,
  // so the lanes of each half of a wave find theirs at one dword
  auto lstore = [&](int buf) {
    uint8_t* sA = smem + buf * kStageBytes;
    uint8_t* sW = sA + BM * BKB;
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = srow + 32 * i;
      *reinterpret_cast<u32x4*>(sA + swz(row, c, BKB)) = rar[i];
      *reinterpret_cast<u32x4*>(sW + swz(row, c, BKB)) = rwr[i];
    }
    if constexpr (MX) {
      uint8_t* ss = sscale + buf * (BM + BN) * 8;
      *reinterpret_cast<uint2*>(ss + tid * 8) =
          make_uint2(__builtin_amdgcn_perm(sa_hi, sa_lo, 0x06040200u),
                     __builtin_amdgcn_perm(sa_hi, sa_lo, 0x07050301u));
      *reinterpret_cast<uint2*>(ss + (BM + tid) * 8) =
          make_uint2(__builtin_amdgcn_perm(sw_hi, sw_lo, 0x06040200u),
                     __builtin_amdgcn_perm(sw_hi, sw_lo, 0x07050301u));
    }
  };

  // Operand fragments of one sub-step of 64 K.  FP8: the lane holds 32 codes
  // (bytes 32 * lh .. +32 of the sub-step's 64) of row l32; both operands use
  // the same byte -> k assignment, so the products pair equal k.  FP4: the
  // lane holds the 32 codes of block 2 * s + lh of the k-step (16 bytes).
  typedef typename FragT<MX>::type frag_t;
  struct Frags {
    frag_t a[4], w[4];
  };
  auto ldfrag = [&](const uint8_t* p, int r, int s) -> frag_t {
    if constexpr (MX) {
      return *reinterpret_cast<const frag_t*>(p + swz(r, 2 * s + lh, BKB));
    } else {
      const int c0 = 4 * s + 2 * lh;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(p + swz(r, c0, BKB));
      const u32x4 hi = *reinterpret_cast<const u32x4*>(p + swz(r, c0 + 1, BKB));
      return frag_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                    (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  };
  auto lfrag = [&](int buf, int s, Frags& f) {
    const uint8_t* sA = smem + buf * kStageBytes;
    const uint8_t* sW = sA + BM * BKB;
#pragma unroll
    for (int t = 0; t < 4; ++t) f.a[t] = ldfrag(sA, wm * 128 + t * 32 + l32, s);
#pragma unroll
    for (int u = 0; u < 4; ++u) f.w[u] = ldfrag(sW, wn * 128 + u * 32 + l32, s);
  };
  // the lane's exponent dword (even or odd blocks) of each of its 8 rows
  auto lscale = [&](int buf, uint32_t* asc, uint32_t* wsc) {
    const uint32_t* ss = reinterpret_cast<const uint32_t*>(sscale + buf * (BM + BN) * 8);
#pragma unroll
    for (int t = 0; t < 4; ++t) asc[t] = ss[(wm * 128 + t * 32 + l32) * 2 + lh];
#pragma unroll
    for (int u = 0; u < 4; ++u) wsc[u] = ss[(BM + wn * 128 + u * 32 + l32) * 2 + lh];
  };

  // 4 x 4 tiles of 32x32 per wave (128 x 128), D[n][m] in 16 fp32 per lane
  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  uint32_t asc[4] = {0, 0, 0, 0}, wsc[4] = {0, 0, 0, 0};
  auto mma = [&](const Frags& f, int s, int u0, int u1) {
#pragma unroll
    for (int u = u0; u < u1; ++u)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (MX) {
          const i32x8 wf = i32x8{f.w[u][0], f.w[u][1], f.w[u][2], f.w[u][3], 0, 0, 0, 0};
          const i32x8 af = i32x8{f.a[t][0], f.a[t][1], f.a[t][2], f.a[t][3], 0, 0, 0, 0};
          acc[u][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wf, af, acc[u][t], 4, 4, 0, (int)__builtin_amdgcn_ubfe(wsc[u], 8 * s, 8), 0,
              (int)__builtin_amdgcn_ubfe(asc[t], 8 * s, 8));
        } else {
          acc[u][t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.w[u], f.a[t], acc[u][t],
                                                                      0, 0, 0, 127, 0, 127);
        }
      }
  };

  constexpr int S = MX ? 4 : 2;   // sub-steps of 64 K per k-step
  gload(0);
  lstore(0);
  __syncthreads();
  Frags cur;
  lfrag(0, 0, cur);
  if constexpr (MX) lscale(0, asc, wsc);
  // One k-step: the next k-step's global loads go out first; sub-step s is
  // multiplied while sub-step s + 1's fragments are read; during the last
  // sub-step the staged registers are written to the other buffer, and after
  // the barrier the first fragments of the next k-step are read while the
  // last MFMAs run.  The loop body is one basic block (no conditionals), so
  // the interleave hints below apply to all of it.
  for (int kb = 0; kb < nk; ++kb) {
    const int buf = kb & 1;
    gload(kb + 1);
#pragma unroll
    for (int s = 0; s + 1 < S; ++s) {
      Frags nxt;
      lfrag(buf, s + 1, nxt);
      mma(cur, s, 0, 4);
      cur = nxt;
    }
    mma(cur, S - 1, 0, 2);
    lstore(buf ^ 1);
    // issue order (interleave hints for the scheduler)
    if constexpr (!MX) {
      // sub-step 0: 16 MFMAs, 16 global loads, 16 fragment reads
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    } else {
      // sub-step 0: 16 MFMAs, 18 global loads, 8 fragment reads
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);
#pragma unroll
      for (int i = 0; i < 7; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      // sub-steps 1 and 2: 16 MFMAs and 8 fragment reads each
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
    // first half of the last sub-step: 8 MFMAs and the LDS stores
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
    }
    if constexpr (MX) __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
    __syncthreads();
    Frags nxt;
    lfrag(buf ^ 1, 0, nxt);
    uint32_t nasc[4], nwsc[4];
    if constexpr (MX) lscale(buf ^ 1, nasc, nwsc);
    mma(cur, S - 1, 2, 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    cur = nxt;
    if constexpr (MX) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        asc[i] = nasc[i];
        wsc[i] = nwsc[i];
      }
    }
  }

  // epilogue: lane holds D[n = 8*(r/4) + 4*lh + r%4][m = l32] of each 32x32 tile
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int m = m0 + wm * 128 + t * 32 + l32;
    float sxm = 1.f;
    if constexpr (!MX) sxm = (m < M) ? reinterpret_cast<const float*>(a_aux)[m] : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int n = n0 + wn * 128 + u * 32 + 8 * b + 4 * lh;
        float s[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (!MX) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s[r] = (n + r < N) ? reinterpret_cast<const float*>(w_aux)[n + r] * sxm : 0.f;
        }
        store_out4(Y, M, N, m, n, acc[u][t][4 * b] * s[0], acc[u][t][4 * b + 1] * s[1],
                   acc[u][t][4 * b + 2] * s[2], acc[u][t][4 * b + 3] * s[3]);
      }
    }
  }
}

template <bool MX, bool SVEC>
hipError_t launch(const void* a, const void* a_aux, int64_t M, const void* w, const void* w_aux,
                  int64_t N, int64_t K, void* y, hipStream_t stream) {
  const int tiles = (int)(((M + BM - 1) / BM) * ((N + BN - 1) / BN));
  hipLaunchKernelGGL((gemm_f8f4_kernel<MX, SVEC>), dim3(tiles), dim3(256), 0, stream,
                     (const uint8_t*)a, a_aux, (int)M, (const uint8_t*)w, w_aux, (int)N, (int)K,
                     (uint16_t*)y);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_fp8(const void* a, const void* a_scales, int64_t M, const void* w,
                           const void* w_scales, int64_t N, int64_t K, void* y,
                           hipStream_t stream) {
  return launch<false, false>(a, a_scales, M, w, w_scales, N, K, y, stream);
}

hipError_t launch_mx_gemm(const void* a_codes, const void* a_e8m0, int64_t M,
                          const void* b_codes, const void* b_e8m0, int64_t N, int64_t K, void* y,
                          hipStream_t stream) {
  // 8-byte exponent loads when each row's exponents start 8-byte aligned
  if (K % 256 == 0) return launch<true, true>(a_codes, a_e8m0, M, b_codes, b_e8m0, N, K, y, stream);
  return launch<true, false>(a_codes, a_e8m0, M, b_codes, b_e8m0, N, K, y, stream);
}

}  // namespace qg
