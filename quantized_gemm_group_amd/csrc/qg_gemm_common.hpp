// Pieces shared by the tiled GEMM kernels (W4A16 prefill, FP8, INT8, MXFP4).
//
// Conventions of every GEMM kernel here:
//  * Y[M][N] = A[M][K] * W[N][K]^T, both operands K-contiguous.
//  * The matrix-core call takes the W fragment as its first operand and the
//    A fragment as its second, so a lane's accumulators hold 4 consecutive
//    output channels n of one row m (16x16 tiles: lane l holds D[n][m] for
//    n = 4*(l/16) + r, m = l%16), which the epilogue writes as one 8-byte
//    store of 4 bf16.
//  * Global loads are raw buffer loads: a row past the end of the operand
//    reads as zero (the buffer's byte range is checked by the hardware), so
//    ragged M and N tiles need no branches; a K tail is masked by pointing
//    the load past the range.
//  * Operand tiles live in LDS with an XOR swizzle of their 16-byte chunks
//    (chunk c of row r at c ^ (r & 7)) so the 8 rows read by 8 consecutive
//    lanes of a 128-bit LDS read land on distinct banks.
#pragma once

#include "qg_device.hpp"

namespace qg {

constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, int64_t bytes) {
  const int64_t lim = bytes > 0x7ffff000LL ? 0x7ffff000LL : bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)lim, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// Byte offset of 16-byte chunk c of row r in a swizzled tile whose rows are
// `row_bytes` long (a multiple of 128).
__device__ __forceinline__ int swz(int r, int c, int row_bytes) {
  return r * row_bytes + ((c ^ (r & 7)) << 4);
}

// Two fp32 values rounded to bf16 (nearest even) by the hardware conversion,
// low half first.
__device__ __forceinline__ uint32_t cvt_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Store 4 consecutive outputs n..n+3 of row m (already scaled) as bf16.
__device__ __forceinline__ void store_out4(uint16_t* __restrict__ y, int M, int N, int m, int n,
                                           float v0, float v1, float v2, float v3) {
  if (m >= M) return;
  uint16_t* p = y + (int64_t)m * N + n;
  if (n < N) QG_DEBUG_STORE((int64_t)m * N + n, v0);
  if (n + 1 < N) QG_DEBUG_STORE((int64_t)m * N + n + 1, v1);
  if (n + 2 < N) QG_DEBUG_STORE((int64_t)m * N + n + 2, v2);
  if (n + 3 < N) QG_DEBUG_STORE((int64_t)m * N + n + 3, v3);
  if (n + 3 < N && (N & 3) == 0) {
    uint2 o;
    o.x = pack_bf16x2(v0, v1);
    o.y = pack_bf16x2(v2, v3);
    *reinterpret_cast<uint2*>(p) = o;
  } else {
    const float v[4] = {v0, v1, v2, v3};
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) p[r] = (uint16_t)f32_to_bf16_bits(v[r]);
  }
}

// Tile order: consecutive workgroups walk down a column of GROUP_M tiles
// before moving right, so tiles that share operand panels run together and
// hit in L2.
__device__ __forceinline__ void tile_coords(int bid, int tiles_m, int tiles_n, int group_m,
                                            int* tm, int* tn) {
  const int per_group = group_m * tiles_n;
  const int g = bid / per_group;
  const int first_m = g * group_m;
  const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int in = bid - g * per_group;
  *tm = first_m + in % gm;
  *tn = in / gm;
}

}  // namespace qg
