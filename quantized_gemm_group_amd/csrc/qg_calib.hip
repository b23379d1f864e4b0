// Roofline calibration probes: the two roofs of 《第 1 章：推理加速全景》
// section 1.5 (attainable throughput = min(memory bandwidth x arithmetic
// intensity, compute peak)) measured on this GPU instead of taken from the
// data sheet.  Neither is a step of the quantized linear layer; the benchmark
// reports them beside the published peaks.
//
//  * stream_read_kernel: a read-only HBM stream, the fastest single-launch
//    pattern found on MI355X (every workgroup reads one contiguous 64 KiB
//    chunk, each lane 16 sixteen-byte non-temporal loads, all issued before
//    the first use, every load instruction covering 1 KiB contiguous).  The XOR of each
//    chunk's 32-bit words goes to sink[chunk], so nothing is dead code and the
//    result is checkable.
//  * mfma_loop_kernel: back-to-back 32x32 matrix instructions with no memory
//    traffic in the loop, four independent accumulators per wave, operands
//    drawn per lane from a hash and perturbed every iteration (only mantissa
//    bits change, so no NaN or infinity appears): the matrix-core rate of
//    each data type under data that toggles like a real GEMM's.

#include "qg_device.hpp"
#include "qg_internal.hpp"

namespace qg {
namespace {

typedef __attribute__((ext_vector_type(16))) int i32x16;

constexpr int kChunkLoads = 16;           // 16-byte loads per lane and chunk

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src,
                                                          uint32_t* __restrict__ sink) {
  // buffer resource over this workgroup's chunk; the loads carry the
  // non-temporal hint (measured on MI355X: 62.4 MB per launch in 10.4 us
  // against 11.4 us without it; 1 GiB at 6.65 against 5.7 TB/s)
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(src + (size_t)blockIdx.x * (kChunkLoads * 256)), (short)0, kChunkLoads * 256 * 16,
      0x00020000);
  u32x4 v[kChunkLoads];
#pragma unroll
  for (int i = 0; i < kChunkLoads; ++i)
    v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         r, (uint32_t)(i * 256 + threadIdx.x) * 16, 0, 2));
  uint32_t x = 0;
#pragma unroll
  for (int i = 0; i < kChunkLoads; ++i) x ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x ^= (uint32_t)__shfl_xor((int)x, o, 64);
  __shared__ uint32_t part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__device__ __forceinline__ uint32_t hash32(uint32_t a) {
  a ^= a >> 16;
  a *= 0x7feb352du;
  a ^= a >> 15;
  a *= 0x846ca68bu;
  a ^= a >> 16;
  return a;
}

// KIND: 0 bf16 (v_mfma_f32_32x32x16_bf16), 1 fp8 E4M3 and 2 fp4 E2M1
// (v_mfma_scale_f32_32x32x64_f8f6f4, unit scales passed per lane as the MX
// GEMM does), 3 int8 (v_mfma_i32_32x32x32_i8).
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const uint32_t gl = blockIdx.x * 256 + threadIdx.x;
  // operand dwords: random, then masked so every value is finite
  //   bf16: sign and mantissa random, exponent 127 (values in +-[1, 2))
  //   fp8 : bit 0 clear (mantissa never 111, the NaN pattern)
  //   fp4, int8: every pattern valid
  constexpr uint32_t keep = KIND == 0 ? 0x807F807Fu : (KIND == 1 ? 0xFEFEFEFEu : 0xFFFFFFFFu);
  constexpr uint32_t set = KIND == 0 ? 0x3F803F80u : 0u;
  constexpr uint32_t flip = KIND == 0 ? 0x007F007Fu : (KIND == 1 ? 0x06060606u : 0xFFFFFFFFu);
  uint32_t a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (hash32(gl * 16 + j) & keep) | set;
    b[j] = (hash32(gl * 16 + 8 + j) & keep) | set;
  }
  uint32_t r = hash32(gl ^ 0x9e3779b9u);
  const int scale = 127 - (int)(threadIdx.x & 1);    // per-lane scale register (2^0, 2^-1)
  f32x16 acc[4];
  i32x16 iacc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      acc[t][e] = 0.f;
      iacc[t][e] = 0;
    }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = i & 3;
      if constexpr (KIND == 0) {
        const bf16x8 av = __builtin_bit_cast(bf16x8, u32x4{a[(i & 1) * 4], a[(i & 1) * 4 + 1],
                                                            a[(i & 1) * 4 + 2], a[(i & 1) * 4 + 3]});
        const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{b[(i & 1) * 4], b[(i & 1) * 4 + 1],
                                                            b[(i & 1) * 4 + 2], b[(i & 1) * 4 + 3]});
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[t], 0, 0, 0);
      } else if constexpr (KIND == 1) {
        const i32x8 av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                          (int)a[4], (int)a[5], (int)a[6], (int)a[7]};
        const i32x8 bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3],
                          (int)b[4], (int)b[5], (int)b[6], (int)b[7]};
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[t], 0, 0, 0, scale,
                                                                 0, scale);
      } else if constexpr (KIND == 2) {
        const int h = (i & 1) * 4;
        const i32x8 av = {(int)a[h], (int)a[h + 1], (int)a[h + 2], (int)a[h + 3], 0, 0, 0, 0};
        const i32x8 bv = {(int)b[h], (int)b[h + 1], (int)b[h + 2], (int)b[h + 3], 0, 0, 0, 0};
        acc[t] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc[t], 4, 4, 0, scale,
                                                                 0, scale);
      } else {
        const int h = (i & 1) * 4;
        const i32x4 av = {(int)a[h], (int)a[h + 1], (int)a[h + 2], (int)a[h + 3]};
        const i32x4 bv = {(int)b[h], (int)b[h + 1], (int)b[h + 2], (int)b[h + 3]};
        iacc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(av, bv, iacc[t], 0, 0, 0);
      }
    }
    // new operand bits for the next iteration (mantissa bits only)
    r = (r << 1) | (r >> 31);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] ^= r & flip;
      b[j] ^= (r >> (j + 1)) & flip;
    }
  }
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += KIND == 3 ? (float)iacc[t][e] : acc[t][e];
  sink[gl] = s;
}

}  // namespace

hipError_t launch_calib_stream_read(const void* src, int64_t bytes, uint32_t* sink,
                                    hipStream_t stream) {
  const int64_t chunks = bytes / (kChunkLoads * 256 * 16);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)chunks), dim3(256), 0, stream,
                     (const u32x4*)src, sink);
  return hipGetLastError();
}

hipError_t launch_calib_mfma(int kind, int64_t waves, int64_t iters, float* sink,
                             hipStream_t stream) {
  const unsigned blocks = (unsigned)(waves / 4);
  switch (kind) {
    case 0: hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(blocks), dim3(256), 0, stream, (int)iters, sink); break;
    case 1: hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(blocks), dim3(256), 0, stream, (int)iters, sink); break;
    case 2: hipLaunchKernelGGL(mfma_loop_kernel<2>, dim3(blocks), dim3(256), 0, stream, (int)iters, sink); break;
    default: hipLaunchKernelGGL(mfma_loop_kernel<3>, dim3(blocks), dim3(256), 0, stream, (int)iters, sink); break;
  }
  return hipGetLastError();
}

}  // namespace qg
