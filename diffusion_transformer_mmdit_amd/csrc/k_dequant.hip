// Decode a quantised weight matrix into dense bf16 [N, K] (the values the
// GEMM kernels stage into LDS when they dequantise a tile: code times scale,
// rounded to bf16). Used where one decoding pass is cheaper than decoding
// every weight tile once per output row-tile inside the GEMM
// (stable-diffusion.rs README: weights held quantised at rest; pictor page:
// 1-bit and ternary g128 formats).
//
// One thread per 32 consecutive weights of a row (k ascending): one 16-byte
// (int4), two 16-byte (int8), one 4-byte (1-bit) or one 8-byte (ternary)
// load. Consecutive threads take consecutive 32-weight runs (of a row, then
// of the next row), so a wavefront's 64 runs are 4 KB of contiguous output.
// Each lane's 64 bytes go through LDS so that every 16-byte store
// instruction of the wavefront writes 1 KB contiguous (a lane's own 64 bytes
// stored directly would leave each instruction a quarter of 4 KB).
// HBM-bound: per weight 0.125 to 1 byte read, 2 bytes written.
#include "gemm_common.h"

namespace mmdit {

// Decodes run t (32 weights of row t / rk) and writes its 64 bytes: directly
// when wst is null, else through the wavefront's 4 KB of LDS at wst
// (all 64 lanes of the wavefront call it together).
template <int FMT>
__device__ __forceinline__ void decode_run(const char* __restrict__ w, const bf16* __restrict__ scales,
                                           bf16* __restrict__ out, int K, int rk, int64_t t, bf16x8* wst) {
  const int64_t n = t / rk;
  const int j = (int)(t - n * rk);
  bf16x8 o[4];
  if constexpr (FMT == 1) {  // int4, groups of 64: run j is bytes 16 j .. of the row
    const u32x4 v = *reinterpret_cast<const u32x4*>(w + n * (K / 2) + 16 * (int64_t)j);
    deq4(v, (float)scales[n * (K / 64) + j / 2], o);
  } else if constexpr (FMT == 2) {  // int8, groups of 64
    const u32x4* p = reinterpret_cast<const u32x4*>(w + n * K + 32 * (int64_t)j);
    const float s = (float)scales[n * (K / 64) + j / 2];
    deq8(p[0], s, o[0], o[1]);
    deq8(p[1], s, o[2], o[3]);
  } else if constexpr (FMT == 3) {  // 1 bit, groups of 128
    const uint32_t bits = *reinterpret_cast<const uint32_t*>(w + n * (K / 8) + 4 * (int64_t)j);
    const uint32_t s16 = reinterpret_cast<const uint16_t*>(scales)[n * (K / 128) + j / 4];
    deq_q1_32(bits, s16, o);
  } else {  // ternary, groups of 128
    const u32x2 v = *reinterpret_cast<const u32x2*>(w + n * (K / 4) + 8 * (int64_t)j);
    const uint32_t s16 = reinterpret_cast<const uint16_t*>(scales)[n * (K / 128) + j / 4];
    deq_tq2_32(v[0], v[1], s16, o);
  }
  if (!wst) {
    bf16x8* dst = reinterpret_cast<bf16x8*>(out + n * K + 32 * (int64_t)j);
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[u] = o[u];
    return;
  }
  // rows are whole runs, so the wavefront's 64 runs are contiguous in out
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < 4; ++u) wst[4 * lane + u] = o[u];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  bf16x8* dst = reinterpret_cast<bf16x8*>(out) + 4 * (t - lane);
#pragma unroll
  for (int u = 0; u < 4; ++u) dst[64 * u + lane] = wst[64 * u + lane];
}

template <int FMT>
__global__ __launch_bounds__(256) void k_dequant(const char* __restrict__ w, const bf16* __restrict__ scales,
                                                 bf16* __restrict__ out, int K, int64_t runs, const int* skip) {
  if (guard_skip(skip)) return;
  __shared__ bf16x8 stage[256 * 4];
  const int64_t t0 = (int64_t)blockIdx.x * 256 + (threadIdx.x & ~63);  // the wavefront's first run
  const int64_t t = t0 + (threadIdx.x & 63);
  const int rk = K / 32;  // runs per row
  if (t0 + 64 > runs) {  // last, partial wavefront: direct stores
    if (t < runs) decode_run<FMT>(w, scales, out, K, rk, t, nullptr);
    return;
  }
  decode_run<FMT>(w, scales, out, K, rk, t, stage + (threadIdx.x & ~63) * 4);
}

hipError_t launch_dequant(const void* w, const void* scales, int fmt, int N, int K, void* out, hipStream_t s,
                          const int* skip) {
  const int group = fmt == 3 || fmt == 4 ? 128 : 64;
  if (N < 0 || K <= 0 || K % group != 0 || fmt < 1 || fmt > 4) return hipErrorInvalidValue;
  const int64_t runs = (int64_t)N * (K / 32);
  if (runs == 0) return hipSuccess;
  const dim3 grid((unsigned)((runs + 255) / 256));
  const char* wp = reinterpret_cast<const char*>(w);
  const bf16* sp = reinterpret_cast<const bf16*>(scales);
  bf16* op = reinterpret_cast<bf16*>(out);
  switch (fmt) {
    case 1: hipLaunchKernelGGL(k_dequant<1>, grid, dim3(256), 0, s, wp, sp, op, K, runs, skip); break;
    case 2: hipLaunchKernelGGL(k_dequant<2>, grid, dim3(256), 0, s, wp, sp, op, K, runs, skip); break;
    case 3: hipLaunchKernelGGL(k_dequant<3>, grid, dim3(256), 0, s, wp, sp, op, K, runs, skip); break;
    default: hipLaunchKernelGGL(k_dequant<4>, grid, dim3(256), 0, s, wp, sp, op, K, runs, skip); break;
  }
  return hipGetLastError();
}

}  // namespace mmdit
