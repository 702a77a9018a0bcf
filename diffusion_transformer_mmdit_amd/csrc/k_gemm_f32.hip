// float32 GEMM C = A W^T for the float32 configuration: true fp32 FMA on the
// vector ALUs (no reduced-precision matrix path), 64x64 block tile, K-tile
// 16 staged in LDS, 4x4 outputs per thread, the same fused epilogues as the
// bf16 kernel (with the library expf in GELU).
#include "gemm_common.h"

namespace mmdit {

constexpr int kF32T = 64;
constexpr int kF32K = 16;

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_f32(GemmBatch gb) {
  if (guard_skip(gb.p[0].skip)) return;
  __shared__ float As[kF32K][kF32T + 4];
  __shared__ float Bs[kF32K][kF32T + 4];
  int prob, tm, tn;
  tile_of(gb, prob, tm, tn);
  const GemmProblem& P = gb.p[prob];
  const int M = P.M, N = P.N, K = P.K;
  const int m0 = tm * kF32T, n0 = tn * kF32T;
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const float* A = reinterpret_cast<const float*>(P.A);
  const float* W = reinterpret_cast<const float*>(P.W);
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += kF32K) {
    // 64 rows x 16 k of A and of W: 4 values per thread each
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * 256;
      const int row = e >> 4, kk = e & 15;
      const int gm = m0 + row, gn = n0 + row, gk = k0 + kk;
      As[kk][row] = (gm < M && gk < K) ? A[(int64_t)gm * P.lda + gk] : 0.f;
      Bs[kk][row] = (gn < N && gk < K) ? W[(int64_t)gn * K + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kF32K; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][ty * 4 + i];
        b[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + ty * 4 + i, n = n0 + tx * 4 + j;
      if (m < M && n < N) gemm_epilogue<EPI, float, true>(P, m, n, acc[i][j]);
    }
}

template <int EPI>
static hipError_t launch_f32(const GemmProblem* p, int nprob, hipStream_t s) {
  GemmBatch gb{};
  int total = 0;
  for (int i = 0; i < 2; ++i) {
    if (i < nprob) {
      gb.p[i] = p[i];
      gb.tiles_m[i] = (p[i].M + kF32T - 1) / kF32T;
      gb.tiles_n[i] = (p[i].N + kF32T - 1) / kF32T;
      total += gb.tiles_m[i] * gb.tiles_n[i];
    } else {
      gb.tiles_m[i] = 1;
      gb.tiles_n[i] = 1;
    }
    gb.tile_start[i + 1] = total;
  }
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_gemm_f32<EPI>, dim3(total), dim3(256), 0, s, gb);
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmProblem* p, int nprob, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_f32<EPI_STORE>(p, nprob, s);
    case EPI_GELU: return launch_f32<EPI_GELU>(p, nprob, s);
    case EPI_GATE_RES: return launch_f32<EPI_GATE_RES>(p, nprob, s);
    case EPI_SPLIT: return launch_f32<EPI_SPLIT>(p, nprob, s);
    case EPI_EULER: return launch_f32<EPI_EULER>(p, nprob, s);
    default: return hipErrorInvalidValue;  // fused QK epilogues: bf16 only
  }
}

}  // namespace mmdit
