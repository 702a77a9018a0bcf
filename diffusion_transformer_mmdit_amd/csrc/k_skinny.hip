// Weight-streaming linear layer for a few rows (M <= 16, bf16 activations):
// y[m, n] = sum_k x[m, k] W[n, k] + b[n]. With so few rows every weight is
// used at most 16 times, so the layer is bound by reading W once from HBM
// (stable-diffusion.rs README: weights held quantised at rest and
// dequantised inside the matmul; here the codes are decoded in registers,
// never stored).
//
// One 256-thread block owns 16 output columns n0 .. n0+15 (16 weight rows);
// its 4 wavefronts take every fourth 128-wide k block and each computes the
// 16 x 16 product on v_mfma_f32_16x16x32_bf16 (x rows as the A operand, zero
// past M; weight rows as B). The k order inside a 128-block is permuted the
// same way for A and B: in MFMA step s (0..3) lane group g = lane / 16 holds
// k = 32 g + 8 s + i (i = 0..7), so over the four steps a lane reads 32
// consecutive k of one weight row: one 16-byte load of 4-bit codes (32 B of
// 8-bit codes, 4 B of 1-bit, 8 B of ternary, 64 B dense), inside one scale
// group. All of a wavefront's weight loads are issued before the first MFMA.
// The four partial 16 x 16 products are summed in LDS in a fixed order.
#include "gemm_common.h"

namespace mmdit {

template <int FMT>
struct SkCodes;
template <> struct SkCodes<0> { u32x4 v[4]; };   // 32 bf16
template <> struct SkCodes<1> { u32x4 v[1]; };   // 32 nibbles
template <> struct SkCodes<2> { u32x4 v[2]; };   // 32 int8
template <> struct SkCodes<3> { uint32_t v; };   // 32 bits
template <> struct SkCodes<4> { uint32_t v[2]; };  // 32 x 2 bits

// 128-wide k blocks a wavefront holds in flight at once: their codes and the
// matching x fragments (16 registers per block) are all requested before the
// first of them is decoded
template <int FMT>
constexpr int sk_chunk() { return FMT == 0 || FMT == 2 ? 4 : 8; }

template <int FMT>
__device__ __forceinline__ void sk_load(SkCodes<FMT>& c, const char* W, const uint16_t* S, int64_t n, int K, int k0,
                                        uint32_t& s16) {
  // k0: first of the lane's 32 consecutive k
  if constexpr (FMT == 0) {
    const u32x4* p = reinterpret_cast<const u32x4*>(W + (n * K + k0) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i) c.v[i] = p[i];
    s16 = 0;
  } else if constexpr (FMT == 1) {
    c.v[0] = *reinterpret_cast<const u32x4*>(W + n * (K / 2) + k0 / 2);
    s16 = S[n * (K / 64) + k0 / 64];
  } else if constexpr (FMT == 2) {
    const u32x4* p = reinterpret_cast<const u32x4*>(W + n * K + k0);
    c.v[0] = p[0];
    c.v[1] = p[1];
    s16 = S[n * (K / 64) + k0 / 64];
  } else if constexpr (FMT == 3) {
    c.v = *reinterpret_cast<const uint32_t*>(W + n * (K / 8) + k0 / 8);
    s16 = S[n * (K / 128) + k0 / 128];
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(W + n * (K / 4) + k0 / 4);
    c.v[0] = v.x;
    c.v[1] = v.y;
    s16 = S[n * (K / 128) + k0 / 128];
  }
}

// The lane's 32 weights as the B fragments of the four MFMA steps.
template <int FMT>
__device__ __forceinline__ void sk_decode(const SkCodes<FMT>& c, uint32_t s16, bf16x8 (&b)[4]) {
  if constexpr (FMT == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) b[i] = __builtin_bit_cast(bf16x8, c.v[i]);
  } else if constexpr (FMT == 1) {
    deq4(c.v[0], __builtin_bit_cast(float, s16 << 16), b);
  } else if constexpr (FMT == 2) {
    const float s = __builtin_bit_cast(float, s16 << 16);
    deq8(c.v[0], s, b[0], b[1]);
    deq8(c.v[1], s, b[2], b[3]);
  } else if constexpr (FMT == 3) {
    deq_q1_32(c.v, s16, b);
  } else {
    deq_tq2_32(c.v[0], c.v[1], s16, b);
  }
}

// Y_F32: y is float32 (else bf16). K % 128 == 0, M in [1, 16].
template <int FMT, bool Y_F32>
__global__ __launch_bounds__(256) void k_linear_skinny(const bf16* __restrict__ x, int M, const char* __restrict__ W,
                                                       const uint16_t* __restrict__ S, const bf16* __restrict__ bias,
                                                       void* __restrict__ y, int N, int K) {
  __shared__ f32x4 red[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16;
  int64_t n = n0 + r;
  n = n < N ? n : N - 1;  // columns past N read a valid row; their outputs are dropped
  const bool row_ok = r < M;
  const bf16* xr = x + (int64_t)(row_ok ? r : 0) * K;
  const int nblk = K / 128;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  constexpr int CH = sk_chunk<FMT>();
  for (int b0 = wave; b0 < nblk; b0 += 4 * CH) {
    // this wavefront's k blocks b0, b0 + 4, ... (up to CH of them)
    SkCodes<FMT> codes[CH];
    uint32_t sc[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int blk = b0 + 4 * j;
      if (blk < nblk) sk_load<FMT>(codes[j], W, S, n, K, blk * 128 + 32 * g, sc[j]);
    }
    // x fragments one block ahead of their MFMAs
    auto load_x = [&](int blk, bf16x8 (&af)[4]) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        af[s] = (bf16x8){};
        if (row_ok && blk < nblk) af[s] = *reinterpret_cast<const bf16x8*>(xr + blk * 128 + 32 * g + 8 * s);
      }
    };
    bf16x8 af[2][4];
    load_x(b0, af[0]);
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int blk = b0 + 4 * j;
      if (j + 1 < CH) load_x(blk + 4, af[(j + 1) & 1]);
      if (blk < nblk) {
        bf16x8 bf[4];
        sk_decode<FMT>(codes[j], sc[j], bf);
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j & 1][s], bf[s], acc, 0, 0, 0);
      }
    }
  }
  // acc[i] = partial C[m = 4 g + i][n0 + r]
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 t = red[0][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const f32x4 u = red[w][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] += u[i];
    }
    const int nn = n0 + r;
    if (nn < N) {
      const float bv = bias ? (float)bias[nn] : 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < M) {
          if constexpr (Y_F32) reinterpret_cast<float*>(y)[(int64_t)m * N + nn] = t[i] + bv;
          else reinterpret_cast<bf16*>(y)[(int64_t)m * N + nn] = (bf16)(t[i] + bv);
        }
      }
    }
  }
}

template <int FMT>
static hipError_t launch_skinny_fmt(const bf16* x, int M, const void* W, const void* S, const void* bias, void* y,
                                    bool y_f32, int N, int K, hipStream_t s) {
  const dim3 grid((N + 15) / 16);
  if (y_f32)
    hipLaunchKernelGGL((k_linear_skinny<FMT, true>), grid, dim3(256), 0, s, x, M, (const char*)W,
                       (const uint16_t*)S, (const bf16*)bias, y, N, K);
  else
    hipLaunchKernelGGL((k_linear_skinny<FMT, false>), grid, dim3(256), 0, s, x, M, (const char*)W,
                       (const uint16_t*)S, (const bf16*)bias, y, N, K);
  return hipGetLastError();
}

hipError_t launch_linear_skinny(const void* x, int M, const void* W, const void* scales, const void* bias, int fmt,
                                void* y, bool y_f32, int N, int K, hipStream_t s) {
  const bf16* xb = reinterpret_cast<const bf16*>(x);
  switch (fmt) {
    case 0: return launch_skinny_fmt<0>(xb, M, W, scales, bias, y, y_f32, N, K, s);
    case 1: return launch_skinny_fmt<1>(xb, M, W, scales, bias, y, y_f32, N, K, s);
    case 2: return launch_skinny_fmt<2>(xb, M, W, scales, bias, y, y_f32, N, K, s);
    case 3: return launch_skinny_fmt<3>(xb, M, W, scales, bias, y, y_f32, N, K, s);
    case 4: return launch_skinny_fmt<4>(xb, M, W, scales, bias, y, y_f32, N, K, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace mmdit
