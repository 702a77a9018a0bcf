// Weight-streaming linear layer for a few rows (M <= 16, bf16 activations):
// y[m, n] = sum_k x[m, k] W[n, k] + b[n]. With so few rows every weight is
// used at most 16 times, so the layer is bound by reading W once from HBM
// (stable-diffusion.rs README: weights held quantised at rest and
// dequantised inside the matmul; here the codes are decoded in registers,
// never stored).
//
// One 512-thread block owns NC groups of 16 output columns; its 8
// wavefronts split k (wavefront w takes the 128-wide k blocks w, w + 8, ...)
// and each computes its 16 x 16 products on v_mfma_f32_16x16x32_bf16 (x
// rows as the A operand: lanes of rows >= M read row 0, whose output rows
// are never stored; weight rows as B). One set of x fragments serves the NC
// column groups. A wavefront requests the codes and x fragments of CH k
// blocks before decoding the first; the 8 partial products are summed in LDS
// in a fixed order. NC and CH per format were chosen by measurement (the
// register count sets how many wavefronts a CU holds, and with them the
// bytes in flight).
//
// Which k a lane holds in MFMA step s (0..3), lane group g = lane / 16:
//   dense: k = 32 s + 8 g + i, so the 4 lanes of a weight row read 64
//   contiguous bytes per load;
//   8-bit: k = 64 (s / 2) + 16 g + 8 (s % 2) + i: two 16-byte loads, each in
//   one scale group;
//   4-bit: k = 32 g + 8 s + i, one 16-byte load (64 contiguous bytes per
//   row); 1-bit and ternary likewise (4 and 8 bytes).
//
// 4-bit weights (groups of 64): a dword of 8 codes (q_0 .. q_7, low nibble
// first) becomes four bf16 pairs with two bit operations each: u = code ^ 8
// = q + 8 in 0..15, and the bf16 bit pattern 0x4300 | u is exactly 128 + u =
// 136 + q; the pairs hold (q_j, q_j+4), and the x fragment is permuted to the
// same order. Lane groups 0, 1 hold scale group 0 of the k block and lane
// groups 2, 3 group 1, so each step runs twice, with the A operand zeroed in
// the other group's lanes. Each group's sum starts from -136 sum_k x (MFMAs
// against a constant -136 operand, shared by the column groups), so it is
// sum_k q_k x_k, and the group scale multiplies that float32 sum: s q is
// never rounded to bf16, unlike the tiled kernels, which multiply bf16(s q).
// The other formats are decoded with their scale by the GEMM decoders.
#include "gemm_common.h"

namespace mmdit {

constexpr int kStWaves = 8;

template <int FMT> struct StCfg;
template <> struct StCfg<0> { static constexpr int NC = 2, CH = 2; };  // dense: 64 B per lane and k block
template <> struct StCfg<1> { static constexpr int NC = 3, CH = 1; };  // 4-bit: 16 B
template <> struct StCfg<2> { static constexpr int NC = 4, CH = 1; };  // 8-bit: 32 B
template <> struct StCfg<3> { static constexpr int NC = 4, CH = 2; };  // 1-bit: 4 B
template <> struct StCfg<4> { static constexpr int NC = 4, CH = 2; };  // ternary: 8 B

template <int FMT> struct SkCodes;
template <> struct SkCodes<0> { u32x4 v[4]; };   // 32 bf16
template <> struct SkCodes<1> { u32x4 v; };      // 32 nibbles
template <> struct SkCodes<2> { u32x4 v[2]; };   // 32 int8
template <> struct SkCodes<3> { uint32_t v; };   // 32 bits
template <> struct SkCodes<4> { uint32_t v[2]; };  // 32 x 2 bits

// k offset, inside the 128-wide block, of lane group g's x fragment in step s
template <int FMT>
__device__ __forceinline__ int sk_xoff(int g, int s) {
  if constexpr (FMT == 0) return 32 * s + 8 * g;
  else if constexpr (FMT == 2) return 64 * (s >> 1) + 16 * g + 8 * (s & 1);
  else return 32 * g + 8 * s;
}

// codes (and scale bits) of weight row n for k block blk, lane group g
template <int FMT>
__device__ __forceinline__ void sk_load(SkCodes<FMT>& c, const char* W, const uint16_t* S, int64_t n, int K, int blk,
                                        int g, uint32_t& sc) {
  if constexpr (FMT == 0) {
    const char* row = W + (n * K + blk * 128) * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) c.v[i] = *reinterpret_cast<const u32x4*>(row + 64 * i + 16 * g);
    sc = 0;
  } else if constexpr (FMT == 1) {
    c.v = *reinterpret_cast<const u32x4*>(W + n * (K / 2) + blk * 64 + 16 * g);
    sc = *reinterpret_cast<const uint32_t*>(S + n * (K / 64) + 2 * blk);  // groups 2 blk, 2 blk + 1
  } else if constexpr (FMT == 2) {
    const char* row = W + n * K + blk * 128;
    c.v[0] = *reinterpret_cast<const u32x4*>(row + 16 * g);       // group 2 blk
    c.v[1] = *reinterpret_cast<const u32x4*>(row + 64 + 16 * g);  // group 2 blk + 1
    sc = *reinterpret_cast<const uint32_t*>(S + n * (K / 64) + 2 * blk);
  } else if constexpr (FMT == 3) {
    c.v = *reinterpret_cast<const uint32_t*>(W + n * (K / 8) + blk * 16 + 4 * g);
    sc = S[n * (K / 128) + blk];
  } else {
    const u32x2 v = *reinterpret_cast<const u32x2*>(W + n * (K / 4) + blk * 32 + 8 * g);
    c.v[0] = v[0];
    c.v[1] = v[1];
    sc = S[n * (K / 128) + blk];
  }
}

// 8 weights of one code dword (4-bit, ^ 8 applied) as bf16 136 + q in the
// order (q_0, q_4, q_1, q_5, q_2, q_6, q_3, q_7)
__device__ __forceinline__ bf16x8 sk_q4_offset(uint32_t u) {
  u32x4 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = ((u >> (4 * j)) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, o);
}

// x fragment (x_0 .. x_7) in the order of sk_q4_offset
__device__ __forceinline__ bf16x8 sk_q4_xperm(const u32x4& d) {
  const u32x4 p = {__builtin_amdgcn_perm(d[2], d[0], 0x05040100u), __builtin_amdgcn_perm(d[2], d[0], 0x07060302u),
                   __builtin_amdgcn_perm(d[3], d[1], 0x05040100u), __builtin_amdgcn_perm(d[3], d[1], 0x07060302u)};
  return __builtin_bit_cast(bf16x8, p);
}

// One k block of NC column groups: acc[c] += x_block W_block^T.
template <int FMT, int NC>
__device__ __forceinline__ void sk_block(const SkCodes<FMT> (&cd)[NC], const uint32_t (&sc)[NC], const u32x4 (&xf)[4],
                                         f32x4 (&acc)[NC], int g) {
  if constexpr (FMT == 1) {
    const bf16x8 m136 = __builtin_bit_cast(bf16x8, (u32x4){0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u});
    bf16x8 ah[2][4];  // the x fragments, zero outside scale group h's lanes
    const bool lo = g < 2;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 v = __builtin_bit_cast(u32x4, sk_q4_xperm(xf[s]));
      const u32x4 z = {0u, 0u, 0u, 0u};
      ah[0][s] = __builtin_bit_cast(bf16x8, lo ? v : z);
      ah[1][s] = __builtin_bit_cast(bf16x8, lo ? z : v);
    }
    f32x4 corr[2];  // -136 sum_k x over each scale group
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      corr[h] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) corr[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[h][s], m136, corr[h], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 bq[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) bq[s] = sk_q4_offset(cd[c].v[s] ^ 0x88888888u);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 ga = corr[h];
#pragma unroll
        for (int s = 0; s < 4; ++s) ga = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[h][s], bq[s], ga, 0, 0, 0);
        const float sv = __builtin_bit_cast(float, h ? (sc[c] & 0xFFFF0000u) : (sc[c] << 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[c][i] = fmaf(sv, ga[i], acc[c][i]);
      }
    }
  } else {
    bf16x8 a[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = __builtin_bit_cast(bf16x8, xf[s]);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      bf16x8 b[4];
      if constexpr (FMT == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = __builtin_bit_cast(bf16x8, cd[c].v[i]);
      } else if constexpr (FMT == 2) {
        deq8(cd[c].v[0], __builtin_bit_cast(float, sc[c] << 16), b[0], b[1]);
        deq8(cd[c].v[1], __builtin_bit_cast(float, sc[c] & 0xFFFF0000u), b[2], b[3]);
      } else if constexpr (FMT == 3) {
        deq_q1_32(cd[c].v, sc[c], b);
      } else {
        deq_tq2_32(cd[c].v[0], cd[c].v[1], sc[c], b);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[s], acc[c], 0, 0, 0);
    }
  }
}

// Y_F32: y is float32 (else bf16). K % 128 == 0, M in [1, 16].
// At most 128 registers per lane: 4 wavefronts per SIMD, two blocks per CU.
template <int FMT, bool Y_F32>
__global__ __launch_bounds__(64 * kStWaves) __attribute__((amdgpu_waves_per_eu(4))) void k_linear_skinny(const bf16* __restrict__ x, int M,
                                                                 const char* __restrict__ W,
                                                                 const uint16_t* __restrict__ S,
                                                                 const bf16* __restrict__ bias,
                                                                 void* __restrict__ y, int N, int K) {
  constexpr int NC = StCfg<FMT>::NC, CH = StCfg<FMT>::CH;
  __shared__ f32x4 red[kStWaves][NC][64];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int r = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 16 * NC;
  int64_t nrow[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int n = n0 + 16 * c + r;
    nrow[c] = n < N ? n : N - 1;  // columns past N read a valid row; their outputs are dropped
  }
  const bf16* xr = x + (int64_t)(r < M ? r : 0) * K;
  const int nblk = K / 128;
  f32x4 acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int b0 = wave; b0 < nblk; b0 += kStWaves * CH) {
    // every load of the chunk's k blocks b0, b0 + 8, ... before any decode
    // (branches on blk are uniform over the wavefront)
    SkCodes<FMT> cd[CH][NC];
    uint32_t sc[CH][NC];
    u32x4 xf[CH][4];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int blk = b0 + kStWaves * j;
      if (blk < nblk) {
#pragma unroll
        for (int c = 0; c < NC; ++c) sk_load<FMT>(cd[j][c], W, S, nrow[c], K, blk, g, sc[j][c]);
#pragma unroll
        for (int s = 0; s < 4; ++s) xf[j][s] = *reinterpret_cast<const u32x4*>(xr + blk * 128 + sk_xoff<FMT>(g, s));
      }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j)
      if (b0 + kStWaves * j < nblk) sk_block<FMT, NC>(cd[j], sc[j], xf[j], acc, g);
  }
  // acc[c][i] = partial C[m = 4 g + i][n0 + 16 c + r]; wavefront c sums
  // column group c over the 8 wavefronts in order
#pragma unroll
  for (int c = 0; c < NC; ++c) red[wave][c][lane] = acc[c];
  __syncthreads();
  if (wave < NC) {
    const int c = wave;
    f32x4 t = red[0][c][lane];
#pragma unroll
    for (int w = 1; w < kStWaves; ++w) {
      const f32x4 u = red[w][c][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) t[i] += u[i];
    }
    const int nn = n0 + 16 * c + r;
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
  const dim3 grid((N + 16 * StCfg<FMT>::NC - 1) / (16 * StCfg<FMT>::NC));
  if (y_f32)
    hipLaunchKernelGGL((k_linear_skinny<FMT, true>), grid, dim3(64 * kStWaves), 0, s, x, M, (const char*)W,
                       (const uint16_t*)S, (const bf16*)bias, y, N, K);
  else
    hipLaunchKernelGGL((k_linear_skinny<FMT, false>), grid, dim3(64 * kStWaves), 0, s, x, M, (const char*)W,
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
