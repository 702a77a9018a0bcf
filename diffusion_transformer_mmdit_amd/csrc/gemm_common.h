// GEMM pieces shared by the bf16 MFMA and float32 kernels: the fused
// epilogues and the multi-problem tile map.
#pragma once
#include "common.h"
#include "kernels.h"

namespace mmdit {

struct GemmBatch {
  GemmProblem p[2];
  int32_t tiles_m[2], tiles_n[2];
  int32_t tile_start[3];
  int32_t ksplit = 1;  // k-ranges per tile (direct-to-LDS split-K)
};

template <typename TA>
__device__ __forceinline__ int64_t seg_offset(const RowSeg& s, int m) {
  const int b = m / s.rows_per_batch;
  const int t = m - b * s.rows_per_batch;
  return (int64_t)b * s.batch_stride + (int64_t)t * s.ld;
}

// Epilogue for one output element (m, n) holding the accumulated dot product.
template <int EPI, typename TA, bool PRECISE>
__device__ __forceinline__ void gemm_epilogue(const GemmProblem& P, int m, int n, float acc) {
  float v = acc;
  if (P.bias) v += to_f32(reinterpret_cast<const TA*>(P.bias)[n]);
  if constexpr (EPI == EPI_STORE) {
    if (P.out_f32) reinterpret_cast<float*>(P.out)[(int64_t)m * P.ldo + n] = v;
    else reinterpret_cast<TA*>(P.out)[(int64_t)m * P.ldo + n] = from_f32<TA>(v);
  } else if constexpr (EPI == EPI_GELU) {
    reinterpret_cast<TA*>(P.out)[(int64_t)m * P.ldo + n] = from_f32<TA>(gelu_tanh_f<PRECISE>(v));
  } else if constexpr (EPI == EPI_SPLIT) {
    if (n < P.split_n) reinterpret_cast<TA*>(P.out)[(int64_t)m * P.ldo + n] = from_f32<TA>(v);
    else reinterpret_cast<TA*>(P.out2)[(int64_t)m * P.ldo2 + (n - P.split_n)] = from_f32<TA>(gelu_tanh_f<PRECISE>(v));
  } else if constexpr (EPI == EPI_GATE_RES) {
    const int b = m / P.res_out.rows_per_batch;
    const float g = P.gate[(int64_t)b * P.gate_bstride + n];
    const int64_t oi = seg_offset<TA>(P.res_in, m) + n;
    const int64_t oo = seg_offset<TA>(P.res_out, m) + n;
    if (P.res_f32) {
      const float r = reinterpret_cast<const float*>(P.res_in.base)[oi];
      reinterpret_cast<float*>(P.res_out.base)[oo] = r + g * v;
    } else {
      const float r = to_f32(reinterpret_cast<const TA*>(P.res_in.base)[oi]);
      reinterpret_cast<TA*>(P.res_out.base)[oo] = from_f32<TA>(r + g * v);
    }
  } else if constexpr (EPI == EPI_EULER) {
    const int64_t oo = seg_offset<TA>(P.res_out, m) + n;
    float* x = reinterpret_cast<float*>(P.res_out.base);
    x[oo] = x[oo] + P.dsigma * v;
    if (P.v_out) P.v_out[(int64_t)m * P.N + n] = v;
  }
}

// Dequantise 16 int8 codes (one 16-byte load) times scale into two bf16x8.
__device__ __forceinline__ void deq8(const u32x4& w, float s, bf16x8& lo, bf16x8& hi) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = w[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float f = (float)(int8_t)(x >> (8 * j)) * s;
      if (i < 2) lo[i * 4 + j] = (bf16)f;
      else hi[(i - 2) * 4 + j] = (bf16)f;
    }
  }
}

// Dequantise 32 int4 codes (one 16-byte load; even k in the low nibble).
__device__ __forceinline__ void deq4(const u32x4& w, float s, bf16x8 out[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t x = w[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = ((int)(x << (28 - 4 * j))) >> 28;
      out[i][j] = (bf16)((float)q * s);
    }
  }
}

// Sub-byte weights, groups of 128 along k. 32 weights (k ascending) into four
// bf16x8, built as bit patterns from the bf16 scale s16 (s >= 0).
// Q1: bit j of `bits` -> weight j, 1 -> +s, 0 -> -s. Per 16-bit half x of
// the negated bits (16 weights), x | x << 15 puts the two sign bits of
// output dword i at bits 2i and 2i + 16, one shift away from bits 15 and 31.
__device__ __forceinline__ void deq_q1_32(uint32_t bits, uint32_t s16, bf16x8 out[4]) {
  const uint32_t sp = s16 | (s16 << 16);
  const uint32_t nb = ~bits;
#pragma unroll
  for (int hq = 0; hq < 2; ++hq) {
    const uint32_t x = (nb >> (16 * hq)) & 0xFFFFu;  // weights 16 hq .. 16 hq + 15
    const uint32_t x2 = x | (x << 15);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      u32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = sp | ((x2 << (15 - 2 * (4 * q + i))) & 0x80008000u);
      out[2 * hq + q] = __builtin_bit_cast(bf16x8, o);
    }
  }
}
// TQ2: the 2-bit code of weight j at bits 2j, 2j+1 of (w0 | w1 << 32);
// code 0 -> -s, 2 -> +s, 1 and 3 -> 0. Per 16-bit half x (8 codes): nz has
// bit 2j set when code j is 0 or 2, ng when it is 0; spread by 14, the flags
// of output dword i sit at bits 4i and 4i + 16, so the dword's two
// magnitudes are one 24-bit multiply of its two nz flags by the scale and
// its two signs one shift of the ng flags.
__device__ __forceinline__ void deq_tq2_32(uint32_t w0, uint32_t w1, uint32_t s16, bf16x8 out[4]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t x = ((q < 2 ? w0 : w1) >> (16 * (q & 1))) & 0xFFFFu;
    const uint32_t nx = ~x;
    const uint32_t nz = nx & 0x5555u;
    const uint32_t ng = nx & (nx >> 1) & 0x5555u;
    const uint32_t nz2 = nz | (nz << 14);
    const uint32_t ng2 = ng | (ng << 14);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t mag = __umul24((nz2 >> (4 * i)) & 0x10001u, s16);
      o[i] = mag | ((ng2 << (15 - 4 * i)) & 0x80008000u);
    }
    out[q] = __builtin_bit_cast(bf16x8, o);
  }
}

// GELU-tanh for the bf16 kernels (results are rounded to bf16 afterwards).
// With u = sqrt(2/pi) (x + 0.044715 x^3), 0.5 x (1 + tanh u) = x / (1 +
// exp(-2u)); exp(-2u) = exp2(x (a + b x^2)) with a = -2 sqrt(2/pi) log2(e),
// b = 0.044715 a. Five VALU operations plus exp2 and a reciprocal on the
// transcendental unit; no 1 - r cancellation for negative x.
__device__ __forceinline__ float gelu_fast(float x) {
  constexpr float a = -2.0f * 0.7978845608028654f * 1.4426950408889634f;
  constexpr float b = 0.044715f * a;
  const float e = __builtin_amdgcn_exp2f(x * fmaf(b, x * x, a));
  return x * __builtin_amdgcn_rcpf(e + 1.0f);
}

// Epilogue of one 32x32 MFMA accumulator block held by a lane: 16 rows
// row(r) = mb + 8 (r / 4) + r % 4 of column n. Column constants (bias, gate)
// come in precomputed. `fast` is true when every row of the block tile lies
// in one batch and the residual rows are contiguous (rows_per_batch >= M);
// otherwise each element takes the generic path. For EPI_SPLIT, `split_side`
// is 0 (all columns of the tile before split_n), 1 (all after) or 2 (mixed).
// GENERAL = false compiles out the per-element fallbacks (the caller
// guarantees fast == true and split_side != 2).
template <int EPI, bool GENERAL>
__device__ __forceinline__ void epi_block_bf16(const GemmProblem& P, int mb, int n, const f32x16& acc,
                                               float bias, float gate, bool fast, int split_side) {
  const int M = P.M;
  if constexpr (EPI == EPI_STORE) {
    if (P.out_f32) {
      float* o = reinterpret_cast<float*>(P.out);
      const int ld = (int)P.ldo;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r >> 2) + (r & 3);
        if (m < M) o[m * ld + n] = acc[r] + bias;
      }
    } else {
      bf16* o = reinterpret_cast<bf16*>(P.out);
      const int ld = (int)P.ldo;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r >> 2) + (r & 3);
        if (m < M) o[m * ld + n] = (bf16)(acc[r] + bias);
      }
    }
  } else if constexpr (EPI == EPI_GELU || EPI == EPI_SPLIT) {
    if (GENERAL && EPI == EPI_SPLIT && split_side == 2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r >> 2) + (r & 3);
        if (m < M) gemm_epilogue<EPI_SPLIT, bf16, false>(P, m, n, acc[r]);
      }
      return;
    }
    const bool to2 = EPI == EPI_SPLIT && split_side == 1;
    const bool gelu = EPI == EPI_GELU || to2;
    bf16* o = reinterpret_cast<bf16*>(to2 ? P.out2 : P.out);
    const int ld = (int)(to2 ? P.ldo2 : P.ldo);
    const int col = to2 ? n - P.split_n : n;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mb + 8 * (r >> 2) + (r & 3);
      float v = acc[r] + bias;
      if (gelu) v = gelu_fast(v);
      if (m < M) o[m * ld + col] = (bf16)v;
    }
  } else if constexpr (EPI == EPI_GATE_RES) {
    if (GENERAL && !fast) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r >> 2) + (r & 3);
        if (m < M) gemm_epilogue<EPI_GATE_RES, bf16, false>(P, m, n, acc[r]);
      }
      return;
    }
    const int ldi = P.res_in.ld, ldo = P.res_out.ld;
    if (P.res_f32) {
      const float* __restrict__ ri = reinterpret_cast<const float*>(P.res_in.base);
      float* __restrict__ ro = reinterpret_cast<float*>(P.res_out.base);
      float rv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int m = mb + 8 * (r >> 2) + (r & 3);
        m = m < M ? m : M - 1;
        rv[r] = ri[m * ldi + n];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r >> 2) + (r & 3);
        if (m < M) ro[m * ldo + n] = rv[r] + gate * (acc[r] + bias);
      }
    } else {
      const bf16* __restrict__ ri = reinterpret_cast<const bf16*>(P.res_in.base);
      bf16* __restrict__ ro = reinterpret_cast<bf16*>(P.res_out.base);
      float rv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int m = mb + 8 * (r >> 2) + (r & 3);
        m = m < M ? m : M - 1;
        rv[r] = (float)ri[m * ldi + n];
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = mb + 8 * (r >> 2) + (r & 3);
        if (m < M) ro[m * ldo + n] = (bf16)(rv[r] + gate * (acc[r] + bias));
      }
    }
    // keep the next block's residual reads below these stores (bounds the
    // number of values in flight, and so the registers)
    asm volatile("" ::: "memory");
  } else {  // EPI_EULER (float32 latent)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = mb + 8 * (r >> 2) + (r & 3);
      if (m < M) gemm_epilogue<EPI_EULER, bf16, false>(P, m, n, acc[r]);
    }
  }
}

// Batch index shared by all rows [m0, m0 + rows) of a tile when the
// residual rows are contiguous (one batch, or rows_per_batch >= M), else -1.
__device__ __forceinline__ int tile_batch(const GemmProblem& P, int m0, int rows) {
  const int rpb = P.res_out.rows_per_batch;
  if (rpb <= 0) return 0;
  if (P.res_in.rows_per_batch < P.M || rpb < P.M) return -1;
  return 0;
}

// Which side of split_n the columns [n0, n0 + cols) fall on: 0, 1, or 2 (both).
__device__ __forceinline__ int split_side_of(const GemmProblem& P, int n0, int cols) {
  if (n0 + cols <= P.split_n) return 0;
  if (n0 >= P.split_n) return 1;
  return 2;
}

// Map a flat block id to (problem, tile_m, tile_n). Hardware hands out block
// ids round-robin over the 8 XCDs; the first remap makes each XCD own a
// contiguous range of logical tiles, the second walks each range in groups
// of kGroupM row-tiles so that neighbouring blocks share A rows and weight
// columns in that XCD's L2.
#ifndef MMDIT_GEMM_GROUP_M
#define MMDIT_GEMM_GROUP_M 6
#endif
constexpr int kGroupM = MMDIT_GEMM_GROUP_M;

// Coordinates of logical tile `t` (problems concatenated, each walked in
// groups of kGroupM row-tiles).
__device__ __forceinline__ void tile_coords(const GemmBatch& gb, int t, int& prob, int& tm, int& tn) {
  prob = t < gb.tile_start[1] ? 0 : 1;
  t -= gb.tile_start[prob];
  const int ntn = gb.tiles_n[prob], ntm = gb.tiles_m[prob];
  const int per_group = kGroupM * ntn;
  const int group = t / per_group;
  const int first_m = group * kGroupM;
  const int gsize = ntm - first_m < kGroupM ? ntm - first_m : kGroupM;
  const int w = t - group * per_group;
  tm = first_m + w % gsize;
  tn = w / gsize;
}

__device__ __forceinline__ void tile_of(const GemmBatch& gb, int& prob, int& tm, int& tn) {
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  tile_coords(gb, bid, prob, tm, tn);
}

}  // namespace mmdit
