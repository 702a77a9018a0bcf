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

// Map a flat block id to (problem, tile_m, tile_n). Hardware hands out block
// ids round-robin over the 8 XCDs; the first remap makes each XCD own a
// contiguous range of logical tiles, the second walks each range in groups
// of kGroupM row-tiles so that neighbouring blocks share A rows and weight
// columns in that XCD's L2.
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_of(const GemmBatch& gb, int& prob, int& tm, int& tn) {
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  prob = bid < gb.tile_start[1] ? 0 : 1;
  const int t = bid - gb.tile_start[prob];
  const int ntn = gb.tiles_n[prob], ntm = gb.tiles_m[prob];
  const int per_group = kGroupM * ntn;
  const int group = t / per_group;
  const int first_m = group * kGroupM;
  const int gsize = ntm - first_m < kGroupM ? ntm - first_m : kGroupM;
  const int w = t - group * per_group;
  tm = first_m + w % gsize;
  tn = w / gsize;
}

}  // namespace mmdit
