// Memory-bound kernels of the MMDiT block: adaLN modulated LayerNorm, fused
// QK RMSNorm + 3D RoPE (writing the attention layout), the RoPE table, the
// modulation / conditioning GEMV, the timestep embedding, latent packing.
//
// mflux-rs, "FLUX.1 MMDiT Architecture": dual-stream and single-stream
// blocks; card "3D RoPE Coordinates": rotary axes [16, 56, 56] over the head
// dimension 128. stable-diffusion.rs README: the fused layer_norm and
// rms_norm kernels it relies on.
#include "common.h"
#include "kernels.h"

namespace mmdit {

__device__ __forceinline__ const char* seg_row(const RowSeg& s, int local, int esize) {
  int b = local / s.rows_per_batch;
  int t = local - b * s.rows_per_batch;
  return reinterpret_cast<const char*>(s.base) +
         ((int64_t)b * s.batch_stride + (int64_t)t * s.ld) * esize;
}

// ------------------------------------------------------------------ adaLN-LN --
// One wavefront per row; each lane holds h/64 values in 4-wide chunks, all
// loaded before the reductions (NC = h / 256 chunks per lane, a template
// constant so the loads are issued back to back).
template <typename TX, typename TY, int NC>
__global__ __launch_bounds__(256) void k_adaln_ln(LnArgs a, int rows) {
  if (guard_skip(a.skip)) return;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int s = r < a.seg_rows[0] ? 0 : 1;
  const int local = s == 0 ? r : r - a.seg_rows[0];
  const TX* x = reinterpret_cast<const TX*>(seg_row(a.seg[s], local, sizeof(TX)));
  const int b = local / a.seg[s].rows_per_batch;
  const float* mod = a.mod[s] + (int64_t)b * a.mod_bstride;
  const float* shift = mod + a.shift_off;
  const float* scale = mod + a.scale_off;
  float v[NC][4];
#pragma unroll
  for (int i = 0; i < NC; ++i) load4(x + (i * 64 + lane) * 4, v[i]);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) sum += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
  const float inv_h = 1.0f / (float)(NC * 256);
  const float mean = wave_sum(sum) * inv_h;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float d = v[i][j] - mean;
      sq += d * d;
    }
  const float var = wave_sum(sq) * inv_h;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  TY* y = reinterpret_cast<TY*>(a.y) + (int64_t)r * a.h;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = (i * 64 + lane) * 4;
    float sh[4], sc[4], o[4];
    load4(shift + c, sh);
    load4(scale + c, sc);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = (1.0f + sc[j]) * ((v[i][j] - mean) * rstd) + sh[j];
    store4(y + c, o);
  }
}

// R rows per 256-thread block (h a multiple of 1024) when the R rows share
// one modulation vector (same segment and batch): shift and scale are read
// once per block instead of once per row (for h 3072 they are 24 KB of
// float32 against 12 KB of x per row), the R rows' x are all requested
// before the reductions, and the R rows' sums share each block reduction.
// Blocks whose rows do not share a modulation vector, and a last partial
// block, run their rows one at a time.
template <typename TX, typename TY, int C, int R>
__global__ __launch_bounds__(256) void k_adaln_ln_rows(LnArgs a, int rows) {
  if (guard_skip(a.skip)) return;
  __shared__ float red[2][R][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * R;
  auto where = [&](int r, int& s, int& local, int& b) {
    s = r < a.seg_rows[0] ? 0 : 1;
    local = s == 0 ? r : r - a.seg_rows[0];
    b = local / a.seg[s].rows_per_batch;
  };
  int s0, l0, b0, s1, l1, b1;
  where(r0, s0, l0, b0);
  where(r0 + R - 1 < rows ? r0 + R - 1 : rows - 1, s1, l1, b1);
  const float inv_h = 1.0f / (float)(C * 1024);
  if (r0 + R <= rows && s0 == s1 && b0 == b1) {
    const float* mod = a.mod[s0] + (int64_t)b0 * a.mod_bstride;
    float v[R][C][4], sh[C][4], sc[C][4];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const TX* x = reinterpret_cast<const TX*>(seg_row(a.seg[s0], l0 + q, sizeof(TX)));
#pragma unroll
      for (int i = 0; i < C; ++i) load4(x + (i * 256 + tid) * 4, v[q][i]);
    }
#pragma unroll
    for (int i = 0; i < C; ++i) {
      load4(mod + a.shift_off + (i * 256 + tid) * 4, sh[i]);
      load4(mod + a.scale_off + (i * 256 + tid) * 4, sc[i]);
    }
    float mean[R], rstd[R];
#pragma unroll
    for (int q = 0; q < R; ++q) {
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < C; ++i) sum += (v[q][i][0] + v[q][i][1]) + (v[q][i][2] + v[q][i][3]);
      sum = wave_sum(sum);
      if (lane == 0) red[0][q][wave] = sum;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < R; ++q) {
      mean[q] = ((red[0][q][0] + red[0][q][1]) + (red[0][q][2] + red[0][q][3])) * inv_h;
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < C; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d = v[q][i][j] - mean[q];
          sq += d * d;
        }
      sq = wave_sum(sq);
      if (lane == 0) red[1][q][wave] = sq;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < R; ++q) {
      const float var = ((red[1][q][0] + red[1][q][1]) + (red[1][q][2] + red[1][q][3])) * inv_h;
      rstd[q] = 1.0f / sqrtf(var + a.eps);
      TY* y = reinterpret_cast<TY*>(a.y) + (int64_t)(r0 + q) * a.h;
#pragma unroll
      for (int i = 0; i < C; ++i) {
        float o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = (1.0f + sc[i][j]) * ((v[q][i][j] - mean[q]) * rstd[q]) + sh[i][j];
        store4(y + (i * 256 + tid) * 4, o);
      }
    }
    return;
  }
  // rows one at a time (block-uniform loop)
  for (int q = 0; q < R; ++q) {
    const int r = r0 + q;
    if (r >= rows) break;
    int s, local, b;
    where(r, s, local, b);
    const TX* x = reinterpret_cast<const TX*>(seg_row(a.seg[s], local, sizeof(TX)));
    const float* mod = a.mod[s] + (int64_t)b * a.mod_bstride;
    float v[C][4];
#pragma unroll
    for (int i = 0; i < C; ++i) load4(x + (i * 256 + tid) * 4, v[i]);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < C; ++i) sum += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
    sum = wave_sum(sum);
    if (lane == 0) red[0][0][wave] = sum;
    __syncthreads();
    const float mean = ((red[0][0][0] + red[0][0][1]) + (red[0][0][2] + red[0][0][3])) * inv_h;
    float sq = 0.f;
#pragma unroll
    for (int i = 0; i < C; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float d = v[i][j] - mean;
        sq += d * d;
      }
    sq = wave_sum(sq);
    if (lane == 0) red[1][0][wave] = sq;
    __syncthreads();
    const float var = ((red[1][0][0] + red[1][0][1]) + (red[1][0][2] + red[1][0][3])) * inv_h;
    const float rstd = 1.0f / sqrtf(var + a.eps);
    TY* y = reinterpret_cast<TY*>(a.y) + (int64_t)r * a.h;
#pragma unroll
    for (int i = 0; i < C; ++i) {
      float sh[4], sc[4], o[4];
      load4(mod + a.shift_off + (i * 256 + tid) * 4, sh);
      load4(mod + a.scale_off + (i * 256 + tid) * 4, sc);
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = (1.0f + sc[j]) * ((v[i][j] - mean) * rstd) + sh[j];
      store4(y + (i * 256 + tid) * 4, o);
    }
    __syncthreads();  // red is reused by the next row
  }
}

#ifndef MMDIT_LN_ROWS
#define MMDIT_LN_ROWS 4
#endif

template <int C>
static void launch_ln_row(const LnArgs& a, int rows, bool x_f32, bool y_bf16, hipStream_t s) {
  constexpr int R = MMDIT_LN_ROWS;
  dim3 grid((rows + R - 1) / R), block(256);
  if (x_f32 && y_bf16)
    hipLaunchKernelGGL((k_adaln_ln_rows<float, bf16, C, R>), grid, block, 0, s, a, rows);
  else if (x_f32)
    hipLaunchKernelGGL((k_adaln_ln_rows<float, float, C, R>), grid, block, 0, s, a, rows);
  else if (y_bf16)
    hipLaunchKernelGGL((k_adaln_ln_rows<bf16, bf16, C, R>), grid, block, 0, s, a, rows);
  else
    hipLaunchKernelGGL((k_adaln_ln_rows<bf16, float, C, R>), grid, block, 0, s, a, rows);
}

template <int NC>
static void launch_ln_nc(const LnArgs& a, int rows, bool x_f32, bool y_bf16, hipStream_t s) {
  dim3 grid((rows + 3) / 4), block(256);
  if (x_f32 && y_bf16)
    hipLaunchKernelGGL((k_adaln_ln<float, bf16, NC>), grid, block, 0, s, a, rows);
  else if (x_f32)
    hipLaunchKernelGGL((k_adaln_ln<float, float, NC>), grid, block, 0, s, a, rows);
  else if (y_bf16)
    hipLaunchKernelGGL((k_adaln_ln<bf16, bf16, NC>), grid, block, 0, s, a, rows);
  else
    hipLaunchKernelGGL((k_adaln_ln<bf16, float, NC>), grid, block, 0, s, a, rows);
}

// h is a multiple of 256 and at most 4096 (checked by the API).
hipError_t launch_adaln_ln(const LnArgs& a, int rows, bool x_f32, bool y_bf16, hipStream_t s) {
  if (a.h % 1024 == 0) {
    switch (a.h / 1024) {
      case 1: launch_ln_row<1>(a, rows, x_f32, y_bf16, s); break;
      case 2: launch_ln_row<2>(a, rows, x_f32, y_bf16, s); break;
      case 3: launch_ln_row<3>(a, rows, x_f32, y_bf16, s); break;
      default: launch_ln_row<4>(a, rows, x_f32, y_bf16, s); break;
    }
    return hipGetLastError();
  }
  switch (a.h / 256) {
    case 1: launch_ln_nc<1>(a, rows, x_f32, y_bf16, s); break;
    case 2: launch_ln_nc<2>(a, rows, x_f32, y_bf16, s); break;
    case 3: launch_ln_nc<3>(a, rows, x_f32, y_bf16, s); break;
    case 4: launch_ln_nc<4>(a, rows, x_f32, y_bf16, s); break;
    case 5: launch_ln_nc<5>(a, rows, x_f32, y_bf16, s); break;
    case 6: launch_ln_nc<6>(a, rows, x_f32, y_bf16, s); break;
    case 7: launch_ln_nc<7>(a, rows, x_f32, y_bf16, s); break;
    case 8: launch_ln_nc<8>(a, rows, x_f32, y_bf16, s); break;
    case 9: launch_ln_nc<9>(a, rows, x_f32, y_bf16, s); break;
    case 10: launch_ln_nc<10>(a, rows, x_f32, y_bf16, s); break;
    case 11: launch_ln_nc<11>(a, rows, x_f32, y_bf16, s); break;
    case 12: launch_ln_nc<12>(a, rows, x_f32, y_bf16, s); break;
    case 13: launch_ln_nc<13>(a, rows, x_f32, y_bf16, s); break;
    case 14: launch_ln_nc<14>(a, rows, x_f32, y_bf16, s); break;
    case 15: launch_ln_nc<15>(a, rows, x_f32, y_bf16, s); break;
    default: launch_ln_nc<16>(a, rows, x_f32, y_bf16, s); break;
  }
  return hipGetLastError();
}

// ------------------------------------------------------- step-cache indicator --
// stable-diffusion.rs README, step caching: the change of the first dual
// block's modulated image input between steps. One wavefront per row, the
// LayerNorm arithmetic of k_adaln_ln; the per-row sums are reduced on the
// host in a fixed order.
template <int NC>
__global__ __launch_bounds__(256) void k_cache_delta(CacheDeltaArgs a) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.rows) return;
  const float* x = a.x + (int64_t)r * a.h;
  const int b = r / a.rows_per_batch;
  const float* shift = a.mod + (int64_t)b * a.mod_bstride;
  const float* scale = shift + a.h;
  float v[NC][4];
#pragma unroll
  for (int i = 0; i < NC; ++i) load4(x + (i * 64 + lane) * 4, v[i]);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) sum += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
  const float inv_h = 1.0f / (float)(NC * 256);
  const float mean = wave_sum(sum) * inv_h;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float d = v[i][j] - mean;
      sq += d * d;
    }
  const float var = wave_sum(sq) * inv_h;
  const float rstd = 1.0f / sqrtf(var + a.eps);
  float* prev = a.prev + (int64_t)r * a.h;
  float dsum = 0.f, psum = 0.f;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = (i * 64 + lane) * 4;
    float sh[4], sc[4], o[4], p[4];
    load4(shift + c, sh);
    load4(scale + c, sc);
    load4(prev + c, p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = (1.0f + sc[j]) * ((v[i][j] - mean) * rstd) + sh[j];
      dsum += fabsf(o[j] - p[j]);
      psum += fabsf(p[j]);
    }
    store4(prev + c, o);
  }
  dsum = wave_sum(dsum);
  psum = wave_sum(psum);
  if (!a.first && lane == 0) {
    a.part[2 * r] = dsum;
    a.part[2 * r + 1] = psum;
  }
}

template <int NC>
static void launch_cd_nc(const CacheDeltaArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((k_cache_delta<NC>), dim3((a.rows + 3) / 4), dim3(256), 0, s, a);
}

// h is a multiple of 256 and at most 4096 (checked by the API).
hipError_t launch_cache_delta(const CacheDeltaArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  switch (a.h / 256) {
    case 1: launch_cd_nc<1>(a, s); break;
    case 2: launch_cd_nc<2>(a, s); break;
    case 3: launch_cd_nc<3>(a, s); break;
    case 4: launch_cd_nc<4>(a, s); break;
    case 5: launch_cd_nc<5>(a, s); break;
    case 6: launch_cd_nc<6>(a, s); break;
    case 7: launch_cd_nc<7>(a, s); break;
    case 8: launch_cd_nc<8>(a, s); break;
    case 9: launch_cd_nc<9>(a, s); break;
    case 10: launch_cd_nc<10>(a, s); break;
    case 11: launch_cd_nc<11>(a, s); break;
    case 12: launch_cd_nc<12>(a, s); break;
    case 13: launch_cd_nc<13>(a, s); break;
    case 14: launch_cd_nc<14>(a, s); break;
    case 15: launch_cd_nc<15>(a, s); break;
    default: launch_cd_nc<16>(a, s); break;
  }
  return hipGetLastError();
}

// y = alpha y + beta x, four floats per thread, grid-stride.
__global__ __launch_bounds__(256) void k_axpby(float4* y, const float4* x, float alpha, float beta, int64_t n4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 xv = x[i];
    float4 o;
    if (alpha == 0.f) {
      o = make_float4(beta * xv.x, beta * xv.y, beta * xv.z, beta * xv.w);
    } else {
      const float4 yv = y[i];
      o = make_float4(alpha * yv.x + beta * xv.x, alpha * yv.y + beta * xv.y, alpha * yv.z + beta * xv.z,
                      alpha * yv.w + beta * xv.w);
    }
    y[i] = o;
  }
}

hipError_t launch_axpby(float* y, const float* x, float alpha, float beta, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t want = (n4 + 255) / 256;
  const int grid = (int)(want < 2048 ? want : 2048);
  hipLaunchKernelGGL(k_axpby, dim3(grid), dim3(256), 0, s, reinterpret_cast<float4*>(y),
                     reinterpret_cast<const float4*>(x), alpha, beta, n4);
  return hipGetLastError();
}

// ------------------------------------------------- device-side cache decision --
// One 256-thread block: thread t sums rows t, t + 256, ... in order (float64),
// then a fixed-order tree over the threads; thread 0 applies the rule.
__global__ __launch_bounds__(256) void k_cache_decide(const float* __restrict__ part, int rows, int first,
                                                      double threshold, CacheState* st) {
  __shared__ double red[2][256];
  double num = 0.0, den = 0.0;
  for (int r = threadIdx.x; r < rows; r += 256) {
    num += (double)part[2 * (int64_t)r];
    den += (double)part[2 * (int64_t)r + 1];
  }
  red[0][threadIdx.x] = num;
  red[1][threadIdx.x] = den;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      red[0][threadIdx.x] += red[0][threadIdx.x + w];
      red[1][threadIdx.x] += red[1][threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x != 0) return;
  CacheState o;
  o.pad = 0;
  if (first) {
    o.skip = 0;
    o.acc = 0.0;
    o.rel = 0.0;
    o.steps = 1;
  } else {
    num = red[0][0];
    den = red[1][0];
    const double rel = den > 0.0 ? num / den : (num > 0.0 ? __builtin_inf() : 0.0);
    double acc = st->acc + rel;
    const bool run = !(acc < threshold);
    if (run) acc = 0.0;
    o.skip = run ? 0 : 1;
    o.acc = acc;
    o.rel = rel;
    o.steps = st->steps + 1;
  }
  o.ran_blocks = 1 - o.skip;
  *st = o;
}

hipError_t launch_cache_decide(const float* part, int rows, int first, double threshold, CacheState* st,
                               hipStream_t s) {
  hipLaunchKernelGGL(k_cache_decide, dim3(1), dim3(256), 0, s, part, rows, first, threshold, st);
  return hipGetLastError();
}

// mode 0: img += resid when *skip, else resid = img; mode 1: resid = img -
// resid unless *skip. Four floats per thread, grid-stride.
template <int MODE>
__global__ __launch_bounds__(256) void k_cache_apply(float4* __restrict__ img, float4* __restrict__ resid,
                                                     int64_t n4, const int* skip) {
  const bool sk = *skip != 0;
  if (MODE == 1 && sk) return;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const float4 xv = img[i];
    if (MODE == 0 && !sk) {
      resid[i] = xv;
    } else {
      const float4 rv = resid[i];
      if (MODE == 0) img[i] = make_float4(xv.x + rv.x, xv.y + rv.y, xv.z + rv.z, xv.w + rv.w);
      else resid[i] = make_float4(xv.x - rv.x, xv.y - rv.y, xv.z - rv.z, xv.w - rv.w);
    }
  }
}

template <int MODE>
static hipError_t launch_cache_apply_mode(float* img, float* resid, int64_t n, const int* skip, hipStream_t s) {
  const int64_t n4 = n / 4;
  if (n4 == 0) return hipSuccess;
  const int64_t want = (n4 + 255) / 256;
  const int grid = (int)(want < 2048 ? want : 2048);
  hipLaunchKernelGGL(k_cache_apply<MODE>, dim3(grid), dim3(256), 0, s, reinterpret_cast<float4*>(img),
                     reinterpret_cast<float4*>(resid), n4, skip);
  return hipGetLastError();
}

hipError_t launch_cache_apply(float* img, float* resid, int64_t n, const int* skip, hipStream_t s) {
  return launch_cache_apply_mode<0>(img, resid, n, skip, s);
}

hipError_t launch_cache_store(float* resid, const float* img, int64_t n, const int* skip, hipStream_t s) {
  return launch_cache_apply_mode<1>(const_cast<float*>(img), resid, n, skip, s);
}

// ----------------------------------------------------------- QK RMSNorm + RoPE --
// Block (64-token tile, head, batch), 256 threads. q and k: 16 lanes per
// token, 8 dims per lane; RMS over the 128 dims of the head, times the
// per-stream scale g, then rotation of the adjacent pairs (2j, 2j+1) by the
// table's angle. V is copied, transposed to [d, token] for the MFMA path.
// Every thread issues all of its loads (4 tokens x q, k, v and the angle
// table) before the first reduction, so 12+ 16-byte loads are in flight.
constexpr int kQkTile = 64;
constexpr int kQkPass = kQkTile / 16;
constexpr int kVPad = 130;  // LDS row stride (elements) of the V transpose tile

__device__ __forceinline__ void qk_rotate(const float (&x)[8], const float (&g)[8],
                                          const float (&cs)[8], float eps, bool valid,
                                          float (&y)[8]) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += x[i] * x[i];
  ss = group_sum<16>(ss);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float y0 = x[2 * j] * rstd * g[2 * j];
    const float y1 = x[2 * j + 1] * rstd * g[2 * j + 1];
    const float c = cs[2 * j], sn = cs[2 * j + 1];
    y[2 * j] = valid ? c * y0 - sn * y1 : 0.f;
    y[2 * j + 1] = valid ? sn * y0 + c * y1 : 0.f;
  }
}

template <typename T, bool VT>
__global__ __launch_bounds__(256) void k_qk_norm_rope(QkNormArgs a) {
  if (guard_skip(a.skip)) return;
  const int t0 = blockIdx.x * kQkTile;
  const int hh = blockIdx.y;
  const int b = blockIdx.z;
  const int h = a.H * 128;
  const int64_t head_off = ((int64_t)b * a.H + hh) * (int64_t)a.Lpad * 128;
  const int tid = threadIdx.x;
  const int d0 = (tid & 15) * 8;

  float xq[kQkPass][8], xk[kQkPass][8], xv[kQkPass][8], cs[kQkPass][8];
  float gq[2][8], gk[2][8];
  bool valid[kQkPass];
  int seg_of[kQkPass];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    load8(reinterpret_cast<const T*>(a.qn[s]) + d0, gq[s]);
    load8(reinterpret_cast<const T*>(a.kn[s]) + d0, gk[s]);
  }
#pragma unroll
  for (int p = 0; p < kQkPass; ++p) {
    const int t = t0 + p * 16 + (tid >> 4);
    valid[p] = t < a.L;
    const int s = t < a.seg_len0 ? 0 : 1;
    seg_of[p] = s;
#pragma unroll
    for (int i = 0; i < 8; ++i) xq[p][i] = xk[p][i] = xv[p][i] = cs[p][i] = 0.f;
    if (valid[p]) {
      const int local = (s == 0 ? t : t - a.seg_len0) + b * (s == 0 ? a.seg_len0 : a.L - a.seg_len0);
      const T* src = reinterpret_cast<const T*>(seg_row(a.seg[s], local, sizeof(T))) + hh * 128 + d0;
      load8(src, xq[p]);
      load8(src + h, xk[p]);
      load8(src + 2 * h, xv[p]);
      const float* tb = a.table + ((int64_t)t * 64 + (d0 >> 1)) * 2;
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(tb);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(tb + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cs[p][i] = c0[i];
        cs[p][4 + i] = c1[i];
      }
    }
  }
  T* Q = reinterpret_cast<T*>(a.Q) + head_off;
  T* K = reinterpret_cast<T*>(a.K) + head_off;
#pragma unroll
  for (int p = 0; p < kQkPass; ++p) {
    const int t = t0 + p * 16 + (tid >> 4);
    float y[8];
    qk_rotate(xq[p], seg_of[p] ? gq[1] : gq[0], cs[p], a.eps, valid[p], y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] *= a.qscale;
    if (t < a.Lpad) store8(Q + (int64_t)t * 128 + d0, y);
    qk_rotate(xk[p], seg_of[p] ? gk[1] : gk[0], cs[p], a.eps, valid[p], y);
    if (t < a.Lpad) store8(K + (int64_t)t * 128 + d0, y);
  }

  if constexpr (!VT) {
    T* V = reinterpret_cast<T*>(a.V) + head_off;
#pragma unroll
    for (int p = 0; p < kQkPass; ++p) {
      const int t = t0 + p * 16 + (tid >> 4);
      if (t < a.Lpad) store8(V + (int64_t)t * 128 + d0, xv[p]);
    }
  } else {
    __shared__ bf16 vs[kQkTile * kVPad];
#pragma unroll
    for (int p = 0; p < kQkPass; ++p) {
      const int tl = p * 16 + (tid >> 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) vs[tl * kVPad + d0 + i] = bf16(xv[p][i]);
    }
    __syncthreads();
    // Vt[b, hh, d, t0 .. t0+63]: 128 rows of 64 tokens, 8 positions per
    // thread; position p holds token vkey_pos(p) (t0 is a multiple of 16)
    bf16* Vt = reinterpret_cast<bf16*>(a.V) + head_off;
#pragma unroll
    for (int c = tid; c < 128 * (kQkTile / 8); c += 256) {
      const int d = c >> 3;
      const int tc = (c & 7) * 8;
      if (t0 + tc < a.Lpad) {
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = vs[vkey_pos(tc + i) * kVPad + d];
        *reinterpret_cast<bf16x8*>(Vt + (int64_t)d * a.Lpad + t0 + tc) = o;
      }
    }
  }
}

// One thread per (batch, head, pad row, 8 dims): Q and K rows t in [L, Lpad)
// and V^T positions p in [L & ~15, Lpad) whose token vkey_pos(p) is >= L.
__global__ void k_qkv_pad_zero(QkNormArgs a) {
  if (guard_skip(a.skip)) return;
  const int L0 = a.L & ~15;
  const int npos = a.Lpad - L0;
  const int64_t n = (int64_t)a.B * a.H * npos * 16;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int d8 = (int)(i % 16);
  const int64_t bh = i / 16 / npos;
  const int p = L0 + (int)(i / 16 % npos);
  const bf16x8 z = {};
  const int64_t head = bh * (int64_t)a.Lpad * 128;
  if (p >= a.L) {
    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.Q) + head + (int64_t)p * 128 + d8 * 8) = z;
    *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(a.K) + head + (int64_t)p * 128 + d8 * 8) = z;
  }
  if (vkey_pos(p) >= a.L) {
    bf16* vt = reinterpret_cast<bf16*>(a.V) + head;
#pragma unroll
    for (int j = 0; j < 8; ++j) vt[(int64_t)(d8 * 8 + j) * a.Lpad + p] = bf16(0.f);
  }
}

hipError_t launch_qkv_pad_zero(const QkNormArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.B * a.H * (a.Lpad - (a.L & ~15)) * 16;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_qkv_pad_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(const QkNormArgs& a, bool bf16_act, bool v_trans, hipStream_t s) {
  dim3 grid((a.Lpad + kQkTile - 1) / kQkTile, a.H, a.B), block(256);
  if (bf16_act && v_trans)
    hipLaunchKernelGGL((k_qk_norm_rope<bf16, true>), grid, block, 0, s, a);
  else if (bf16_act)
    hipLaunchKernelGGL((k_qk_norm_rope<bf16, false>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((k_qk_norm_rope<float, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- RoPE table --
// table[t, p] = (cos, sin)(ids[t, axis] * theta^(-2j / d_axis)) in float64,
// pairs p ordered axis 0, axis 1, axis 2.
__global__ void k_rope_table(const int32_t* ids, int L, int a0, int a1, int a2, double theta,
                             float* table) {
  const int np = (a0 + a1 + a2) / 2;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)L * np) return;
  const int t = (int)(i / np);
  const int p = (int)(i - (int64_t)t * np);
  int axis, j, da;
  if (p < a0 / 2) { axis = 0; j = p; da = a0; }
  else if (p < (a0 + a1) / 2) { axis = 1; j = p - a0 / 2; da = a1; }
  else { axis = 2; j = p - (a0 + a1) / 2; da = a2; }
  const double omega = pow(theta, -2.0 * (double)j / (double)da);
  const double ang = (double)ids[t * 3 + axis] * omega;
  table[i * 2] = (float)cos(ang);
  table[i * 2 + 1] = (float)sin(ang);
}

hipError_t launch_rope_table(const int32_t* ids, int L, int a0, int a1, int a2, double theta,
                             float* table, hipStream_t s) {
  const int64_t n = (int64_t)L * ((a0 + a1 + a2) / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ids, L, a0,
                     a1, a2, theta, table);
  return hipGetLastError();
}

// ---------------------------------------------------------------------- GEMV --
// y[b, n] (+)= bias[n] + sum_k W[n, k] f(x[b, k]). The input vector(s) are
// staged in LDS as float32 (after SiLU); each wavefront reduces two weight
// rows at a time with 16-byte loads along K. Up to 4 batch rows per launch.
constexpr int kGemvRowsPerWave = 2;

// Stages f(x) (SiLU or identity, float32) for B batch rows into LDS.
template <typename TX>
__device__ __forceinline__ void gemv_stage_x(float* xs, const void* x, int B, int K, int x_bstride, bool silu) {
  for (int i = threadIdx.x; i < B * K; i += 256) {
    const int bb = i / K, k = i - bb * K;
    float v = to_f32(reinterpret_cast<const TX*>(x)[(int64_t)bb * x_bstride + k]);
    xs[i] = silu ? silu_f<true>(v) : v;
  }
  __syncthreads();
}

// Rows n0 .. n0 + kGemvRowsPerWave - 1 of y[b, :] (+)= bias + W f(x[b, :]) for
// one wavefront; f(x) is staged in LDS.
template <typename TW>
__device__ __forceinline__ void gemv_rows(const float* xs, const TW* W, const TW* bias, float* y, int N, int K, int B,
                                          int y_bstride, bool accumulate, int n0, int lane) {
  constexpr int VEC = 16 / sizeof(TW);
  const int nchunk = K / VEC;
  float acc[kGemvRowsPerWave][kGemvMaxB];
#pragma unroll
  for (int r = 0; r < kGemvRowsPerWave; ++r)
#pragma unroll
    for (int bb = 0; bb < kGemvMaxB; ++bb) acc[r][bb] = 0.f;
  for (int c = lane; c < nchunk; c += 64) {
    float w[kGemvRowsPerWave][VEC];
#pragma unroll
    for (int r = 0; r < kGemvRowsPerWave; ++r) {
      const int n = n0 + r;
      if (n < N) {
        if constexpr (VEC == 8) load8(W + (int64_t)n * K + c * VEC, w[r]);
        else load4(W + (int64_t)n * K + c * VEC, w[r]);
      } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i) w[r][i] = 0.f;
      }
    }
#pragma unroll
    for (int bb = 0; bb < kGemvMaxB; ++bb) {
      if (bb < B) {
        const float* xv = xs + bb * K + c * VEC;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const float xi = xv[i];
#pragma unroll
          for (int r = 0; r < kGemvRowsPerWave; ++r) acc[r][bb] += w[r][i] * xi;
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kGemvRowsPerWave; ++r) {
#pragma unroll
    for (int bb = 0; bb < kGemvMaxB; ++bb) {
      const float v = wave_sum(acc[r][bb]);
      const int n = n0 + r;
      if (lane == 0 && bb < B && n < N) {
        float o = v + (bias ? to_f32(bias[n]) : 0.f);
        float* dst = y + (int64_t)bb * y_bstride + n;
        *dst = accumulate ? *dst + o : o;
      }
    }
  }
}

template <typename TW, typename TX>
__global__ __launch_bounds__(256) void k_gemv(GemvArgs a) {
  if (guard_skip(a.skip)) return;
  extern __shared__ float xs[];  // [B, K]
  gemv_stage_x<TX>(xs, a.x, a.B, a.K, a.x_bstride, a.silu_in);
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kGemvRowsPerWave;
  gemv_rows<TW>(xs, reinterpret_cast<const TW*>(a.W), reinterpret_cast<const TW*>(a.bias), a.y, a.N, a.K, a.B,
                a.y_bstride, a.accumulate, n0, lane);
}

// Several GEMVs over the same input in one launch (float32 or bf16 x, SiLU applied):
// block b serves the segment whose block range holds b.
template <typename TW>
__global__ __launch_bounds__(256) void k_gemv_multi(GemvMultiArgs a) {
  if (guard_skip(a.skip)) return;
  extern __shared__ float xs[];  // [B, K]
  int sg = 0;
  for (int i = 1; i < a.nseg; ++i)
    if ((int)blockIdx.x >= a.seg[i].block0) sg = i;
  const GemvSeg& g = a.seg[sg];
  if (a.x_bf16) gemv_stage_x<bf16>(xs, a.x, a.B, a.K, a.x_bstride, true);
  else gemv_stage_x<float>(xs, a.x, a.B, a.K, a.x_bstride, true);
  const int lane = threadIdx.x & 63;
  const int n0 = (((int)blockIdx.x - g.block0) * 4 + (threadIdx.x >> 6)) * kGemvRowsPerWave;
  gemv_rows<TW>(xs, reinterpret_cast<const TW*>(g.W), reinterpret_cast<const TW*>(g.bias), g.y, g.N, a.K, a.B,
                g.y_bstride, false, n0, lane);
}

// Streaming form for bf16 weights and K = 512 NCH: a wavefront owns 4 rows,
// each lane the 16-byte chunks lane + 64 c (c < NCH) of every row, and all
// 4 NCH loads of a lane are issued before the first multiply, so enough
// bytes are in flight to keep HBM busy (6.0 TB/s on the step's modulation
// shapes, against 3.7 for two rows per wavefront loaded chunk by chunk). The 4 row sums are reduced together:
// exchange across halves (lane ^ 32: two rows go each way), then across
// quarters (lane ^ 16: one row), then a butterfly over 16 lanes; lane 16 q
// ends with row q.
constexpr int kGemv4Rows = 4;
// With several batch rows, row groups of 4 x kGemv4Rows rows per block:
// SiLU(x) is staged in LDS once per block and serves all of them (one group
// per block staged it 4 times as often: at 4 batch rows, 48 KB of LDS
// traffic per 16 weight rows). One batch row keeps one group per block.
template <int BB>
constexpr int gemv4_groups() { return BB > 1 ? 4 : 1; }

template <int NCH, int BB>
__global__ __launch_bounds__(256) void k_gemv_multi4(GemvMultiArgs a) {
  if (guard_skip(a.skip)) return;
  extern __shared__ float xs[];  // [B, K]
  int sg = 0;
  for (int i = 1; i < a.nseg; ++i)
    if ((int)blockIdx.x >= a.seg[i].block0) sg = i;
  const GemvSeg& g = a.seg[sg];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int K = NCH * 512, N = g.N;
  const bf16* W = reinterpret_cast<const bf16*>(g.W);
  const bf16* bias = reinterpret_cast<const bf16*>(g.bias);
  // x first: requesting the weights ahead of the staging barrier measured
  // slower (4.1 against 6.0 TB/s on 24 x 18432 x 3072)
  // SiLU(x) staged as two halves per batch row: floats 0..3 of every
  // 8-float chunk, then floats 4..7, so that a lane's two 16-byte reads of
  // its chunk lane + 64 c are 16 bytes apart from its neighbours' (one
  // 32-byte read per lane would put 8 lanes on each bank)
  for (int i = threadIdx.x; i < BB * K; i += 256) {
    const int bb = i / K, k = i - bb * K;
    const int64_t xi = (int64_t)bb * a.x_bstride + k;
    const float v = silu_f<true>(a.x_bf16 ? (float)reinterpret_cast<const bf16*>(a.x)[xi]
                                          : reinterpret_cast<const float*>(a.x)[xi]);
    xs[bb * K + ((k >> 2) & 1) * (K / 2) + (k >> 3) * 4 + (k & 3)] = v;
  }
  __syncthreads();
  constexpr int RG = gemv4_groups<BB>();
  for (int rg = 0; rg < RG; ++rg) {
    const int n0 = ((((int)blockIdx.x - g.block0) * RG + rg) * 4 + wave) * kGemv4Rows;
    if (n0 >= N) break;  // uniform over the wavefront; no barrier follows
    bf16x8 w[kGemv4Rows][NCH];
#pragma unroll
    for (int r = 0; r < kGemv4Rows; ++r) {
      const int n = n0 + r < N ? n0 + r : N - 1;  // rows past N re-read the last row; dropped below
#pragma unroll
      for (int c = 0; c < NCH; ++c) w[r][c] = *reinterpret_cast<const bf16x8*>(W + (int64_t)n * K + (lane + 64 * c) * 8);
    }
    float acc[kGemv4Rows][BB];
#pragma unroll
    for (int r = 0; r < kGemv4Rows; ++r)
#pragma unroll
      for (int bb = 0; bb < BB; ++bb) acc[r][bb] = 0.f;
    // each weight converted once, then multiplied by every batch row (per
    // (row, batch row) the additions run over c, then i, whatever BB is)
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      float xv[BB][8];
#pragma unroll
      for (int bb = 0; bb < BB; ++bb) {
        const f32x4 x0 = *reinterpret_cast<const f32x4*>(xs + bb * K + (lane + 64 * c) * 4);
        const f32x4 x1 = *reinterpret_cast<const f32x4*>(xs + bb * K + K / 2 + (lane + 64 * c) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xv[bb][i] = x0[i];
          xv[bb][4 + i] = x1[i];
        }
      }
#pragma unroll
      for (int r = 0; r < kGemv4Rows; ++r) {
        float wf[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) wf[i] = (float)w[r][c][i];
#pragma unroll
        for (int bb = 0; bb < BB; ++bb)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[r][bb] += wf[i] * xv[bb][i];
      }
    }
    const bool hi32 = lane & 32, hi16 = lane & 16;
#pragma unroll
    for (int bb = 0; bb < BB; ++bb) {
      // halves: lanes < 32 keep rows 0, 1; lanes >= 32 keep rows 2, 3
      const float s0 = hi32 ? acc[0][bb] : acc[2][bb];
      const float s1 = hi32 ? acc[1][bb] : acc[3][bb];
      const float k0 = hi32 ? acc[2][bb] : acc[0][bb];
      const float k1 = hi32 ? acc[3][bb] : acc[1][bb];
      const float u0 = k0 + __shfl_xor(s0, 32);
      const float u1 = k1 + __shfl_xor(s1, 32);
      // quarters: lanes with bit 4 clear keep the first row of the pair
      float v = (hi16 ? u1 : u0) + __shfl_xor(hi16 ? u0 : u1, 16);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o);
      const int n = n0 + 2 * (lane >> 5) + ((lane >> 4) & 1);
      if ((lane & 15) == 0 && n < N) g.y[(int64_t)bb * g.y_bstride + n] = v + (bias ? (float)bias[n] : 0.f);
    }
  }
}

template <int NCH>
static void launch_gemv4_b(const GemvMultiArgs& a, int blocks, size_t lds, hipStream_t s) {
  switch (a.B) {
    case 1: hipLaunchKernelGGL((k_gemv_multi4<NCH, 1>), dim3(blocks), dim3(256), lds, s, a); break;
    case 2: hipLaunchKernelGGL((k_gemv_multi4<NCH, 2>), dim3(blocks), dim3(256), lds, s, a); break;
    case 3: hipLaunchKernelGGL((k_gemv_multi4<NCH, 3>), dim3(blocks), dim3(256), lds, s, a); break;
    default: hipLaunchKernelGGL((k_gemv_multi4<NCH, 4>), dim3(blocks), dim3(256), lds, s, a); break;
  }
}
// K = 512 .. 4096 in steps of 512, B = 1 .. kGemvMaxB (checked by the caller)
static void launch_gemv4_k(const GemvMultiArgs& a, int blocks, size_t lds, hipStream_t s) {
  switch (a.K / 512) {
    case 1: launch_gemv4_b<1>(a, blocks, lds, s); break;
    case 2: launch_gemv4_b<2>(a, blocks, lds, s); break;
    case 3: launch_gemv4_b<3>(a, blocks, lds, s); break;
    case 4: launch_gemv4_b<4>(a, blocks, lds, s); break;
    case 5: launch_gemv4_b<5>(a, blocks, lds, s); break;
    case 6: launch_gemv4_b<6>(a, blocks, lds, s); break;
    case 7: launch_gemv4_b<7>(a, blocks, lds, s); break;
    default: launch_gemv4_b<8>(a, blocks, lds, s); break;
  }
}

hipError_t launch_gemv_multi(const GemvMultiArgs& a0, bool w_bf16, hipStream_t s) {
  GemvMultiArgs a = a0;
  int blocks = 0;
  if (w_bf16 && a.K % 512 == 0 && a.K <= 4096 && a.B >= 1 && a.B <= kGemvMaxB) {
    const int rows_per_block = 4 * kGemv4Rows * (a.B > 1 ? gemv4_groups<2>() : gemv4_groups<1>());
    for (int i = 0; i < a.nseg; ++i) {
      a.seg[i].block0 = blocks;
      blocks += (a.seg[i].N + rows_per_block - 1) / rows_per_block;
    }
    if (blocks == 0) return hipSuccess;
    const size_t lds = (size_t)a.B * a.K * sizeof(float);
    launch_gemv4_k(a, blocks, lds, s);
    return hipGetLastError();
  }
  const int rows_per_block = 4 * kGemvRowsPerWave;
  for (int i = 0; i < a.nseg; ++i) {
    a.seg[i].block0 = blocks;
    blocks += (a.seg[i].N + rows_per_block - 1) / rows_per_block;
  }
  if (blocks == 0) return hipSuccess;
  const size_t lds = (size_t)a.B * a.K * sizeof(float);
  if (w_bf16)
    hipLaunchKernelGGL((k_gemv_multi<bf16>), dim3(blocks), dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL((k_gemv_multi<float>), dim3(blocks), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvArgs& a0, bool w_bf16, bool x_f32, hipStream_t s) {
  for (int b0 = 0; b0 < a0.B; b0 += kGemvMaxB) {
    GemvArgs a = a0;
    a.B = a0.B - b0 < kGemvMaxB ? a0.B - b0 : kGemvMaxB;
    a.x = reinterpret_cast<const char*>(a0.x) + (int64_t)b0 * a0.x_bstride * (x_f32 ? 4 : (w_bf16 ? 2 : 4));
    a.y = a0.y + (int64_t)b0 * a0.y_bstride;
    const int rows_per_block = 4 * kGemvRowsPerWave;
    dim3 grid((a.N + rows_per_block - 1) / rows_per_block), block(256);
    const size_t lds = (size_t)a.B * a.K * sizeof(float);
    if (w_bf16 && x_f32)
      hipLaunchKernelGGL((k_gemv<bf16, float>), grid, block, lds, s, a);
    else if (w_bf16)
      hipLaunchKernelGGL((k_gemv<bf16, bf16>), grid, block, lds, s, a);
    else
      hipLaunchKernelGGL((k_gemv<float, float>), grid, block, lds, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ------------------------------------------------------- timestep embedding --
// tau = 1000 sigma; f_i = exp(-ln(10000) i / half); [cos(tau f) | sin(tau f)],
// evaluated in float64.
__global__ void k_temb(float* out, int B, int dim, double sigma) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= B * dim) return;
  const int half = dim / 2;
  const int j = i % dim;
  const int k = j < half ? j : j - half;
  const double f = exp(-log(10000.0) * (double)k / (double)half);
  const double ang = 1000.0 * sigma * f;
  out[i] = (float)(j < half ? cos(ang) : sin(ang));
}

hipError_t launch_timestep_embedding(float* out, int B, int dim, double sigma, hipStream_t s) {
  hipLaunchKernelGGL(k_temb, dim3((B * dim + 255) / 256), dim3(256), 0, s, out, B, dim, sigma);
  return hipGetLastError();
}

// ------------------------------------------------------------------ packing --
// x[b, hp*Wp + wp, c*4 + ph*2 + pw] = z[b, c, 2hp + ph, 2wp + pw], raw bits.
template <typename U>
__global__ void k_pack(const U* src, U* dst, int B, int C, int H, int W, bool unpack) {
  const int64_t n = (int64_t)B * C * H * W;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  // i enumerates the packed layout [B, Hp*Wp, 4C]
  const int Hp = H / 2, Wp = W / 2, C4 = 4 * C;
  const int64_t per_b = (int64_t)Hp * Wp * C4;
  const int b = (int)(i / per_b);
  const int64_t rem = i - b * per_b;
  const int tok = (int)(rem / C4);
  const int ch = (int)(rem - (int64_t)tok * C4);
  const int hp = tok / Wp, wp = tok - (tok / Wp) * Wp;
  const int c = ch >> 2, ph = (ch >> 1) & 1, pw = ch & 1;
  const int64_t zi = (((int64_t)b * C + c) * H + (2 * hp + ph)) * W + (2 * wp + pw);
  if (unpack) dst[zi] = src[i];
  else dst[i] = src[zi];
}

hipError_t launch_pack(const void* src, void* dst, int B, int C, int H, int W, int elem_bytes,
                       bool unpack, hipStream_t s) {
  const int64_t n = (int64_t)B * C * H * W;
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(k_pack<uint16_t>, grid, block, 0, s, (const uint16_t*)src, (uint16_t*)dst,
                       B, C, H, W, unpack);
  else
    hipLaunchKernelGGL(k_pack<uint32_t>, grid, block, 0, s, (const uint32_t*)src, (uint32_t*)dst,
                       B, C, H, W, unpack);
  return hipGetLastError();
}

// ------------------------------------------------------------------ convert --
template <typename TS, typename TD>
__global__ void k_convert(const TS* src, TD* dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = from_f32<TD>(to_f32(src[i]));
}

hipError_t launch_convert(const void* src, bool src_f32, void* dst, bool dst_f32, int64_t n,
                          hipStream_t s) {
  if (n == 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (src_f32 && dst_f32)
    hipLaunchKernelGGL((k_convert<float, float>), grid, block, 0, s, (const float*)src, (float*)dst, n);
  else if (src_f32)
    hipLaunchKernelGGL((k_convert<float, bf16>), grid, block, 0, s, (const float*)src, (bf16*)dst, n);
  else if (dst_f32)
    hipLaunchKernelGGL((k_convert<bf16, float>), grid, block, 0, s, (const bf16*)src, (float*)dst, n);
  else
    hipLaunchKernelGGL((k_convert<bf16, bf16>), grid, block, 0, s, (const bf16*)src, (bf16*)dst, n);
  return hipGetLastError();
}

}  // namespace mmdit
