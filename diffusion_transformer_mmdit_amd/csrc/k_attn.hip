// Joint softmax attention over the concatenated [text; image] tokens, no
// mask, scale 1/sqrt(d) (mflux-rs card "Dual-Stream MMDiT": bidirectional
// attention between the two streams; card "Single-Stream Blocks": one
// self-attention sequence; stable-diffusion.rs README: the fused
// scaled_dot_product_attention it relies on).
//
// bf16 path (flash attention, gfx950 MFMA 32x32x16):
//  * a block owns 128 queries of one (batch, head); each of its 4 wavefronts
//    owns 32 queries; K and V^T tiles of 64 keys are staged in LDS, double
//    buffered, and shared by the 4 wavefronts;
//  * S^T = K Q^T is computed so that each lane holds the scores of ONE query
//    (its MFMA column): the running max needs one cross-lane exchange and the
//    running sum none until the end;
//  * the probabilities stay in registers and feed O^T += V^T P^T directly as
//    the MFMA B operand: no LDS round trip for P. V arrives transposed
//    ([d, token]) from the QK-norm kernel so the A operand reads are 8-byte
//    row segments;
//  * online softmax in float32 with exp2 of log2(e)-scaled scores; the
//    running max is moved only when it grows by more than 2^8.
#include "common.h"
#include "kernels.h"

namespace mmdit {

constexpr int kAttnQ = 128;   // queries per block
constexpr int kAttnK = 64;    // keys per tile
constexpr int kKPad = 136;    // K tile row stride (elements)
constexpr int kVPadT = 72;    // V^T tile row stride (elements): 16-byte aligned rows

// Position of key k (within a 64-key tile) in a V^T tile row: bits 2 and 3
// swapped, i.e. within each group of 16 keys the order is 0-3, 8-11, 4-7,
// 12-15.
__device__ __forceinline__ int vkey_pos(int k) {
  return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1);
}

__device__ __forceinline__ bf16* out_row(const AttnArgs& a, int b, int t) {
  const int s = t < a.seg_len0 ? 0 : 1;
  const RowSeg& g = a.out[s];
  const int local_t = s == 0 ? t : t - a.seg_len0;
  return reinterpret_cast<bf16*>(g.base) + (int64_t)b * g.batch_stride + (int64_t)local_t * g.ld;
}

__global__ __launch_bounds__(256, 2) void k_attn_bf16(AttnArgs a) {
  __shared__ bf16 Ks[2][kAttnK * kKPad];
  __shared__ bf16 Vs[2][128 * kVPadT];
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const int q0 = blockIdx.x * kAttnQ;
  const int hh = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.H + hh;
  const bf16* Qh = reinterpret_cast<const bf16*>(a.Q) + bh * a.Lpad * 128;
  const bf16* Kh = reinterpret_cast<const bf16*>(a.K) + bh * a.Lpad * 128;
  const bf16* Vh = reinterpret_cast<const bf16*>(a.V) + bh * 128 * (int64_t)a.Lpad;

  // Q as the B operand of S^T = K Q^T: column = query, 8 consecutive dims.
  const int qrow = q0 + wave * 32 + l32;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)qrow * 128 + kk * 16 + g * 8);

  const int ntiles = (a.L + kAttnK - 1) / kAttnK;
  bf16x8 rk[4], rv[4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      rk[i] = *reinterpret_cast<const bf16x8*>(Kh + ((int64_t)kt * kAttnK + (c >> 4)) * 128 + (c & 15) * 8);
      rv[i] = *reinterpret_cast<const bf16x8*>(Vh + (int64_t)(c >> 3) * a.Lpad + kt * kAttnK + (c & 7) * 8);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      *reinterpret_cast<bf16x8*>(&Ks[buf][(c >> 4) * kKPad + (c & 15) * 8]) = rk[i];
      // keys are stored with bits 2 and 3 of their index swapped, so the 8
      // keys one lane feeds to the P.V MFMA are contiguous (one 16-byte read)
      bf16* vd = &Vs[buf][(c >> 3) * kVPadT];
      const int k0 = (c & 7) * 8;  // first key of this 8-key chunk
      bf16x4 lo = {rv[i][0], rv[i][1], rv[i][2], rv[i][3]};
      bf16x4 hi = {rv[i][4], rv[i][5], rv[i][6], rv[i][7]};
      *reinterpret_cast<bf16x4*>(vd + vkey_pos(k0)) = lo;
      *reinterpret_cast<bf16x4*>(vd + vkey_pos(k0 + 4)) = hi;
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16){};
  // Scores never hold NaN here; the file is built with -fno-honor-nans so
  // fmaxf needs no canonicalisation. kNegBig stands for minus infinity.
  constexpr float kNegBig = -1e30f;
  float m_run = kNegBig, l_run = 0.f;
  const float c2 = a.scale * 1.4426950408889634f;  // scale * log2(e)

  // One 64-key tile. mask: the tile reaches past L (only the last one can).
  // The running max m_run is moved only when some lane's tile max exceeds it
  // by more than 2^8 (log2 units): p = exp2(s - m_run) then stays below 256,
  // and p, l and O all use the same m_run, so the result is exact.
  auto tile = [&](int kt, int cur, bool mask) {
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = (f32x16){};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        bf16x8 kf = *reinterpret_cast<const bf16x8*>(&Ks[cur][(kb * 32 + l32) * kKPad + kk * 16 + g * 8]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[kb], 0, 0, 0);
      }
    }
    // s[kb][r] = score(query l32, key kt*64 + kb*32 + 8*(r/4) + 4*g + r%4)
    if (__builtin_expect(mask, 0)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * kAttnK + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= a.L) s[kb][r] = kNegBig;
        }
    }
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[0][r], s[0][r + 1]));
#pragma unroll
    for (int r = 0; r < 16; r += 2) mx = fmaxf(mx, fmaxf(s[1][r], s[1][r + 1]));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
    if (__any(mx > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -m_run));
        psum += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (bf16)p;
      }
    }
    l_run += psum;
    // O^T += V^T P^T; MFMA kb2 covers keys 16*kb2 + 8*(i/4) + 4*g + i%4
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) {
        // keys 16 kb2 + 4g + {0..3} and 16 kb2 + 8 + 4g + {0..3}, stored contiguously
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vs[cur][(db * 32 + l32) * kVPadT + 16 * kb2 + 8 * g]);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb2], o[db], 0, 0, 0);
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  const bool ragged = (a.L % kAttnK) != 0;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ntiles) load_tile(kt + 1);
    tile(kt, cur, ragged && kt == ntiles - 1);
    if (kt + 1 < ntiles) store_tile(cur ^ 1);
    __syncthreads();
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (qrow < a.L) {
    bf16* dst = out_row(a, b, qrow) + hh * 128;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[db][rg * 4 + i] * inv);
        *reinterpret_cast<bf16x4*>(dst + db * 32 + rg * 8 + g * 4) = v;
      }
    }
  }
}

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.Lpad / kAttnQ, a.H, a.B), block(256);
  hipLaunchKernelGGL(k_attn_bf16, grid, block, 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- float32 path --
// One wavefront per query at a time; lane j scores key j of a 64-key chunk,
// then every lane accumulates its two output dims over the chunk.
constexpr int kF32QPerBlock = 16;

__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  __shared__ float qs[4][128];
  __shared__ float ps[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int hh = blockIdx.y, b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.H + hh;
  const float* Qh = reinterpret_cast<const float*>(a.Q) + bh * a.Lpad * 128;
  const float* Kh = reinterpret_cast<const float*>(a.K) + bh * a.Lpad * 128;
  const float* Vh = reinterpret_cast<const float*>(a.V) + bh * a.Lpad * 128;
  for (int qi = wave; qi < kF32QPerBlock; qi += 4) {
    const int t = blockIdx.x * kF32QPerBlock + qi;
    if (t >= a.L) break;
    qs[wave][lane] = Qh[(int64_t)t * 128 + lane];
    qs[wave][lane + 64] = Qh[(int64_t)t * 128 + lane + 64];
    __builtin_amdgcn_wave_barrier();
    float m_run = -INFINITY, l_run = 0.f, o0 = 0.f, o1 = 0.f;
    for (int k0 = 0; k0 < a.L; k0 += 64) {
      const int key = k0 + lane;
      float sc = -INFINITY;
      if (key < a.L) {
        const float* kr = Kh + (int64_t)key * 128;
        float acc = 0.f;
        for (int d = 0; d < 128; ++d) acc += qs[wave][d] * kr[d];
        sc = acc * a.scale;
      }
      const float m_new = fmaxf(m_run, wave_max(sc));
      const float p = key < a.L ? expf(sc - m_new) : 0.f;
      const float alpha = expf(m_run - m_new);
      l_run = l_run * alpha + wave_sum(p);
      m_run = m_new;
      ps[wave][lane] = p;
      __builtin_amdgcn_wave_barrier();
      o0 *= alpha;
      o1 *= alpha;
      const int nk = a.L - k0 < 64 ? a.L - k0 : 64;
      for (int j = 0; j < nk; ++j) {
        const float pj = ps[wave][j];
        o0 += pj * Vh[(int64_t)(k0 + j) * 128 + lane];
        o1 += pj * Vh[(int64_t)(k0 + j) * 128 + lane + 64];
      }
      __builtin_amdgcn_wave_barrier();
    }
    const int s = t < a.seg_len0 ? 0 : 1;
    const RowSeg& g = a.out[s];
    const int lt = s == 0 ? t : t - a.seg_len0;
    float* dst = reinterpret_cast<float*>(g.base) + (int64_t)b * g.batch_stride + (int64_t)lt * g.ld + hh * 128;
    dst[lane] = o0 / l_run;
    dst[lane + 64] = o1 / l_run;
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.L + kF32QPerBlock - 1) / kF32QPerBlock, a.H, a.B), block(256);
  hipLaunchKernelGGL(k_attn_f32, grid, block, 0, s, a);
  return hipGetLastError();
}

}  // namespace mmdit
