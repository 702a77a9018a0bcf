// Joint softmax attention over the concatenated [text; image] tokens, no
// mask, scale 1/sqrt(d) (mflux-rs card "Dual-Stream MMDiT": bidirectional
// attention between the two streams; card "Single-Stream Blocks": one
// self-attention sequence; stable-diffusion.rs README: the fused
// scaled_dot_product_attention it relies on).
//
// bf16 path (flash attention, gfx950 MFMA 32x32x16):
//  * a block owns 32 * NW queries of one (batch, head); each of its NW
//    wavefronts owns 32 queries; K and V^T tiles of 64 keys are staged in
//    LDS, double buffered, and shared by the NW wavefronts. They arrive by
//    direct-to-LDS loads (global_load_lds_dwordx4: no registers, no LDS
//    store instructions), issued one tile ahead;
//  * NW = 8: one block of 8 wavefronts per CU (two per SIMD). Two resident
//    blocks of 4 would run at unequal speeds (the older block's wavefronts
//    win issue), leaving one of them alone on the CU at the end of a round;
//    one block, in step at every tile barrier, avoids that and stages each
//    K/V tile once for 256 queries;
//  * LDS rows are stored with their 16-byte chunks XOR-swizzled by the row
//    index, so the MFMA operand reads (one 16-byte read per lane) of 16
//    consecutive rows hit distinct banks;
//  * S^T = K Q^T is computed so that each lane holds the scores of ONE query
//    (its MFMA column): the running max needs one cross-lane exchange;
//  * the probabilities stay in registers and feed O^T += V^T P^T directly as
//    the MFMA B operand. V^T arrives from the QK-norm kernel with its tokens
//    in vkey_pos order, so each lane's 8 keys are one contiguous 16 bytes;
//  * the softmax denominator is produced by the MFMA too: a fifth output
//    block multiplies P^T by a matrix of ones, so every row of it holds the
//    running sum of the (bf16) probabilities, with no per-score adds;
//  * online softmax in float32 with exp2 of log2(e)-scaled scores; the
//    running max is moved only when it grows by more than 2^8.
#include "common.h"
#include "kernels.h"

namespace mmdit {

constexpr int kAttnK = 64;    // keys per tile
constexpr int kKBuf = kAttnK * 256;  // bytes of a K tile (64 rows x 256 B)
constexpr int kVBuf = 128 * 128;     // bytes of a V^T tile (128 rows x 128 B)
constexpr int kStage = kKBuf + kVBuf;

__device__ __forceinline__ bf16* out_row(const AttnArgs& a, int b, int t) {
  const int s = t < a.seg_len0 ? 0 : 1;
  const RowSeg& g = a.out[s];
  const int local_t = s == 0 ? t : t - a.seg_len0;
  return reinterpret_cast<bf16*>(g.base) + (int64_t)b * g.batch_stride + (int64_t)local_t * g.ld;
}

// 64 lanes each copy 16 bytes from base + voff to LDS at m0_base + 16 * lane.
__device__ __forceinline__ void attn_dma16(const void* base, uint32_t voff, uint32_t m0_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(m0_base), "v"(voff), "s"(base) : "memory", "m0");
}

// LDS layouts (one stage): K tile row r (key) at r*256, 16-byte chunk c
// (dims 8c..8c+7) at position c ^ (r & 15); V^T tile row r (dim) at
// kKBuf + r*128, chunk c (positions 8c..8c+7) at c ^ ((r >> 1) & 7).
// Query blocks of 32 * NW rows per (batch, head); the last may reach past
// Lpad (its rows there load row Lpad - 1 and write nothing).
template <int NW>
__host__ __device__ __forceinline__ int attn_qblocks(const AttnArgs& a) {
  return (a.Lpad + 32 * NW - 1) / (32 * NW);
}

// Unit u = (b * H + head) * qblocks + query block: the unit's 32 * NW
// queries against all keys; writes the normalised output rows.
template <int NW>
__device__ __forceinline__ void attn_unit(const AttnArgs& a, char* smem, int unit) {
  constexpr int J = 16 / NW;  // DMA instructions per wave and operand
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const int qb_n = attn_qblocks<NW>(a);
  const int q0 = (unit % qb_n) * (32 * NW);
  const int hh = (unit / qb_n) % a.H, b = unit / qb_n / a.H;
  const int64_t bh = (int64_t)b * a.H + hh;
  const bf16* Qh = reinterpret_cast<const bf16*>(a.Q) + bh * a.Lpad * 128;
  const char* Kh = reinterpret_cast<const char*>(a.K) + bh * a.Lpad * 128 * 2;
  const char* Vh = reinterpret_cast<const char*>(a.V) + bh * 128 * (int64_t)a.Lpad * 2;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);

  // Q as the B operand of S^T = K Q^T: column = query, 8 consecutive dims.
  const int qrow = q0 + wave * 32 + l32;
  const int qld = qrow < a.Lpad ? qrow : a.Lpad - 1;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)qld * 128 + kk * 16 + g * 8);

  // Direct-to-LDS requests of one tile: 16 K and 16 V^T instructions of 64
  // lanes, J of each per wave; lane i of instruction jj fills LDS slot
  // jj*64 + i.
  uint32_t koff[J], voff[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int jj = wave * J + j;
    {  // K: row r = 4 jj + lane/16, slot lane%16 holds chunk (slot ^ (r & 15))
      const int r = jj * 4 + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      koff[j] = (uint32_t)((r * 128 + c * 8) * 2);
    }
    {  // V^T: row r = 8 jj + lane/8, slot lane%8 holds chunk (slot ^ ((r >> 1) & 7))
      const int r = jj * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      voff[j] = (uint32_t)(r * a.Lpad * 2 + c * 16);
    }
  }
  auto issue_tile = [&](int kt, int buf) {
    const uint32_t st = lds0 + (uint32_t)(buf * kStage);
    const char* kb = Kh + (size_t)kt * kAttnK * 256;
    const char* vb = Vh + (size_t)kt * kAttnK * 2;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      attn_dma16(kb, koff[j], st + (uint32_t)((wave * J + j) * 1024));
      attn_dma16(vb, voff[j], st + (uint32_t)(kKBuf + (wave * J + j) * 1024));
    }
  };

  // Per-lane LDS read offsets: K fragment (row kb*32 + l32, chunk 2kk + g),
  // V^T fragment (row db*32 + l32, chunk 2kb2 + g); the swizzle depends only
  // on l32, the block offsets (kb, db) are immediates.
  uint32_t kro[8], vro[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kro[kk] = (uint32_t)(l32 * 256 + (((2 * kk + g) ^ (l32 & 15)) * 16));
#pragma unroll
  for (int kb2 = 0; kb2 < 4; ++kb2)
    vro[kb2] = (uint32_t)(kKBuf + l32 * 128 + (((2 * kb2 + g) ^ ((l32 >> 1) & 7)) * 16));

  // o[0..3]: O^T blocks of 32 dims; o[4]: P^T times ones (row sums)
  f32x16 o[5];
#pragma unroll
  for (int db = 0; db < 5; ++db) o[db] = (f32x16){};
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16)1.0f;
  // Scores never hold NaN here; the file is built with -fno-honor-nans so
  // fmaxf needs no canonicalisation. kNegBig stands for minus infinity.
  constexpr float kNegBig = -1e30f;
  float m_run = kNegBig;
  const float c2 = a.scale * 1.4426950408889634f;  // scale * log2(e)

  // One 64-key tile in stage `cur`. mask: the tile reaches past L (only the
  // last one can). The running max m_run is moved only when some lane's tile
  // max exceeds it by more than 2^8 (log2 units): p = exp2(s - m_run) then
  // stays below 256, and p and O (including the row sums) use the same
  // m_run, so the result is exact.
  auto tile = [&](int kt, int cur, bool mask) {
    const char* st = smem + cur * kStage;
    f32x16 s[2];
    s[0] = (f32x16){};
    s[1] = (f32x16){};
    // all 16 K fragments requested up front: one LDS latency per tile
    bf16x8 kf[8][2];
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      kf[kk][0] = *reinterpret_cast<const bf16x8*>(st + kro[kk]);
      kf[kk][1] = *reinterpret_cast<const bf16x8*>(st + kro[kk] + 32 * 256);
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk][0], qf[kk], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk][1], qf[kk], s[1], 0, 0, 0);
    }
    // keep that order: the scheduler would otherwise pull each read next to
    // its MFMA and wait on it
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // 16 LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // 16 MFMAs
    __builtin_amdgcn_sched_barrier(0);
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
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
    for (int r = 3; r < 15; r += 2) mx = fmaxf(mx, fmaxf(s[0][r], s[0][r + 1]));
    mx = fmaxf(mx, fmaxf(s[0][15], s[1][0]));
#pragma unroll
    for (int r = 1; r < 15; r += 2) mx = fmaxf(mx, fmaxf(s[1][r], s[1][r + 1]));
    mx = fmaxf(mx, s[1][15]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
    if (__any(mx > m_run + 8.0f)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int db = 0; db < 5; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        pb[kb * 2 + (r >> 3)][r & 7] = (bf16)__builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -m_run));
    // O^T += V^T P^T; MFMA kb2 covers keys 16*kb2 + 8*(i/4) + 4*g + i%4,
    // stored contiguously; o[4] += ones P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      bf16x8 va[4];
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) va[kb2] = *reinterpret_cast<const bf16x8*>(st + vro[kb2] + db * 32 * 128);
#pragma unroll
      for (int kb2 = 0; kb2 < 4; ++kb2) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[kb2], pb[kb2], o[db], 0, 0, 0);
    }
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2) o[4] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pb[kb2], o[4], 0, 0, 0);
  };

  const int ntiles = (a.L + kAttnK - 1) / kAttnK;
  issue_tile(0, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the first tile (and Q) landed
  __syncthreads();
  const bool ragged = (a.L % kAttnK) != 0;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < ntiles) issue_tile(kt + 1, cur ^ 1);  // its stage was freed by the last barrier
    tile(kt, cur, ragged && kt == ntiles - 1);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile kt+1 landed
    __syncthreads();
  }
  // every row of o[4] holds this lane's query's probability sum
  const float inv = 1.0f / o[4][0];
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

// One block per unit, units in order (the query blocks of a head are
// adjacent, so blocks running together share that head's K/V tiles in L2).
template <int NW>
__global__ __launch_bounds__(64 * NW, 2) void k_attn_bf16(AttnArgs a) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  attn_unit<NW>(a, smem, blockIdx.x);
}

template <int NW>
hipError_t launch_attention_nw(const AttnArgs& a, hipStream_t s) {
  // K/V byte offsets from the per-(batch, head) base are 32-bit
  if ((int64_t)a.Lpad * 128 * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int units = attn_qblocks<NW>(a) * a.H * a.B;
  const size_t lds = 2 * kStage;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_attn_bf16<NW>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_attn_bf16<NW>, dim3(units), dim3(64 * NW), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t s) { return launch_attention_nw<kAttnWaves>(a, s); }

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
