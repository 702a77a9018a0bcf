// Joint softmax attention over the concatenated [text; image] tokens, no
// mask, scale 1/sqrt(d) (mflux-rs card "Dual-Stream MMDiT": bidirectional
// attention between the two streams; card "Single-Stream Blocks": one
// self-attention sequence; stable-diffusion.rs README: the fused
// scaled_dot_product_attention it relies on).
//
// bf16 path (flash attention, gfx950 MFMA 32x32x16):
//  * a block of 8 wavefronts owns 256 queries of one (batch, head), each
//    wavefront 32 of them; one block per CU (two wavefronts per SIMD). K and
//    V^T tiles of 64 keys are staged in LDS, double buffered, and shared by
//    the 8 wavefronts. They arrive by direct-to-LDS loads
//    (global_load_lds_dwordx4: no registers, no LDS store instructions);
//  * ping-pong: waves 0-3 and 4-7 (one of each per SIMD) run the same phase
//    sequence one phase apart, with a block barrier after every phase. A
//    wave alternates an MFMA phase [O^T += V^T(t-1) P^T(t-1) and
//    S^T(t) = K(t) Q^T] and a VALU phase [online softmax of S(t)], so in
//    every phase one wavefront of each SIMD feeds the matrix core while the
//    other computes its exponentials. The MFMA phase issues its LDS operand
//    reads one MFMA group ahead of use, at raised wave priority;
//  * LDS rows are stored with their 16-byte chunks XOR-swizzled by the row
//    index, so the MFMA operand reads (one 16-byte read per lane) of 16
//    consecutive rows hit distinct banks;
//  * S^T = K Q^T is computed so that each lane holds the scores of ONE query
//    (its MFMA column): the running max needs one cross-lane exchange;
//  * the probabilities stay in registers and feed O^T += V^T P^T directly as
//    the MFMA B operand. V^T arrives from the QK-norm kernel with its tokens
//    in vkey_pos order, so each lane's 8 keys are one contiguous 16 bytes;
//  * online softmax in float32 with exp2 of log2(e)-scaled scores; the
//    running max is moved only when a row sum of probabilities (which bounds
//    each of them) exceeds a fixed bound, so most tiles need no tile max;
//    row sums are float32 VALU adds in the softmax phase.
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
// Query blocks of 32 * kAttnWaves rows per (batch, head); the last may reach
// past Lpad (its rows there load row Lpad - 1 and write nothing).
__host__ __device__ __forceinline__ int attn_qblocks(const AttnArgs& a) {
  return (a.Lpad + 32 * kAttnWaves - 1) / (32 * kAttnWaves);
}

// Unit u = (b * H + head) * qblocks + query block: the unit's 256 queries
// against the keys of 64-key tiles [t0, t1). With rec null (t0 = 0, t1 =
// all tiles) it writes the normalised output rows; otherwise the piece's
// unnormalised O, running max m (scores times scale * log2 e) and row sum l
// go to the record rec (O [256][128], m [256], l [256], float32). Phase
// 2t + grp is a wave's MFMA phase of tile t, phase 2t + 1 + grp its softmax
// of tile t.
__device__ __forceinline__ void attn_unit(const AttnArgs& a, char* smem, int unit, int t0, int t1, float* rec) {
  constexpr int NW = kAttnWaves, J = 16 / NW;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int grp = wave >> 2;
  const int g = lane >> 5, l32 = lane & 31;
  const int qb_n = attn_qblocks(a);
  const int q0 = (unit % qb_n) * (32 * NW);
  const int hh = (unit / qb_n) % a.H, b = unit / qb_n / a.H;
  const int64_t bh = (int64_t)b * a.H + hh;
  const bf16* Qh = reinterpret_cast<const bf16*>(a.Q) + bh * a.Lpad * 128;
  const char* Kh = reinterpret_cast<const char*>(a.K) + bh * a.Lpad * 128 * 2;
  const char* Vh = reinterpret_cast<const char*>(a.V) + bh * 128 * (int64_t)a.Lpad * 2;
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);

  const int qrow = q0 + wave * 32 + l32;
  const int qld = qrow < a.Lpad ? qrow : a.Lpad - 1;
  bf16x8 qf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(Qh + (int64_t)qld * 128 + kk * 16 + g * 8);

  uint32_t koff[J], voff[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int jj = wave * J + j;
    {
      const int r = jj * 4 + (lane >> 4);
      const int c = (lane & 15) ^ (r & 15);
      koff[j] = (uint32_t)((r * 128 + c * 8) * 2);
    }
    {
      const int r = jj * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      voff[j] = (uint32_t)(r * a.Lpad * 2 + c * 16);
    }
  }
  auto issue_k = [&](int kt) {
    const uint32_t st = lds0 + (uint32_t)((kt & 1) * kStage);
    const char* kb = Kh + (size_t)kt * kAttnK * 256;
#pragma unroll
    for (int j = 0; j < J; ++j) attn_dma16(kb, koff[j], st + (uint32_t)((wave * J + j) * 1024));
  };
  auto issue_v = [&](int kt) {
    const uint32_t st = lds0 + (uint32_t)((kt & 1) * kStage);
    const char* vb = Vh + (size_t)kt * kAttnK * 2;
#pragma unroll
    for (int j = 0; j < J; ++j) attn_dma16(vb, voff[j], st + (uint32_t)(kKBuf + (wave * J + j) * 1024));
  };

  uint32_t kro[8], vro[4];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) kro[kk] = (uint32_t)(l32 * 256 + (((2 * kk + g) ^ (l32 & 15)) * 16));
#pragma unroll
  for (int kb2 = 0; kb2 < 4; ++kb2)
    vro[kb2] = (uint32_t)(kKBuf + l32 * 128 + (((2 * kb2 + g) ^ ((l32 >> 1) & 7)) * 16));

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = (f32x16){};
  // Scores arrive as exp2 arguments: Q carries scale * log2(e), and the
  // score MFMAs of every tile after the first start from -m_run, so
  // s = S c2 - m_run with m_run the running max (first tile: s = S c2).
  f32x16 s[2];
  bf16x8 pb[4];
  constexpr float kNegBig = -1e30f;
  float m_run = kNegBig, l_run = 0.f;
  float s_init = 0.f;  // -m_run once the first tile has set m_run

  // MFMA phase pieces. V^T fragments of dim blocks db0, db0+1 (8 reads) and
  // K fragments of dims 16*kk0 .. 16*kk0+63 (8 reads); MFMA groups of 8:
  // O^T[db0..db0+1] += V^T P^T, and S^T += K Q^T (two chains each, alternated).
  auto rd_v = [&](bf16x8 (&v)[8], const char* st, int db0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const bf16x8*>(st + vro[i & 3] + (db0 + (i >> 2)) * 32 * 128);
  };
  auto rd_k = [&](bf16x8 (&k)[8], const char* st, int kk0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k[2 * i] = *reinterpret_cast<const bf16x8*>(st + kro[kk0 + i]);
      k[2 * i + 1] = *reinterpret_cast<const bf16x8*>(st + kro[kk0 + i] + 32 * 256);
    }
  };
  auto mm_v = [&](const bf16x8 (&v)[8], int db0) {
#pragma unroll
    for (int kb2 = 0; kb2 < 4; ++kb2) {
      o[db0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[kb2], pb[kb2], o[db0], 0, 0, 0);
      o[db0 + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[4 + kb2], pb[kb2], o[db0 + 1], 0, 0, 0);
    }
  };
  // key blocks kb0, kb0+1 of all four dim blocks (four chains alternated)
  auto mm_v4 = [&](const bf16x8 (&v01)[8], const bf16x8 (&v23)[8], int kb0) {
#pragma unroll
    for (int kb2 = kb0; kb2 < kb0 + 2; ++kb2) {
      o[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v01[kb2], pb[kb2], o[0], 0, 0, 0);
      o[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v01[4 + kb2], pb[kb2], o[1], 0, 0, 0);
      o[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v23[kb2], pb[kb2], o[2], 0, 0, 0);
      o[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v23[4 + kb2], pb[kb2], o[3], 0, 0, 0);
    }
  };
  auto mm_k = [&](const bf16x8 (&k)[8], int kk0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[2 * i], qf[kk0 + i], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[2 * i + 1], qf[kk0 + i], s[1], 0, 0, 0);
    }
  };
  // Each read group is issued one MFMA group ahead of its use (the
  // scheduler would otherwise issue every read just before its MFMA and
  // wait on it).
  auto phase_pv_qk = [&](int t) {  // O^T += V^T(t-1) P^T(t-1); S^T(t) = K(t) Q^T
    const char* sv = smem + ((t + 1) & 1) * kStage;
    const char* sk = smem + (t & 1) * kStage;
    bf16x8 va[8], vb[8], ka[8], kc[8];
    rd_v(va, sv, 0);
    rd_v(vb, sv, 2);
    mm_v4(va, vb, 0);
    rd_k(ka, sk, 0);
    mm_v4(va, vb, 2);
    rd_k(kc, sk, 4);
#pragma unroll
    for (int i = 0; i < 16; ++i) s[0][i] = s[1][i] = s_init;
    mm_k(ka, 0);
    mm_k(kc, 4);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto phase_qk = [&](int t) {  // first tile: S^T(t) only
    const char* sk = smem + (t & 1) * kStage;
    bf16x8 ka[8], kc[8];
    rd_k(ka, sk, 0);
    rd_k(kc, sk, 4);
#pragma unroll
    for (int i = 0; i < 16; ++i) s[0][i] = s[1][i] = s_init;
    mm_k(ka, 0);
    mm_k(kc, 4);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto phase_pv = [&](int t) {  // after the last tile: O^T += V^T(t-1) P^T(t-1) only
    const char* sv = smem + ((t + 1) & 1) * kStage;
    bf16x8 va[8], vb[8];
    rd_v(va, sv, 0);
    rd_v(vb, sv, 2);
    mm_v(va, 0);
    mm_v(vb, 2);
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // softmax of S(kt). Probabilities p = exp2(s) = exp2(S c2 - m_run) go to bf16 for
  // the PV product; their row sums stay float32. Fast path: m_run is kept
  // while every p stays at most kPMax. All p are non-negative, so a row sum
  // (both lanes of a query) at most kPMax bounds each of them, and no tile max
  // is needed. A larger (or non-finite) sum, and the first tile, take the
  // slow path: the tile max moves m_run, O and l are rescaled, and p is
  // recomputed (then every p <= 1). p, O and the row sums all use the same
  // m_run, so the result is exact either way.
  constexpr float kPMax = 4096.f;
  auto probs = [&]() {
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[kb][r]);
        if (r & 1) ps1 += p; else ps0 += p;
        pb[kb * 2 + (r >> 3)][r & 7] = (bf16)p;
      }
    return ps0 + ps1;
  };
  auto softmax = [&](int kt, bool mask, bool first) {
    if (__builtin_expect(mask, 0)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * kAttnK + kb * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= a.L) s[kb][r] = kNegBig;
        }
    }
    float ps = 0.f;
    bool slow = first;
    if (!slow) {
      ps = probs();
      slow = __any(!(ps + __shfl_xor(ps, 32, 64) <= kPMax));
    }
    if (__builtin_expect(slow, 0)) {
      float mx = fmaxf(fmaxf(s[0][0], s[0][1]), s[0][2]);
#pragma unroll
      for (int r = 3; r < 15; r += 2) mx = fmaxf(mx, fmaxf(s[0][r], s[0][r + 1]));
      mx = fmaxf(mx, fmaxf(s[0][15], s[1][0]));
#pragma unroll
      for (int r = 1; r < 15; r += 2) mx = fmaxf(mx, fmaxf(s[1][r], s[1][r + 1]));
      mx = fmaxf(mx, s[1][15]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // s = S c2 - base with base = -s_init (0 on the first tile)
      const float base = -s_init;
      const float m_new = fmaxf(m_run, mx + base);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      const float delta = m_new - base;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] -= delta;
      ps = probs();
    }
    l_run += ps;
    s_init = -m_run;
    // keep the conversions in this phase (they would sink to their MFMAs)
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(pb[i]));
  };

  const int ntiles = (a.L + kAttnK - 1) / kAttnK;
  const bool ragged = (a.L % kAttnK) != 0;
  issue_k(t0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): K(0) (and Q) landed
  __syncthreads();
  // Phase 2u + grp of a wave is its MFMA phase of tile u, phase 2u + 1 + grp
  // its softmax of tile u; every wave passes 2 * ntiles + 2 barriers. At
  // the start of each even phase 2u, K(u+1) and V(u) are requested (their
  // buffers held K(u-1) and V(u-2), last read in phase 2u - 1); each odd
  // phase ends with vmcnt(0), so they have landed before phase 2u + 2.
  auto bar = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto issue = [&](int u) {
    if (u + 1 < t1) issue_k(u + 1);
    if (u < t1) issue_v(u);
  };
  auto hi = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto lo = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto sm = [&](int t) { softmax(t, ragged && t == ntiles - 1, t == t0); };
  auto wait_vm = [&]() { __builtin_amdgcn_s_waitcnt(0x0F70); };
  // first tile (MFMA phase: S(0) only), tiles 1 .. ntiles-1, then the last
  // PV; group 1 runs the same sequence one phase later
  if (grp == 0) {
    issue(t0);
    hi(); phase_qk(t0); lo();
    bar();
    sm(t0);
    wait_vm();
    bar();
    for (int t = t0 + 1; t < t1; ++t) {
      issue(t);
      hi(); phase_pv_qk(t); lo();
      bar();
      sm(t);
      wait_vm();
      bar();
    }
    hi(); phase_pv(t1); lo();
    bar();
    wait_vm();
    bar();
  } else {
    issue(t0);
    bar();
    hi(); phase_qk(t0); lo();
    wait_vm();
    bar();
    for (int t = t0 + 1; t < t1; ++t) {
      issue(t);
      sm(t - 1);
      bar();
      hi(); phase_pv_qk(t); lo();
      wait_vm();
      bar();
    }
    sm(t1 - 1);
    bar();
    hi(); phase_pv(t1); lo();
    wait_vm();
    bar();
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (rec) {  // partial piece: unnormalised O, m and l of each query
    if (qrow < a.L) {
      const int qi = wave * 32 + l32;
      float* dst = rec + (size_t)qi * 128;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *reinterpret_cast<f32x4*>(dst + db * 32 + rg * 8 + g * 4) =
              (f32x4){o[db][rg * 4], o[db][rg * 4 + 1], o[db][rg * 4 + 2], o[db][rg * 4 + 3]};
      if (g == 0) {
        rec[(size_t)32 * kAttnWaves * 128 + qi] = m_run;
        rec[(size_t)32 * kAttnWaves * 129 + qi] = l_tot;
      }
    }
    return;
  }
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

// Tail split: worker w of a.workers takes tiles [begin, end) of the
// flattened (tail unit, key tile) space, begin = w * T / workers with T =
// tail units * tiles per unit. A share is shorter than one unit, so it holds
// at most two pieces: the end of tail unit begin / nt (record 2w) and the
// start of the next (record 2w + 1).
__device__ __forceinline__ int64_t attn_share_begin(int w, int64_t T, int workers) {
  return (int64_t)w * T / workers;
}

__global__ __launch_bounds__(64 * kAttnWaves, 2) void k_attn_bf16(AttnArgs a) {
  if (guard_skip(a.skip)) return;
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int nt = (a.L + kAttnK - 1) / kAttnK;
  if (!a.part || (int)blockIdx.x < a.full_units) {
    attn_unit(a, smem, blockIdx.x, 0, nt, nullptr);
    return;
  }
  const int w = blockIdx.x - a.full_units;
  const int tail = attn_qblocks(a) * a.H * a.B - a.full_units;
  const int64_t T = (int64_t)tail * nt;
  const int64_t begin = attn_share_begin(w, T, a.workers), end = attn_share_begin(w + 1, T, a.workers);
  if (begin >= end) return;  // uniform over the block
  const int u0 = (int)(begin / nt);
  const int64_t split = (int64_t)(u0 + 1) * nt;
  attn_unit(a, smem, a.full_units + u0, (int)(begin - (int64_t)u0 * nt), (int)((end < split ? end : split) - (int64_t)u0 * nt),
            a.part + (size_t)(2 * w) * kAttnRecFloats);
  if (end > split) {
    __syncthreads();
    attn_unit(a, smem, a.full_units + u0 + 1, 0, (int)(end - split), a.part + (size_t)(2 * w + 1) * kAttnRecFloats);
  }
}

// Combines the pieces of each tail unit: for query q and dims 4j .. 4j+3,
// O = sum_i 2^(m_i - M) O_i / sum_i 2^(m_i - M) l_i with M = max_i m_i,
// written as bf16 to the output row. 32 threads per query, 8 queries per
// 256-thread block; unit tail u covers blocks u * 32 .. u * 32 + 31.
// A unit of nt tiles meets at most ceil(nt / share) + 1 shares, share =
// tail * nt / workers; the launcher splits only when tail >= workers / 6,
// so a unit has at most 7 pieces.
constexpr int kAttnMaxPieces = 8;

__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  if (guard_skip(a.skip)) return;
  constexpr int QU = 32 * kAttnWaves;  // queries per unit
  const int nt = (a.L + kAttnK - 1) / kAttnK;
  const int tail = attn_qblocks(a) * a.H * a.B - a.full_units;
  const int T = tail * nt;  // < 2^31: tail < kAttnTailWorkers, nt < 2^23
  const int ur = blockIdx.x / (QU / 8);
  const int q = (blockIdx.x % (QU / 8)) * 8 + (threadIdx.x >> 5);
  const int j = threadIdx.x & 31;
  const int unit = a.full_units + ur;
  const int qb_n = attn_qblocks(a);
  const int qrow = (unit % qb_n) * QU + q;
  if (qrow >= a.L) return;
  const int hh = (unit / qb_n) % a.H, b = unit / qb_n / a.H;
  // the records of this unit's pieces: the workers whose share meets
  // [ur * nt, (ur + 1) * nt)
  const int W = a.workers;
  const int lo = ur * nt, hi = lo + nt;
  int slot[kAttnMaxPieces];
  int np = 0;
  for (int v = (int)((int64_t)lo * W / T); v < W && np < kAttnMaxPieces; ++v) {
    const int bg = (int)((int64_t)v * T / W), en = (int)((int64_t)(v + 1) * T / W);
    if (bg >= hi) break;
    if (en <= lo || bg >= en) continue;
    slot[np++] = 2 * v + (bg / nt == ur ? 0 : 1);
  }
  float mx = -3.0e38f;
  for (int i = 0; i < np; ++i) mx = fmaxf(mx, a.part[(size_t)slot[i] * kAttnRecFloats + (size_t)QU * 128 + q]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, lsum = 0.f;
  for (int i = 0; i < np; ++i) {
    const float* r = a.part + (size_t)slot[i] * kAttnRecFloats;
    const float e = __builtin_amdgcn_exp2f(r[(size_t)QU * 128 + q] - mx);
    lsum += e * r[(size_t)QU * 129 + q];
    const f32x4 o = *reinterpret_cast<const f32x4*>(r + (size_t)q * 128 + 4 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += e * o[i];
  }
  const float inv = 1.0f / lsum;
  bf16* dst = out_row(a, b, qrow) + hh * 128 + 4 * j;
  *reinterpret_cast<bf16x4*>(dst) = (bf16x4){(bf16)(acc[0] * inv), (bf16)(acc[1] * inv), (bf16)(acc[2] * inv),
                                             (bf16)(acc[3] * inv)};
}

hipError_t launch_attention_bf16(const AttnArgs& in, hipStream_t s) {
  // K/V byte offsets from the per-(batch, head) base are 32-bit
  if ((int64_t)in.Lpad * 128 * 2 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  AttnArgs a = in;
  const int units = attn_qblocks(a) * a.H * a.B;
  const int C = kAttnTailWorkers;
  const int tail = units % C;
  // Split the last round only when it would leave at least three quarters
  // of the CUs idle. Pieces cost a start (Q loads, the first tile's max, the
  // pipeline fill) and a float32 record, and the merge reads every record:
  // measured at 4608 tokens (tail 176 of 256) the split call took 262 us
  // against 251 us whole, at 1280 tokens (tail 120, 20 tiles per unit)
  // 61 us against 40 us, and at 8704 tokens (tail 48) 780 us against 894 us.
  // tail >= C / 6 bounds the pieces of a unit (kAttnMaxPieces).
  const int nt = (a.L + kAttnK - 1) / kAttnK;
  const bool split = a.part && tail >= C / 6 && tail <= C / 4 && (int64_t)tail * nt >= 4 * (int64_t)C;
  a.full_units = split ? units - tail : units;
  a.workers = split ? C : 0;
  if (!split) a.part = nullptr;
  const size_t lds = 2 * kStage;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = ensure_lds_limit((const void*)k_attn_bf16, (int)lds, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_bf16, dim3(a.full_units + a.workers), dim3(64 * kAttnWaves), lds, s, a);
  if (a.part) hipLaunchKernelGGL(k_attn_merge, dim3(tail * (32 * kAttnWaves / 8)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- float32 path --
// One wavefront per query at a time; lane j scores key j of a 64-key chunk,
// then every lane accumulates its two output dims over the chunk.
constexpr int kF32QPerBlock = 16;

__global__ __launch_bounds__(256) void k_attn_f32(AttnArgs a) {
  if (guard_skip(a.skip)) return;
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
