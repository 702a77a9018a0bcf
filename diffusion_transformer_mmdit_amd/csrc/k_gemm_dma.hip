// Dense bf16 GEMM C = A W^T for the large projections (gfx950).
//
// 256 x 256 block tile, K-tile BK (64 by default), 4 wavefronts (2 x 2,
// 128 x 128 each) on v_mfma_f32_32x32x16_bf16 with the accumulators in AGPRs.
//
// Operand tiles move HBM -> LDS with the gfx950 direct-to-LDS load
// (global_load_lds_dwordx4): no VGPR staging and no LDS store instructions.
// LDS holds S stages (2 x 64 KB by default), one k-tile each. One barrier per
// k-tile, placed before its last 16-MFMA substep: after it, the requests for
// k-tile kt+S (into the stage k-tile kt just freed) and the reads of k-tile
// kt+1's first fragments are interleaved with those last 16 MFMAs, so each
// load has about one k-tile of MFMAs to arrive.
//
// LDS layout: each row (BK bf16 of one M or N index) is stored as BK/8
// 16-byte chunks in the order c ^ f(r) (f = swz<BK> below), so the 16-byte
// fragment reads of consecutive rows fall in distinct banks (for 32 and for
// 64 banks). The swizzle is applied on the load side: lane i of a DMA
// instruction writes slot i, so it fetches the global chunk destined for that
// slot.
#include <type_traits>

#include "gemm_common.h"

namespace mmdit {

constexpr int kDBM = 256, kDBN = 256;

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// 64 lanes each copy 16 bytes from base + voff (per-lane 32-bit byte offset,
// base a wave-uniform 64-bit address) to LDS at m0_base + 16 * lane.
// CPOL selects the cache-policy bits of the load (0: default, 1: sc0, 2: nt).
template <int CPOL>
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t m0_base) {
  if constexpr (CPOL == 1)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 sc0" : : "s"(m0_base), "v"(voff), "s"(base) : "memory", "m0");
  else if constexpr (CPOL == 2)
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2 nt" : : "s"(m0_base), "v"(voff), "s"(base) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" : : "s"(m0_base), "v"(voff), "s"(base) : "memory", "m0");
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt unconstrained), n <= 63.
__device__ __forceinline__ void wait_vm(int n) {
  // n is a compile-time constant at every call site after unrolling/inlining
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
#define MMDIT_VM(N) case N: __builtin_amdgcn_s_waitcnt(((N) & 15) | (0x7 << 4) | (0xF << 8) | (((N) >> 4) << 14)); break;
    MMDIT_VM(8) MMDIT_VM(16) MMDIT_VM(24) MMDIT_VM(32) MMDIT_VM(40) MMDIT_VM(48) MMDIT_VM(56)
#undef MMDIT_VM
    default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
  }
}

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Work unit of this workgroup: tile (prob, tm, tn) and k-range ks. Units are
// numbered k-range first (unit = ks * tiles + tile), so after the XCD remap
// of tile_of the units of one XCD share a k-range and neighbouring tiles.
__device__ __forceinline__ void unit_of(const GemmBatch& gb, int& prob, int& tm, int& tn, int& ks) {
  const int nb = gridDim.x;
  int bid = blockIdx.x;
  if ((nb & 7) == 0) bid = (bid & 7) * (nb >> 3) + (bid >> 3);
  const int tiles = gb.tile_start[2];
  ks = bid / tiles;
  tile_coords(gb, bid - ks * tiles, prob, tm, tn);
}

// Chunk order inside an LDS row of BK bf16 (16-byte chunks): chunk c of row r
// sits at position c ^ swz(r). Chosen so the 16-byte fragment reads of
// consecutive rows (same c) hit distinct banks for 32 and for 64 banks.
template <int BK>
__device__ __forceinline__ int swz(int r) {
  if constexpr (BK == 32) return ((r >> 1) ^ (r >> 2)) & 3;
  else return (r & 7) ^ ((r >> 3) & 1);
}

// Instruction order of one k-substep (NR fragment reads for the next substep,
// NM MFMAs): each read issued right behind an MFMA, so the LDS requests are
// spread over the first half of the substep and have the second half to
// return; the scheduler would otherwise pull each read next to its consumer
// and wait on it. Operand requests (inline asm, ordered with the reads as
// memory operations) stay behind the read they follow in the source. The
// fences keep substeps from being merged.
template <int NR, int NM>
__device__ __forceinline__ void substep_schedule() {
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
  __builtin_amdgcn_sched_barrier(0);
}

// Pins a kernel-argument value in registers: the compiler may otherwise
// re-load it from the argument segment (and wait on that load) next to every
// use, which dominated the epilogue.
template <typename T>
__device__ __forceinline__ T pin(T v) {
  asm volatile("" : "+s"(v));
  return v;
}
// Global-address-space views (pinned pointers lose that information, and
// generic accesses would be issued as flat instructions).
typedef __attribute__((address_space(1))) char gchar;
typedef __attribute__((address_space(1))) const char gcchar;
typedef __attribute__((address_space(1))) f32x4 gf32x4;
typedef __attribute__((address_space(1))) const f32x4 gcf32x4;
typedef __attribute__((address_space(1))) bf16x4 gbf16x4;
typedef __attribute__((address_space(1))) const bf16x4 gcbf16x4;
typedef __attribute__((address_space(1))) bf16x8 gbf16x8;


// FULL: every row and column of the wave tile is in range and (gated
// residual) all its rows lie in one batch of both residual views, so rows
// advance by a fixed stride and no per-row checks are needed. ALT: for the
// split epilogue, the tile lies after the split column (GELU, second
// output); for the gated residual, the residual is float32.
template <int EPI, int TN, bool FULL, bool ALT>
__device__ __forceinline__ void dma_epilogue_impl(const GemmProblem& P, float* stg, int m0w, int n0w, int lane,
                                                  const f32x16 (&acc)[4][TN / 32], const float (&bias)[4],
                                                  int ks) {
  constexpr int NJF = TN / 32;          // 32-column blocks of the wavefront tile
  constexpr int LPR = TN / 4;           // lanes per row in the read-back phase
  constexpr int RPI = 64 / LPR;         // rows per read-back instruction
  constexpr int RPL = 32 / RPI;         // rows per lane per 32-row chunk
  constexpr int LD = TN + 4;            // staging row stride (floats)
  // rows per group of in-flight residual loads (bounded by registers)
  constexpr int GR = EPI == EPI_GATE_RES && NJF == 2 ? 4 : 8;
  const int M = pin(P.M), N = pin(P.N);
  const int c4 = lane % LPR, rs = lane / LPR;
  const int n = n0w + 4 * c4;  // this lane's 4 columns (read-back phase)
  const bool n_ok = FULL || n < N;
  constexpr bool to2 = EPI == EPI_SPLIT && ALT;
  gchar* obase;
  int64_t ld;  // row stride in bytes of the written rows
  gcchar* ibase = nullptr;
  int64_t ldi = 0;
  f32x4 gate1 = {0.f, 0.f, 0.f, 0.f};
  int rpb_i = 1, rpb_o = 1, gbs = 0;
  int64_t bs_i = 0, bs_o = 0, ld_i = 0, ld_o = 0;
  constexpr bool f32r = EPI == EPI_GATE_RES && ALT;
  gcchar* gbase = nullptr;
  if constexpr (EPI == EPI_GATE_RES) {
    ibase = (gcchar*)pin(reinterpret_cast<const char*>(P.res_in.base));
    obase = (gchar*)pin(reinterpret_cast<char*>(P.res_out.base));
    gbase = (gcchar*)pin(reinterpret_cast<const char*>(P.gate));
    rpb_i = pin(P.res_in.rows_per_batch);
    rpb_o = pin(P.res_out.rows_per_batch);
    ld_i = pin(P.res_in.ld);
    ld_o = pin(P.res_out.ld);
    gbs = pin(P.gate_bstride);
    bs_i = pin(P.res_in.batch_stride);
    bs_o = pin(P.res_out.batch_stride);
    const int esz = f32r ? 4 : 2;
    if constexpr (FULL) {
      // one batch for all rows: rows are affine in m
      const int b_o = m0w / rpb_o, b_i = m0w / rpb_i;
      obase += ((int64_t)b_o * bs_o + (int64_t)(m0w - b_o * rpb_o) * ld_o + n) * esz;
      ibase += ((int64_t)b_i * bs_i + (int64_t)(m0w - b_i * rpb_i) * ld_i + n) * esz;
      gate1 = *(gcf32x4*)(gbase + ((int64_t)b_o * gbs + n) * 4);
    }
    ld = ld_o * esz;
    ldi = ld_i * esz;
  } else if constexpr (EPI == EPI_PARTIAL) {
    // float32 rows of k-range ks: part[ks][m][n], row stride N
    obase = (gchar*)pin(reinterpret_cast<char*>(P.part));
    ld = (int64_t)N * 4;
    obase += ((int64_t)ks * M * N + (int64_t)m0w * N + n) * 4;
  } else {
    obase = (gchar*)pin(reinterpret_cast<char*>(to2 ? P.out2 : P.out));
    ld = pin(to2 ? P.ldo2 : P.ldo) * 2;
    obase += ((int64_t)m0w * (ld / 2) + n - (to2 ? pin(P.split_n) : 0)) * 2;
  }
  if constexpr (EPI == EPI_GATE_RES && FULL) {
    // Residual rows requested one group ahead: the loads of group k + 1 are
    // in flight while group k is combined and stored (GR rows per lane and
    // group, RPL / GR groups per 32-row chunk).
    constexpr int GPC = RPL / GR, NG = 4 * GPC;
    typedef typename std::conditional<f32r, f32x4, bf16x4>::type RT;
    typedef __attribute__((address_space(1))) const RT gcRT;
    RT rbuf[2][GR];
    auto row_of = [&](int k, int t) { return 32 * (k / GPC) + RPI * (GR * (k % GPC) + t) + rs; };
#pragma unroll
    for (int t = 0; t < GR; ++t) rbuf[0][t] = *(gcRT*)(ibase + row_of(0, t) * ldi);
#pragma unroll
    for (int k = 0; k < NG; ++k) {
      const int i = k / GPC, h = k % GPC;
      if (h == 0) {
#pragma unroll
        for (int j = 0; j < NJF; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<f32x4*>(stg + (lane & 31) * LD + 32 * j + 8 * g + 4 * (lane >> 5)) =
                (f32x4){acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      }
      f32x4 a[GR];
#pragma unroll
      for (int t = 0; t < GR; ++t) a[t] = *reinterpret_cast<const f32x4*>(stg + (RPI * (GR * h + t) + rs) * LD + 4 * c4);
      if (k + 1 < NG) {
#pragma unroll
        for (int t = 0; t < GR; ++t) rbuf[(k + 1) & 1][t] = *(gcRT*)(ibase + row_of(k + 1, t) * ldi);
      }
#pragma unroll
      for (int t = 0; t < GR; ++t) {
        const RT rv = rbuf[k & 1][t];
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (float)rv[e] + gate1[e] * (a[t][e] + bias[e]);
        gchar* dstp = obase + row_of(k, t) * ld;
        if constexpr (f32r)
          *(gf32x4*)dstp = (f32x4){o[0], o[1], o[2], o[3]};
        else
          *(gbf16x4*)dstp = (bf16x4){(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // stage rows 32i .. 32i+31: lane owns row lane%32 of each group
#pragma unroll
    for (int j = 0; j < NJF; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(stg + (lane & 31) * LD + 32 * j + 8 * g + 4 * (lane >> 5)) =
            (f32x4){acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
    // read back RPL rows per lane (row 32i + RPI t + rs) in groups of GR; for
    // the gated residual, a group's loads are all issued before its stores
#pragma unroll
    for (int h = 0; h < RPL / GR; ++h) {
      f32x4 a[GR];
#pragma unroll
      for (int t = 0; t < GR; ++t) a[t] = *reinterpret_cast<const f32x4*>(stg + (RPI * (GR * h + t) + rs) * LD + 4 * c4);
      if constexpr (EPI == EPI_GATE_RES) {
        f32x4 res[GR], gt[GR];
        int64_t oo[GR];  // byte offsets of the written rows (general case)
#pragma unroll
        for (int t = 0; t < GR; ++t) {
          const int r = 32 * i + RPI * (GR * h + t) + rs;  // row within the wave tile
          if constexpr (FULL) {
            gt[t] = gate1;
            if constexpr (f32r) {
              res[t] = *(gcf32x4*)(ibase + r * ldi);
            } else {
              const bf16x4 v = *(gcbf16x4*)(ibase + r * ldi);
              res[t] = (f32x4){(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
            }
          } else {
            int m = m0w + r;
            const bool ok = m < M && n_ok;
            m = m < M ? m : M - 1;
            const int b_o = m / rpb_o, t_o = m - b_o * rpb_o;
            const int b_i = m / rpb_i, t_i = m - b_i * rpb_i;
            const int esz = f32r ? 4 : 2;
            oo[t] = ((int64_t)b_o * bs_o + (int64_t)t_o * ld_o + n) * esz;
            const int64_t oi = ((int64_t)b_i * bs_i + (int64_t)t_i * ld_i + n) * esz;
            res[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
            gt[t] = res[t];
            if (ok) {
              gt[t] = *(gcf32x4*)(gbase + ((int64_t)b_o * gbs + n) * 4);
              if constexpr (f32r) {
                res[t] = *(gcf32x4*)(ibase + oi);
              } else {
                const bf16x4 v = *(gcbf16x4*)(ibase + oi);
                res[t] = (f32x4){(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
              }
            }
          }
        }
#pragma unroll
        for (int t = 0; t < GR; ++t) {
          const int r = 32 * i + RPI * (GR * h + t) + rs;
          if (!FULL && (m0w + r >= M || !n_ok)) continue;
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = res[t][e] + gt[t][e] * (a[t][e] + bias[e]);
          gchar* dst = FULL ? obase + r * ld : obase + oo[t];
          if constexpr (f32r)
            *(gf32x4*)dst = (f32x4){o[0], o[1], o[2], o[3]};
          else
            *(gbf16x4*)dst = (bf16x4){(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
        }
      } else {
#pragma unroll
        for (int t = 0; t < GR; ++t) {
          const int r = 32 * i + RPI * (GR * h + t) + rs;
          if (!FULL && (m0w + r >= M || !n_ok)) continue;
          if constexpr (EPI == EPI_PARTIAL) {
            *(gf32x4*)(obase + r * ld) = a[t];
            continue;
          }
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = a[t][e] + bias[e];
          if constexpr (EPI == EPI_GELU || to2) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = gelu_fast(v[e]);
          }
          *(gbf16x4*)(obase + r * ld) = (bf16x4){(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
        }
      }
    }
  }
}

// Epilogue of a wave's 128 x TN tile, staged through LDS in 32-row chunks
// (float32, row stride TN + 4, so 16-byte writes of 16 consecutive rows hit
// distinct banks) so that each lane then owns 4 consecutive columns of a row:
// bias, GELU and the gated residual are applied to 4-column vectors, and each
// global access instruction covers whole row segments. The accumulator holds
// C transposed per register group:
// acc[i][j][4g + e] = C[m0w + 32i + lane%32][n0w + 32j + 8g + 4(lane/32) + e],
// so staging is one 16-byte LDS write per group. The caller has made the LDS
// free (barrier after the last operand reads); each wave uses its own slice.
// Column counts and row strides are multiples of 4 (checked before launch):
// a lane's 4 columns are all in range or all out of range. `bias` holds the
// lane's 4 columns' bias (loaded by the caller ahead of time). Outputs are
// bf16 (plain) or bf16 / float32 (gated residual), or the float32 partial
// sums of k-range `side` (EPI_PARTIAL, no bias).
template <int EPI, int TN>
__device__ __forceinline__ void dma_epilogue(const GemmProblem& P, char* smem, int m0w, int n0w, int wave,
                                             int lane, const f32x16 (&acc)[4][TN / 32], int side,
                                             const float (&bias)[4]) {
  float* stg = reinterpret_cast<float*>(smem) + wave * (32 * (TN + 4));
  bool full = m0w + 128 <= P.M && n0w + TN <= P.N;
  if constexpr (EPI == EPI_GATE_RES) {
    const int rpb_o = P.res_out.rows_per_batch, rpb_i = P.res_in.rows_per_batch;
    full = full && m0w / rpb_o == (m0w + 127) / rpb_o && m0w / rpb_i == (m0w + 127) / rpb_i;
  }
  bool alt = false;
  if constexpr (EPI == EPI_SPLIT) alt = side == 1;
  if constexpr (EPI == EPI_GATE_RES) alt = P.res_f32;
  if (full) {
    if (alt) dma_epilogue_impl<EPI, TN, true, true>(P, stg, m0w, n0w, lane, acc, bias, side);
    else dma_epilogue_impl<EPI, TN, true, false>(P, stg, m0w, n0w, lane, acc, bias, side);
  } else {
    if (alt) dma_epilogue_impl<EPI, TN, false, true>(P, stg, m0w, n0w, lane, acc, bias, side);
    else dma_epilogue_impl<EPI, TN, false, false>(P, stg, m0w, n0w, lane, acc, bias, side);
  }
}

// Fused QK RMSNorm + RoPE for a wavefront tile of the q or k columns
// (mflux-rs card "Dual-Stream MMDiT": q and k RMS-normalised per head;
// card "3D RoPE Coordinates": adjacent pairs rotated by the token's angles).
// The wavefront's 128 columns are exactly one head. Each 32-row chunk is
// staged through LDS as in dma_epilogue_impl; lane (r = lane % 32, hf =
// lane / 32) then takes dims 64 hf .. 64 hf + 63 of chunk row r, so a row's
// sum of squares is the lane's 64 terms plus its partner's (lane ^ 32), and
// every rotation pair lies in one lane. Rows go to Q (K) [B, H, Lpad, 128].
//
// When the chunk's 32 rows are consecutive tokens of one batch (every chunk
// but a ragged last one or one that straddles a batch), their angles are one
// contiguous 16 KB block of the table and their output rows one contiguous
// 8 KB block of Q (K): the angles arrive by whole-wavefront 1 KB loads
// (requested one chunk ahead) and are handed to the lanes of their rows
// through the chunk's LDS slice, and the bf16 results go back through the
// slice so that each store writes 4 whole rows. Other chunks load each row's
// angles and store each row's halves lane by lane. A wavefront touches only
// its own LDS slice, and its LDS operations complete in program order.
template <int TN>
__device__ __forceinline__ void qk_epilogue(const GemmProblem& P, char* smem, int m0w, int n0w, int wave,
                                            int lane, const f32x16 (&acc)[4][TN / 32]) {
  static_assert(TN == 128, "one head per wavefront tile");
  constexpr int LD = TN + 4;   // float32 row stride of the slice (angles use 128 of it)
  constexpr int LDB = 136;     // bf16 row stride of the staged output rows
  float* stg = reinterpret_cast<float*>(smem) + wave * (32 * LD);
  // output rows: a second slice per wavefront, after the four float32 slices
  bf16* stgb = reinterpret_cast<bf16*>(smem + 4 * 32 * LD * 4) + wave * (32 * LDB);
  const int M = pin(P.M);
  const int qk_h = pin(P.qk_h);
  const int which = n0w >= qk_h ? 1 : 0;  // 0 q, 1 k
  const int hh = (n0w - which * qk_h) >> 7;
  const int H = qk_h >> 7;
  const int rows = pin(P.qk_rows), tok0 = pin(P.qk_tok0), Lpad = pin(P.qk_Lpad);
  const float eps = P.qk_eps;
  const int r = lane & 31, hf = lane >> 5;
  gchar* dst = (gchar*)pin(reinterpret_cast<char*>(which ? P.qk_K : P.qk_Q));
  gcchar* gsc = (gcchar*)(reinterpret_cast<const char*>(which ? P.kn : P.qn) + 128 * hf);
  gcchar* bp = (gcchar*)pin(reinterpret_cast<const char*>(P.bias));
  gcchar* rope = (gcchar*)pin(reinterpret_cast<const char*>(P.rope));
  // the lane's 64 norm weights and biases serve all four chunks
  bf16x8 g8[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) g8[q] = *(const __attribute__((address_space(1))) bf16x8*)(gsc + 16 * q);
  bf16x4 b4[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) b4[q] = bp ? *(gcbf16x4*)(bp + (n0w + 64 * hf + 4 * q) * 2) : bf16x4{};
  // chunk i: first row mc, batch bF, first token tF; fast when its 32 rows
  // are in range and in one batch (then tokens tF .. tF + 31)
  auto chunk = [&](int i, int& bF, int& tF) {
    const int mc = m0w + 32 * i;
    bF = mc / rows;
    tF = tok0 + (mc - bF * rows);
    return mc + 32 <= M && (mc + 31) / rows == bF;
  };
  f32x4 tbl[16];  // angles of a fast chunk as loaded: floats 256 q + 4 lane .. + 3 of its block
  auto load_block = [&](int tF) {
    gcchar* tb = rope + (int64_t)tF * 512;
#pragma unroll
    for (int q = 0; q < 16; ++q) tbl[q] = *(gcf32x4*)(tb + q * 1024 + lane * 16);
  };
  {
    int b0, t0;
    if (chunk(0, b0, t0)) load_block(t0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int bF, tF;
    const bool fast = chunk(i, bF, tF);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(stg + r * LD + 32 * j + 8 * g + 4 * hf) =
            (f32x4){acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
    float v[64];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(stg + r * LD + 64 * hf + 4 * q);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * q + e] = x[e] + (float)b4[q][e];
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 64; ++c) ss += v[c] * v[c];
    ss += __shfl_xor(ss, 32);
    // q rows carry the attention's score scale
    const float rstd = (which ? 1.0f : P.qk_qscale) / sqrtf(ss * (1.0f / 128.0f) + eps);
    int m = m0w + 32 * i + r;
    const bool ok = m < M;
    m = ok ? m : M - 1;  // rows past the end read a valid row's angles and store nothing
    const int b = m / rows;
    const int t = tok0 + (m - b * rows);
    asm volatile("" ::: "memory");  // the chunk's reads of the slice stay ahead of the angle writes
    if (fast) {
      // angles of row 2q + lane / 32 (floats 4 (lane % 32) ..) into the slice
#pragma unroll
      for (int q = 0; q < 16; ++q) *reinterpret_cast<f32x4*>(stg + (2 * q + hf) * LD + 4 * r) = tbl[q];
      if (i + 1 < 4) {
        int bn, tn;
        if (chunk(i + 1, bn, tn)) load_block(tn);
      }
    }
    asm volatile("" ::: "memory");
    const float* arow = stg + r * LD + 64 * hf;
    gcchar* tb = rope + ((int64_t)t * 128 + 64 * hf) * 4;
    gchar* orow = dst + ((((int64_t)b * H + hh) * Lpad + t) * 128 + 64 * hf) * 2;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      f32x4 ca, cb;
      if (fast) {
        ca = *reinterpret_cast<const f32x4*>(arow + 8 * q);
        cb = *reinterpret_cast<const f32x4*>(arow + 8 * q + 4);
      } else {
        ca = *(gcf32x4*)(tb + 32 * q);
        cb = *(gcf32x4*)(tb + 32 * q + 16);
      }
      const float cs[8] = {ca[0], ca[1], ca[2], ca[3], cb[0], cb[1], cb[2], cb[3]};
      bf16x8 o;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float y0 = v[8 * q + 2 * u] * rstd * (float)g8[q][2 * u];
        const float y1 = v[8 * q + 2 * u + 1] * rstd * (float)g8[q][2 * u + 1];
        const float c = cs[2 * u], sn = cs[2 * u + 1];
        o[2 * u] = (bf16)(c * y0 - sn * y1);
        o[2 * u + 1] = (bf16)(sn * y0 + c * y1);
      }
      if (fast) *reinterpret_cast<bf16x8*>(stgb + r * LDB + 64 * hf + 8 * q) = o;
      else if (ok) *(gbf16x8*)(orow + 16 * q) = o;
    }
    asm volatile("" ::: "memory");
    if (fast) {
      // rows through the output slice: store k writes rows 4k .. 4k + 3 whole
      gchar* out = dst + (((int64_t)bF * H + hh) * Lpad + tF) * 256;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int rr = 4 * k + (lane >> 4);
        const bf16x8 w = *reinterpret_cast<const bf16x8*>(stgb + rr * LDB + 8 * (lane & 15));
        *(gbf16x8*)(out + rr * 256 + 16 * (lane & 15)) = w;
      }
    }
    asm volatile("" ::: "memory");  // the slices' reads stay ahead of the next chunk's writes
  }
}

// V columns of the fused QKV epilogue: the wavefront's 128 columns are the
// 128 dims of one head, written transposed to V^T [B, H, 128, Lpad] where
// position p holds token vkey_pos(p) (the key order the attention kernel's
// PV product reads). Each 32-row chunk is staged through LDS; lane l then
// takes dims l and l + 64. When the chunk's 32 rows are consecutive tokens
// of one batch starting at a multiple of 16, the positions are the same 32
// tokens permuted within 16-token groups, so each dim is four 16-byte
// stores; otherwise every element is stored at its own position.
template <int TN>
__device__ __forceinline__ void v_epilogue(const GemmProblem& P, char* smem, int m0w, int n0w, int wave,
                                           int lane, const f32x16 (&acc)[4][TN / 32]) {  // 128 rows
  static_assert(TN == 128, "one head per wavefront tile");
  constexpr int LD = TN + 4;
  float* stg = reinterpret_cast<float*>(smem) + wave * (32 * LD);
  const int M = pin(P.M);
  const int qk_h = pin(P.qk_h);
  const int hh = (n0w - 2 * qk_h) >> 7;
  const int H = qk_h >> 7;
  const int rows = pin(P.qk_rows), tok0 = pin(P.qk_tok0), Lpad = pin(P.qk_Lpad);
  gchar* vt = (gchar*)pin(reinterpret_cast<char*>(P.qk_V));
  const bf16* bp = reinterpret_cast<const bf16*>(P.bias);
  float bias[2] = {0.f, 0.f};
  if (bp) {
    bias[0] = (float)bp[n0w + lane];
    bias[1] = (float)bp[n0w + lane + 64];
  }
  const int r = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<f32x4*>(stg + r * LD + 32 * j + 8 * g + 4 * hf) =
            (f32x4){acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
    const int mc = m0w + 32 * i;  // first row of the chunk
    const int bF = mc / rows;
    const int tF = tok0 + (mc - bF * rows);
    const bool fast = mc + 32 <= M && (mc + 31) / rows == bF && (tF & 15) == 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int d = lane + 64 * q;
      if (fast) {
        float x[32];
#pragma unroll
        for (int rr = 0; rr < 32; ++rr) x[rr] = stg[rr * LD + d] + bias[q];
        gchar* row = vt + ((((int64_t)bF * H + hh) * 128 + d) * Lpad + tF) * 2;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bf16x8 o;
#pragma unroll
          for (int u = 0; u < 8; ++u) o[u] = (bf16)x[vkey_pos(8 * c + u)];
          *(gbf16x8*)(row + 16 * c) = o;
        }
      } else {
        for (int rr = 0; rr < 32; ++rr) {
          const int m = mc + rr;
          if (m >= M) break;
          const int b = m / rows;
          const int t = tok0 + (m - b * rows);
          gchar* dst = vt + ((((int64_t)b * H + hh) * 128 + d) * Lpad + vkey_pos(t)) * 2;
          *(__attribute__((address_space(1))) bf16*)dst = (bf16)(stg[rr * LD + d] + bias[q]);
        }
      }
    }
  }
}

// FMT 0: dense bf16 weights, both operands by DMA. FMT 1 / 2: 4-bit / 8-bit
// group-quantised weights (groups of 64 along k = one k-tile, so one bf16
// scale per weight row per k-tile): the packed codes of k-tile kt+1 are
// loaded into registers when k-tile kt+1's A DMA is issued, and dequantised
// into the B half of its stage (same swizzled bf16 layout) just before the
// barrier that publishes it. FMT 3 / 4: 1-bit / ternary codes with groups of
// 128 along k (two k-tiles share a scale), staged the same way in pieces of
// 32 weights.
template <int EPI, int BK, int S, int CPOL, int FMT, int DS, int W>
__global__ __launch_bounds__(64 * W, 1) void k_gemm_dma(GemmBatch gb) {
  if (guard_skip(gb.p[0].skip)) return;
  constexpr int NT = 64 * W;                       // threads
  constexpr int WN = W / 2;                        // wavefront columns (2 rows of wavefronts)
  constexpr int TN = kDBN / WN;                    // columns of a wavefront tile (128 rows)
  constexpr int NJF = TN / 32;                     // 32-column MFMA blocks per wavefront
  constexpr int CH = BK / 8;                       // 16-byte chunks per row
  constexpr int KS = BK / 16;                      // MFMA k-substeps per k-tile
  constexpr int HALF = kDBM * BK * 2;              // bytes of the A (or B) part of a stage
  constexpr int STAGE = 2 * HALF;
  constexpr int NJ = kDBM * CH / NT;               // DMA instructions per wave for A (and for dense B)
  constexpr int G = FMT == 0 ? 2 * NJ : NJ;        // DMA instructions per wave per k-tile
  // quantised B (4/8-bit): raw 16-byte chunks per thread per k-tile (rows of BK codes)
  constexpr bool SUB = FMT == 3 || FMT == 4;       // sub-byte, groups of 128 along k
  constexpr int QB = FMT == 2 ? BK : BK / 2;       // bytes per weight row per k-tile
  constexpr int QCH = SUB ? 1 : kDBN * QB / 16 / NT;  // raw chunks per thread
  constexpr int QPR = SUB ? 1 : QB / 16;           // raw chunks per row
  // sub-byte B: pieces of 32 weights (4 bytes 1-bit, 8 bytes ternary), 2 per row
  constexpr int PCS = SUB ? 2 * kDBN / NT : 1;     // pieces per thread per k-tile
  static_assert(FMT == 0 || BK == 64, "quantised weights need 64-wide k-tiles (one scale group)");
  static_assert(!SUB || PCS >= 1, "one sub-byte piece per thread at least");
  static_assert(S * STAGE >= W * 32 * (TN + 4) * 4, "epilogue staging must fit in the operand stages");
  static_assert(EPI != EPI_QKV && EPI != EPI_SPLIT_QKV || S * STAGE >= W * 32 * ((TN + 4) * 4 + 136 * 2),
                "QK epilogue output slices must fit in the operand stages");
  static_assert(EPI != EPI_PARTIAL || FMT == 0, "split-K runs on dense weights");
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int prob, tm, tn, ks;
  unit_of(gb, prob, tm, tn, ks);
  const GemmProblem& P = gb.p[prob];
  const int M = P.M, N = P.N, K = P.K;
  const int m0 = tm * kDBM, n0 = tn * kDBN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave / WN) * 128, wn0 = (wave % WN) * TN;
  const uint32_t lds0 = lds_offset(smem);

  // Per-lane source of each DMA instruction: a 32-bit byte offset (row fixed
  // for the whole K loop) from the wave-uniform base of A or W, which advances
  // with k. Lane i of instruction j of wave w fills 16-byte slot
  // (w*NJ + j)*64 + i of the tile.
  const char* abase = reinterpret_cast<const char*>(P.A);
  const char* bbase = reinterpret_cast<const char*>(P.W);
  // k-tiles of this unit: all of them, or range ks of ksplit near-equal ranges
  int nk = K / BK;
  if constexpr (EPI == EPI_PARTIAL) {
    const int nsplit = gb.ksplit;
    const int k0t = ks * nk / nsplit;
    nk = (ks + 1) * nk / nsplit - k0t;
    abase += (size_t)k0t * BK * 2;
    bbase += (size_t)k0t * BK * 2;
  }
  uint32_t aoffg[NJ], boffg[FMT == 0 ? NJ : 1];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int sl = (wave * NJ + j) * 64 + lane;
    const int r = sl / CH, c = (sl % CH) ^ swz<BK>(sl / CH);
    int gm = m0 + r;
    gm = gm < M ? gm : M - 1;  // rows past the edge re-read a valid row; their outputs are dropped
    aoffg[j] = (uint32_t)(((int64_t)gm * P.lda + c * 8) * 2);
    if constexpr (FMT == 0) {
      int gn = n0 + r;
      gn = gn < N ? gn : N - 1;
      boffg[j] = (uint32_t)(((int64_t)gn * K + c * 8) * 2);
    }
  }
  // DMA instruction q (0 .. G-1) of k-tile kt: q < NJ for A, else B.
  // request q of k-tile `src` into the stage of k-tile `dst` (src == dst
  // except for the harmless re-reads described at the main loop)
  auto dma_to = [&](int src, int dst, int q) {
    const uint32_t st = lds0 + (uint32_t)((dst % S) * STAGE);
    const size_t koff = (size_t)src * BK * 2;
    if (q < NJ) dma16<CPOL>(abase + koff, aoffg[q], st + (uint32_t)((wave * NJ + q) * 1024));
    else if constexpr (FMT == 0)
      dma16<CPOL>(bbase + koff, boffg[q - NJ], st + HALF + (uint32_t)((wave * NJ + q - NJ) * 1024));
  };
  auto dma_one = [&](int kt, int q) {
    const uint32_t st = lds0 + (uint32_t)((kt % S) * STAGE);
    const size_t koff = (size_t)kt * BK * 2;
    if (q < NJ) dma16<CPOL>(abase + koff, aoffg[q], st + (uint32_t)((wave * NJ + q) * 1024));
    else if constexpr (FMT == 0)
      dma16<CPOL>(bbase + koff, boffg[q - NJ], st + HALF + (uint32_t)((wave * NJ + q - NJ) * 1024));
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int q = 0; q < G; ++q) dma_one(kt, q);
  };

  // Quantised B: raw chunk i of this thread is chunk q = tid + NT i of the
  // k-tile: weight row q / QPR, part q % QPR.
  u32x4 braw[FMT == 0 ? 1 : QCH];
  float bscale[FMT == 0 ? 1 : QCH];
  // sub-byte piece i of this thread is piece pc = tid * PCS + i: weight row
  // pc / 2, weights 32 (pc % 2) .. + 31 of the k-tile
  uint32_t sraw[PCS][2];
  uint32_t sscale[PCS];
  auto load_braw = [&](int kt) {
    if constexpr (SUB) {
      const uint16_t* sc = reinterpret_cast<const uint16_t*>(P.scales);
#pragma unroll
      for (int i = 0; i < PCS; ++i) {
        const int pc = tid * PCS + i;
        int gn = n0 + pc / 2;
        gn = gn < N ? gn : N - 1;
        sscale[i] = sc[(int64_t)gn * (K / 128) + kt / 2];
        if constexpr (FMT == 3) {
          sraw[i][0] = *reinterpret_cast<const uint32_t*>(bbase + (int64_t)gn * (K / 8) + (int64_t)kt * 8 + (pc % 2) * 4);
          sraw[i][1] = 0;
        } else {
          const uint2 v = *reinterpret_cast<const uint2*>(bbase + (int64_t)gn * (K / 4) + (int64_t)kt * 16 + (pc % 2) * 8);
          sraw[i][0] = v.x;
          sraw[i][1] = v.y;
        }
      }
    } else if constexpr (FMT != 0) {
#pragma unroll
      for (int i = 0; i < QCH; ++i) {
        const int q = tid + NT * i;
        int gn = n0 + q / QPR;
        gn = gn < N ? gn : N - 1;
        braw[i] = *reinterpret_cast<const u32x4*>(bbase + (int64_t)gn * (K / 64) * QB + (int64_t)kt * QB + (q % QPR) * 16);
        bscale[i] = (float)reinterpret_cast<const bf16*>(P.scales)[(int64_t)gn * (K / 64) + kt];
      }
    }
  };
  auto store_b = [&](int kt) {
    if constexpr (SUB) {
      char* st = smem + (kt % S) * STAGE + HALF;
#pragma unroll
      for (int i = 0; i < PCS; ++i) {
        const int pc = tid * PCS + i;
        const int r = pc / 2, half = pc % 2;
        const int sw = swz<BK>(r);
        bf16x8 o[4];
        if constexpr (FMT == 3) deq_q1_32(sraw[i][0], sscale[i], o);
        else deq_tq2_32(sraw[i][0], sraw[i][1], sscale[i], o);
#pragma unroll
        for (int u = 0; u < 4; ++u) *reinterpret_cast<bf16x8*>(st + (r * CH + ((4 * half + u) ^ sw)) * 16) = o[u];
      }
    } else if constexpr (FMT != 0) {
      char* st = smem + (kt % S) * STAGE + HALF;
#pragma unroll
      for (int i = 0; i < QCH; ++i) {
        const int q = tid + NT * i;
        const int r = q / QPR, part = q % QPR;
        const int sw = swz<BK>(r);
        if constexpr (FMT == 2) {
          bf16x8 lo, hi;
          deq8(braw[i], bscale[i], lo, hi);
          *reinterpret_cast<bf16x8*>(st + (r * CH + ((2 * part) ^ sw)) * 16) = lo;
          *reinterpret_cast<bf16x8*>(st + (r * CH + ((2 * part + 1) ^ sw)) * 16) = hi;
        } else {
          bf16x8 o[4];
          deq4(braw[i], bscale[i], o);
#pragma unroll
          for (int u = 0; u < 4; ++u) *reinterpret_cast<bf16x8*>(st + (r * CH + ((4 * part + u) ^ sw)) * 16) = o[u];
        }
      }
    }
  };

  // Fragment reads for k-substep kk: A rows wm0 + 32i + lane%32, chunk
  // 2kk + lane/32. The swizzle depends only on the row's low 4 bits, so one
  // lane offset per kk serves all i (+ i * 32 rows, an immediate).
  uint32_t aoff[KS], boff[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const int ra = wm0 + (lane & 31);
    const int rb = wn0 + (lane & 31);
    const int c = kk * 2 + (lane >> 5);
    aoff[kk] = (uint32_t)((ra * CH + (c ^ swz<BK>(ra))) * 16);
    boff[kk] = HALF + (uint32_t)((rb * CH + (c ^ swz<BK>(rb))) * 16);
  }
  auto read_a = [&](int kt, int kk, int i) {
    return *reinterpret_cast<const bf16x8*>(smem + (kt % S) * STAGE + aoff[kk] + i * 32 * CH * 16);
  };
  auto read_b = [&](int kt, int kk, int i) {
    return *reinterpret_cast<const bf16x8*>(smem + (kt % S) * STAGE + boff[kk] + i * 32 * CH * 16);
  };
  auto read_frags = [&](int kt, int kk, bf16x8* fa, bf16x8* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = read_a(kt, kk, i);
#pragma unroll
    for (int j = 0; j < NJF; ++j) fb[j] = read_b(kt, kk, j);
  };

  f32x16 acc[4][NJF];
  // Weight rows go in as the MFMA's first operand, so the accumulator holds
  // C transposed: acc[i][j][r] = C[m0 + wm0 + 32i + lane%32]
  //                                [n0 + wn0 + 32j + 8(r/4) + 4(lane/32) + r%4],
  // four consecutive output columns of one row per group of four registers.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJF; ++j) acc[i][j] = (f32x16){};
  auto mfmas = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJF; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
  };

  // bias of this lane's epilogue columns (requested now, used at the end)
  float ebias[4] = {0.f, 0.f, 0.f, 0.f};
  {
    const bf16* bp = EPI == EPI_PARTIAL ? nullptr : reinterpret_cast<const bf16*>(P.bias);
    const int n = n0 + wn0 + 4 * (lane % (TN / 4));
    if (bp && n < N) {
      const bf16x4 v = *reinterpret_cast<const bf16x4*>(bp + n);
#pragma unroll
      for (int e = 0; e < 4; ++e) ebias[e] = (float)v[e];
    }
  }

  constexpr int DSP = FMT == 0 ? DS : 1;
  constexpr int PER = (G + DSP - 1) / DSP;  // requests per substep
  // Dense operands, 2 stages: the loop issues every request unconditionally
  // (no branch per request). Requests past the last k-tile re-read k-tile
  // nk-1 into a stage that is never read again; the prologue issues only the
  // first PER requests of k-tile 1, and iteration 0 continues them exactly as
  // every later iteration continues the previous one's.
  constexpr bool UNCOND = FMT == 0 && S == 2;
  if constexpr (UNCOND) {
    issue(0);
    const int k1 = nk > 1 ? 1 : 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) dma_to(k1, 1, q);
    wait_vm(PER);
  } else if constexpr (FMT == 0) {
    // Prologue: one k-tile per stage requested; wait for k-tile 0.
#pragma unroll
    for (int u = 0; u < S; ++u)
      if (u < nk) issue(u);
    const int ahead = (S - 1) < (nk - 1) ? (S - 1) : (nk - 1);
    wait_vm(G * ahead);
  } else {
    static_assert(FMT == 0 || S == 2, "quantised path uses a 2-stage ring");
    issue(0);
    load_braw(0);
    wait_vm(0);
    store_b(0);
    if (nk > 1) {
      issue(1);
      load_braw(1);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): B of k-tile 0 written
  }
  barrier();
  bf16x8 fa[2][4], fb[2][NJF];
  read_frags(0, 0, fa[0], fb[0]);
  // k-tile kt: fragments of substep kk+1 are read while substep kk multiplies.
  // Before the last substep: wait for k-tile kt+1 (k-tiles up to kt+S-1 have
  // been requested; quantised B is dequantised into its stage here), barrier;
  // then the last substep's 16 MFMAs run with the reads of k-tile kt+1's
  // first fragments interleaved between them, and the requests for k-tile
  // kt+S (into the stage k-tile kt just freed) start. Dense operands spread
  // those requests over DS substeps (the last one of k-tile kt and the first
  // DS-1 of k-tile kt+1), so the vector-memory queue never holds a whole
  // k-tile's requests at once and the MFMAs behind them keep issuing.
  static_assert(DSP >= 1 && DSP <= KS, "spread must fit in one k-tile");
  // substep with the MFMAs interleaved: reads of the next fragments behind
  // the first 8 MFMAs, requests q0 .. q1-1 of k-tile dkt behind the first ones.
  auto substep_dma = [&](const bf16x8* ca, const bf16x8* cb, bf16x8* na, bf16x8* nb, int rkt, int rkk,
                         bool dma, int dkt, int q0, int q1) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJF; ++j) {
        const int u = i * NJF + j;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cb[j], ca[i], acc[i][j], 0, 0, 0);
        if (u < 4) na[u] = read_a(rkt, rkk, u);
        else if (u < 4 + NJF) nb[u - 4] = read_b(rkt, rkk, u - 4);
        if constexpr (UNCOND) {
          if (u < q1 - q0) dma_to(dkt < nk ? dkt : nk - 1, dkt, q0 + u);
        } else {
          if (dma && u < q1 - q0) dma_one(dkt, q0 + u);
        }
      }
    substep_schedule<4 + NJF, 4 * NJF>();
  };
  for (int kt = 0; kt < nk - 1; ++kt) {
#pragma unroll
    for (int kk = 0; kk < KS - 1; ++kk) {
      if (kk < DSP - 1) {
        // continue the requests of k-tile kt-1+S begun in k-tile kt-1
        const int q0 = (kk + 1) * PER, q1 = (kk + 2) * PER < G ? (kk + 2) * PER : G;
        substep_dma(fa[kk & 1], fb[kk & 1], fa[(kk + 1) & 1], fb[(kk + 1) & 1], kt, kk + 1,
                    (UNCOND || kt >= 1) && kt - 1 + S < nk, kt - 1 + S, q0, q1);
        continue;
      }
      read_frags(kt, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
      if (FMT != 0 && kk == KS - 2) {
        wait_vm(0);  // A DMA and raw codes of k-tile kt+1 have landed
        store_b(kt + 1);
      }
      mfmas(fa[kk & 1], fb[kk & 1]);
      if constexpr (FMT == 0) substep_schedule<4 + NJF, 4 * NJF>();
    }
    if constexpr (FMT == 0) {
      int ahead = nk - 2 - kt;
      ahead = ahead < S - 2 ? ahead : S - 2;
      wait_vm(G * (ahead > 0 ? ahead : 0));
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's reads of k-tile kt (and B writes) are done
    barrier();
    const bool more = kt + S < nk;
    constexpr int L = (KS - 1) & 1, X = KS & 1;
    substep_dma(fa[L], fb[L], fa[X], fb[X], kt + 1, 0, more, kt + S, 0, PER < 4 * NJF ? PER : 4 * NJF);
    if constexpr (PER > 4 * NJF) {
      if (more) {
#pragma unroll
        for (int q = 4 * NJF; q < PER; ++q) dma_one(kt + S, q);
      }
    }
    if constexpr (FMT != 0) {
      if (more) load_braw(kt + S);
    }
  }
  // Last k-tile; column-major MFMA order keeps this tail distinct from the
  // loop body, which the compiler would otherwise fold back into the loop.
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    if (kk + 1 < KS) read_frags(nk - 1, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
#pragma unroll
    for (int j = 0; j < NJF; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[kk & 1][j], fa[kk & 1][i], acc[i][j], 0, 0, 0);
  }

  // every wave has finished reading the operand stages and no request is
  // still writing one: LDS is free
  wait_vm(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  barrier();
  if constexpr (EPI == EPI_QKV || EPI == EPI_SPLIT_QKV) {
    // q | k and v columns (tile-aligned: qk_h is a multiple of the tile
    // width) take the fused epilogues; the rest is a plain or split store
    if (n0 < 2 * P.qk_h) {
      if constexpr (TN == 128) qk_epilogue<TN>(P, smem, m0 + wm0, n0 + wn0, wave, lane, acc);
    } else if (n0 < 3 * P.qk_h) {
      if constexpr (TN == 128) v_epilogue<TN>(P, smem, m0 + wm0, n0 + wn0, wave, lane, acc);
    } else if constexpr (EPI == EPI_QKV) {
      dma_epilogue<EPI_STORE, TN>(P, smem, m0 + wm0, n0 + wn0, wave, lane, acc, 0, ebias);
    } else {
      dma_epilogue<EPI_SPLIT, TN>(P, smem, m0 + wm0, n0 + wn0, wave, lane, acc, split_side_of(P, n0, kDBN), ebias);
    }
  } else {
    const int side = EPI == EPI_SPLIT ? split_side_of(P, n0, kDBN) : EPI == EPI_PARTIAL ? ks : 0;
    dma_epilogue<EPI, TN>(P, smem, m0 + wm0, n0 + wn0, wave, lane, acc, side, ebias);
  }
}

// Tile-loop configuration used by the library.
#ifndef MMDIT_DMA_BK
#define MMDIT_DMA_BK 64
#endif
#ifndef MMDIT_DMA_STAGES
#define MMDIT_DMA_STAGES 2
#endif
#ifndef MMDIT_DMA_CPOL
#define MMDIT_DMA_CPOL 0
#endif
#ifndef MMDIT_DMA_SPREAD
#define MMDIT_DMA_SPREAD 3
#endif
#ifndef MMDIT_DMA_WAVES
#define MMDIT_DMA_WAVES 4
#endif
constexpr int kDBK = MMDIT_DMA_BK;

template <int EPI, int BK = MMDIT_DMA_BK, int S = MMDIT_DMA_STAGES, int CPOL = MMDIT_DMA_CPOL, int FMT = 0,
          int DS = MMDIT_DMA_SPREAD, int W = MMDIT_DMA_WAVES>
static hipError_t launch_dma_epi(const GemmProblem* p, int nprob, hipStream_t s) {
  GemmBatch gb{};
  int total = 0;
  for (int i = 0; i < 2; ++i) {
    if (i < nprob) {
      gb.p[i] = p[i];
      gb.tiles_m[i] = (p[i].M + kDBM - 1) / kDBM;
      gb.tiles_n[i] = (p[i].N + kDBN - 1) / kDBN;
      total += gb.tiles_m[i] * gb.tiles_n[i];
    } else {
      gb.tiles_m[i] = 1;
      gb.tiles_n[i] = 1;
    }
    gb.tile_start[i + 1] = total;
  }
  if (total == 0) return hipSuccess;
  const size_t lds = (size_t)S * 2 * kDBM * BK * 2;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = ensure_lds_limit((const void*)k_gemm_dma<EPI, BK, S, CPOL, FMT, DS, W>, (int)lds, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_dma<EPI, BK, S, CPOL, FMT, DS, W>), dim3(total), dim3(64 * W), lds, s, gb);
  return hipGetLastError();
}

static bool aligned(const void* p, int bytes) { return ((uintptr_t)p % bytes) == 0; }

int64_t gemm_dma_tiles(int M, int N) { return (int64_t)((M + kDBM - 1) / kDBM) * ((N + kDBN - 1) / kDBN); }

// Launches with fewer 256 x 256 tiles than this leave too many of the 256 CUs
// idle for the direct-to-LDS kernel (one tile per CU); they run on the
// 128 / 64-row tiles of the register-staged kernel, or split along k.
#ifndef MMDIT_DMA_MIN_TILES
#define MMDIT_DMA_MIN_TILES 128
#endif
constexpr int64_t kDmaMinTiles = MMDIT_DMA_MIN_TILES;

// True when the DMA kernel can run the launch: no Euler epilogue, one weight
// format per launch, K a multiple of the k-tile, rows of A 16-byte aligned,
// N >= 128, column counts, row strides and base pointers of every output
// (and of bias, gate and residual) aligned for 4-column vector access, and a
// tile-aligned split column (split epilogue). Sets the launch's tile count.
static bool dma_shape_ok(const GemmProblem* p, int nprob, int epi, int64_t& tiles) {
  if (epi == EPI_EULER) return false;
  tiles = 0;
  int fmt = -1;
  for (int i = 0; i < nprob; ++i) {
    const GemmProblem& q = p[i];
    if (q.M == 0) continue;
    if (fmt >= 0 && q.fmt != fmt) return false;  // one format per launch
    fmt = q.fmt;
    if (q.K % kDBK != 0 || q.lda % 8 != 0 || q.N < 128 || q.N % 4 != 0) return false;
    // per-lane operand offsets are 32-bit
    if ((int64_t)q.M * q.lda * 2 >= (int64_t(1) << 32) || (int64_t)q.N * q.K * 2 >= (int64_t(1) << 32)) return false;
    if (fmt != 0 && (kDBK != 64 || MMDIT_DMA_STAGES != 2)) return false;
    if ((epi == EPI_QKV || epi == EPI_SPLIT_QKV) &&
        (fmt != 0 || MMDIT_DMA_WAVES != 4 || q.qk_h % kDBN != 0 || 3 * q.qk_h > q.N || q.qk_rows <= 0))
      return false;
    if ((fmt == 3 || fmt == 4) && q.K % 128 != 0) return false;
    if (q.bias && !aligned(q.bias, 8)) return false;
    if (epi == EPI_GATE_RES) {
      const int esz = q.res_f32 ? 16 : 8;
      if (q.res_in.ld % 4 || q.res_out.ld % 4 || q.res_in.batch_stride % 4 || q.res_out.batch_stride % 4 ||
          q.gate_bstride % 4 || !aligned(q.res_in.base, esz) || !aligned(q.res_out.base, esz) ||
          !aligned(q.gate, 16) || q.res_in.rows_per_batch <= 0 || q.res_out.rows_per_batch <= 0)
        return false;
    } else {
      if (q.out_f32 || q.ldo % 4 || !aligned(q.out, 8)) return false;  // bf16 outputs only
      if ((epi == EPI_SPLIT || epi == EPI_SPLIT_QKV) && (q.split_n % kDBN != 0 || q.ldo2 % 4 || !aligned(q.out2, 8)))
        return false;
    }
    tiles += gemm_dma_tiles(q.M, q.N);
  }
  return true;
}

// The DMA kernel takes the launch whole when its shape allows and it has
// enough tiles to occupy most of the CUs.
bool gemm_dma_eligible(const GemmProblem* p, int nprob, int epi) {
  int64_t tiles = 0;
  return dma_shape_ok(p, nprob, epi, tiles) && tiles >= kDmaMinTiles;
}

// Split-K: k-ranges of at least kSplitMinKTiles k-tiles, at most kMaxSplit
// ranges, and no more units than one per CU.
constexpr int kMaxSplit = 4, kSplitMinKTiles = 8, kSplitUnits = 256;

int splitk_ways(int64_t tiles, int K) {
  if (tiles <= 0 || tiles >= kDmaMinTiles) return 1;
  int64_t w = kSplitUnits / tiles;
  if (w > kMaxSplit) w = kMaxSplit;
  const int64_t byk = (int64_t)(K / kDBK) / kSplitMinKTiles;
  if (w > byk) w = byk;
  return w >= 2 ? (int)w : 1;
}

int gemm_splitk_ways(const GemmProblem* p, int nprob, int epi) {
  int64_t tiles = 0;
  if (epi != EPI_GATE_RES || !dma_shape_ok(p, nprob, epi, tiles)) return 1;
  int K = 0;
  for (int i = 0; i < nprob; ++i) {
    if (p[i].M == 0) continue;
    if (p[i].fmt != 0) return 1;  // dense weights only
    K = K == 0 || p[i].K < K ? p[i].K : K;
  }
  return splitk_ways(tiles, K);
}

// Split-K completion of the gated residual: v = bias + the k-ranges' partial
// sums added in range order, res_out = res_in + gate[b, n] * v. One thread
// per 4 consecutive columns of a row (column counts, strides and pointers
// are 4-column aligned, as the DMA kernel requires).
__global__ __launch_bounds__(256) void k_splitk_gate_res(GemmBatch gb) {
  if (guard_skip(gb.p[0].skip)) return;
  const int64_t q0 = (int64_t)gb.p[0].M * (gb.p[0].N / 4);
  const int64_t q1 = (int64_t)gb.p[1].M * (gb.p[1].N / 4);
  int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= q0 + q1) return;
  const int prob = q < q0 ? 0 : 1;
  if (prob) q -= q0;
  const GemmProblem& P = gb.p[prob];
  const int nq = P.N / 4;
  const int m = (int)(q / nq), n = (int)(q - (int64_t)m * nq) * 4;
  const int64_t mn = (int64_t)P.M * P.N;
  const float* src = P.part + (int64_t)m * P.N + n;
  f32x4 v = *reinterpret_cast<const f32x4*>(src);
  for (int k = 1; k < gb.ksplit; ++k) {
    const f32x4 w = *reinterpret_cast<const f32x4*>(src + k * mn);
    v = v + w;
  }
  if (P.bias) {
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(P.bias) + n);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += (float)b[e];
  }
  const int b = m / P.res_out.rows_per_batch;
  const f32x4 g = *reinterpret_cast<const f32x4*>(P.gate + (int64_t)b * P.gate_bstride + n);
  const int64_t oi = seg_offset<bf16>(P.res_in, m) + n;
  const int64_t oo = seg_offset<bf16>(P.res_out, m) + n;
  if (P.res_f32) {
    const f32x4 r = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(P.res_in.base) + oi);
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = r[e] + g[e] * v[e];
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(P.res_out.base) + oo) = o;
  } else {
    const bf16x4 r = *reinterpret_cast<const bf16x4*>(reinterpret_cast<const bf16*>(P.res_in.base) + oi);
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (bf16)((float)r[e] + g[e] * v[e]);
    *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(P.res_out.base) + oo) = o;
  }
}

// Quantised weights run with eight wavefronts (two per SIMD): each
// wavefront's dequantisation (VALU work that does not overlap its own MFMAs)
// then runs beside the other wavefront's MFMAs on the same SIMD. With four
// wavefronts the conversion adds 23-50 % to the dense time at 4608 rows; with
// eight, 12-30 %.
template <int EPI>
static hipError_t launch_dma_fmt(const GemmProblem* p, int nprob, hipStream_t s) {
  int fmt = 0;
  for (int i = 0; i < nprob; ++i)
    if (p[i].M > 0) fmt = p[i].fmt;
  switch (fmt) {
    case 1: return launch_dma_epi<EPI, MMDIT_DMA_BK, MMDIT_DMA_STAGES, MMDIT_DMA_CPOL, 1, MMDIT_DMA_SPREAD, 8>(p, nprob, s);
    case 2: return launch_dma_epi<EPI, MMDIT_DMA_BK, MMDIT_DMA_STAGES, MMDIT_DMA_CPOL, 2, MMDIT_DMA_SPREAD, 8>(p, nprob, s);
    case 3: return launch_dma_epi<EPI, MMDIT_DMA_BK, MMDIT_DMA_STAGES, MMDIT_DMA_CPOL, 3, MMDIT_DMA_SPREAD, 8>(p, nprob, s);
    case 4: return launch_dma_epi<EPI, MMDIT_DMA_BK, MMDIT_DMA_STAGES, MMDIT_DMA_CPOL, 4, MMDIT_DMA_SPREAD, 8>(p, nprob, s);
    default: return launch_dma_epi<EPI>(p, nprob, s);
  }
}

hipError_t launch_gemm_dma(const GemmProblem* p, int nprob, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_dma_fmt<EPI_STORE>(p, nprob, s);
    case EPI_GELU: return launch_dma_fmt<EPI_GELU>(p, nprob, s);
    case EPI_GATE_RES: return launch_dma_fmt<EPI_GATE_RES>(p, nprob, s);
    case EPI_SPLIT: return launch_dma_fmt<EPI_SPLIT>(p, nprob, s);
    case EPI_QKV: return launch_dma_epi<EPI_QKV>(p, nprob, s);
    case EPI_SPLIT_QKV: return launch_dma_epi<EPI_SPLIT_QKV>(p, nprob, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_dma_splitk(const GemmProblem* p, int nprob, int epi, int ways, float* part, hipStream_t s) {
  if (epi != EPI_GATE_RES || ways < 2 || nprob < 1 || nprob > 2) return hipErrorInvalidValue;
  GemmBatch gb{};
  int tiles = 0;
  int64_t quads = 0;
  size_t at = 0;
  for (int i = 0; i < 2; ++i) {
    if (i < nprob) {
      gb.p[i] = p[i];
      gb.p[i].part = part + at;
      at += (size_t)ways * p[i].M * p[i].N;
      gb.tiles_m[i] = (p[i].M + kDBM - 1) / kDBM;
      gb.tiles_n[i] = (p[i].N + kDBN - 1) / kDBN;
      tiles += gb.tiles_m[i] * gb.tiles_n[i];
      quads += (int64_t)p[i].M * (p[i].N / 4);
    } else {
      gb.tiles_m[i] = 1;
      gb.tiles_n[i] = 1;
    }
    gb.tile_start[i + 1] = tiles;
  }
  gb.ksplit = ways;
  if (tiles == 0) return hipSuccess;
  constexpr int BK = MMDIT_DMA_BK, S = MMDIT_DMA_STAGES;
  const size_t lds = (size_t)S * 2 * kDBM * BK * 2;
  static std::atomic<uint64_t> lds_set{0};
  const void* kfn = (const void*)k_gemm_dma<EPI_PARTIAL, BK, S, MMDIT_DMA_CPOL, 0, MMDIT_DMA_SPREAD, MMDIT_DMA_WAVES>;
  const hipError_t e = ensure_lds_limit(kfn, (int)lds, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_gemm_dma<EPI_PARTIAL, BK, S, MMDIT_DMA_CPOL, 0, MMDIT_DMA_SPREAD, MMDIT_DMA_WAVES>),
                     dim3(tiles * ways), dim3(64 * MMDIT_DMA_WAVES), lds, s, gb);
  hipLaunchKernelGGL(k_splitk_gate_res, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, s, gb);
  return hipGetLastError();
}

}  // namespace mmdit
