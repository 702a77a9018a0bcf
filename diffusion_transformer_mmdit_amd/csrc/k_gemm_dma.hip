// Dense bf16 GEMM C = A W^T for the large projections (gfx950).
//
// 256 x 256 block tile, K-tile 32, 4 wavefronts (2 x 2, 128 x 128 each) on
// v_mfma_f32_32x32x16_bf16 with the accumulators in AGPRs.
//
// Operand tiles move HBM -> LDS with the gfx950 direct-to-LDS load
// (global_load_lds_dwordx4): no VGPR staging and no LDS store instructions.
// LDS holds 4 stages (4 x 32 KB); the tile for k-step kt+3 is requested while
// k-step kt is multiplied, so each load has about two k-steps (~2000 MFMA
// cycles) to arrive. One barrier per k-step; it sits between the two 16-deep
// halves of the k-step so that the fragment reads of the next stage overlap
// the MFMAs of the current one.
//
// LDS layout: each 64-byte row (32 bf16 of one M or N index) is stored as four
// 16-byte chunks in the order c ^ f(r), f(r) = ((r >> 1) ^ (r >> 2)) & 3, so the
// 16-byte fragment reads of consecutive rows fall in distinct banks (for 32 and
// for 64 banks). The swizzle is applied on the load side: lane i of a DMA
// instruction writes slot i, so it fetches the global chunk destined for that slot.
#include "gemm_common.h"

namespace mmdit {

constexpr int kDBM = 256, kDBN = 256, kDBK = 32;
constexpr int kStageBytes = (kDBM + kDBN) * kDBK * 2;  // 32 KB
constexpr int kStages = 4;

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// 64 lanes each copy 16 bytes from gptr (per lane) to LDS at m0_base + 16 * lane.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t m0_base) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(m0_base), "v"(gptr)
      : "memory", "m0");
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt unconstrained), n <= 63.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ int swz(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

template <int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm_dma(GemmBatch gb) {
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  int prob, tm, tn;
  tile_of(gb, prob, tm, tn);
  const GemmProblem& P = gb.p[prob];
  const int M = P.M, N = P.N, K = P.K;
  const int m0 = tm * kDBM, n0 = tn * kDBN;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm0 = (wave >> 1) * 128, wn0 = (wave & 1) * 128;
  const uint32_t lds0 = lds_offset(smem);

  // Per-lane global source of each of the 4 A and 4 B DMA instructions
  // (row offsets fixed for the whole K loop; the k offset advances).
  const bf16* A = reinterpret_cast<const bf16*>(P.A);
  const bf16* W = reinterpret_cast<const bf16*>(P.W);
  const bf16* asrc[4];
  const bf16* bsrc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int s = (wave * 4 + j) * 64 + lane;  // slot (16 B) within the 256-row tile
    const int r = s >> 2, c = (s & 3) ^ swz(s >> 2);
    int gm = m0 + r;
    gm = gm < M ? gm : M - 1;  // rows past the edge re-read a valid row; their outputs are dropped
    int gn = n0 + r;
    gn = gn < N ? gn : N - 1;
    asrc[j] = A + (int64_t)gm * P.lda + c * 8;
    bsrc[j] = W + (int64_t)gn * K + c * 8;
  }
  auto issue = [&](int kt) {
    const uint32_t st = lds0 + (uint32_t)((kt & (kStages - 1)) * kStageBytes);
    const int k0 = kt * kDBK;
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(asrc[j] + k0, st + (uint32_t)((wave * 4 + j) * 1024));
#pragma unroll
    for (int j = 0; j < 4; ++j) dma16(bsrc[j] + k0, st + 16384u + (uint32_t)((wave * 4 + j) * 1024));
  };

  // Fragment read offsets (bytes, within a stage) for k-half kk: A rows
  // wm0 + 32i + lane%32, chunk 2kk + lane/32; B likewise with wn0.
  uint32_t aoff[2][4], boff[2][4];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ra = wm0 + i * 32 + (lane & 31);
      const int rb = wn0 + i * 32 + (lane & 31);
      const int c = kk * 2 + (lane >> 5);
      aoff[kk][i] = (uint32_t)((ra * 4 + (c ^ swz(ra))) * 16);
      boff[kk][i] = 16384u + (uint32_t)((rb * 4 + (c ^ swz(rb))) * 16);
    }
  auto read_frags = [&](int kt, int kk, bf16x8* fa, bf16x8* fb) {
    const char* st = smem + (kt & (kStages - 1)) * kStageBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const bf16x8*>(st + aoff[kk][i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) fb[i] = *reinterpret_cast<const bf16x8*>(st + boff[kk][i]);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
  auto mfmas = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  const int nk = K / kDBK;
  // prologue: tiles 0, 1, 2 requested; wait for tile 0
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
  if (nk > 2) wait_vm<16>();
  else if (nk > 1) wait_vm<8>();
  else wait_vm<0>();
  barrier();
  bf16x8 fa0[4], fb0[4], fa1[4], fb1[4];
  read_frags(0, 0, fa0, fb0);
  // every k-step but the last: the barrier path is unconditional inside the
  // loop so the waits the compiler derives for the fragment registers do
  // not merge with the last step's
  for (int kt = 0; kt < nk - 1; ++kt) {
    read_frags(kt, 1, fa1, fb1);
    mfmas(fa0, fb0);
    // tile kt+1 must have landed; tile kt+2 may still be in flight
    if (kt + 2 < nk) wait_vm<8>();
    else wait_vm<0>();
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's stage-kt reads are done
    barrier();
    if (kt + 3 < nk) issue(kt + 3);
    read_frags(kt + 1, 0, fa0, fb0);
    mfmas(fa1, fb1);
  }
  // last k-step; column-major MFMA order keeps this tail distinct from the
  // loop body, which the compiler would otherwise fold back into the loop
  read_frags(nk - 1, 1, fa1, fb1);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa0[i], fb0[j], acc[i][j], 0, 0, 0);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa1[i], fb1[j], acc[i][j], 0, 0, 0);

  // acc[i][j][r] = C[m0 + wm0 + 32i + 8(r/4) + 4(lane/32) + r%4][n0 + wn0 + 32j + lane%32]
  const int bu = EPI == EPI_GATE_RES ? tile_batch(P, m0, kDBM) : 0;
  const int side = EPI == EPI_SPLIT ? split_side_of(P, n0, kDBN) : 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + wn0 + j * 32 + (lane & 31);
    const bool n_ok = n < N;
    const int nc = n_ok ? n : N - 1;
    const float bias = P.bias ? (float)reinterpret_cast<const bf16*>(P.bias)[nc] : 0.f;
    const float gate = (EPI == EPI_GATE_RES && bu >= 0) ? P.gate[(int64_t)bu * P.gate_bstride + nc] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (n_ok) epi_block_bf16<EPI, false>(P, m0 + wm0 + i * 32 + 4 * (lane >> 5), n, acc[i][j], bias, gate, bu >= 0, side);
  }
}

template <int EPI>
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
  const size_t lds = (size_t)kStages * kStageBytes;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)k_gemm_dma<EPI>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(k_gemm_dma<EPI>, dim3(total), dim3(256), lds, s, gb);
  return hipGetLastError();
}

// True when the DMA kernel applies: dense weights, K a multiple of 32, rows of
// A 16-byte aligned, N >= 128, contiguous residual rows (gated epilogue), a
// tile-aligned split column (split epilogue), and enough 256 x 256 tiles to
// occupy most of the 256 CUs.
bool gemm_dma_eligible(const GemmProblem* p, int nprob, int epi) {
  if (epi == EPI_EULER) return false;
  int64_t tiles = 0;
  for (int i = 0; i < nprob; ++i) {
    if (p[i].M == 0) continue;
    if (p[i].fmt != 0 || p[i].K % kDBK != 0 || p[i].lda % 8 != 0 || p[i].N < 128) return false;
    // the epilogue here has only the contiguous-residual and tile-aligned split paths
    if (epi == EPI_GATE_RES && (p[i].res_in.rows_per_batch < p[i].M || p[i].res_out.rows_per_batch < p[i].M))
      return false;
    if (epi == EPI_SPLIT && p[i].split_n % kDBN != 0) return false;
    tiles += (int64_t)((p[i].M + kDBM - 1) / kDBM) * ((p[i].N + kDBN - 1) / kDBN);
  }
  return tiles >= 200;
}

hipError_t launch_gemm_dma(const GemmProblem* p, int nprob, int epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return launch_dma_epi<EPI_STORE>(p, nprob, s);
    case EPI_GELU: return launch_dma_epi<EPI_GELU>(p, nprob, s);
    case EPI_GATE_RES: return launch_dma_epi<EPI_GATE_RES>(p, nprob, s);
    case EPI_SPLIT: return launch_dma_epi<EPI_SPLIT>(p, nprob, s);
    default: return launch_dma_epi<EPI_EULER>(p, nprob, s);
  }
}

}  // namespace mmdit
