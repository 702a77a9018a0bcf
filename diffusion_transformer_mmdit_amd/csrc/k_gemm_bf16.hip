// bf16 GEMM C = A W^T on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16),
// float32 accumulation, fused epilogues. Used for every projection of the
// block: QKV / linear1, attention out-projection, MLP fc1 / fc2, linear2,
// the input projections and the final layer.
//
// Weights may be dense bf16 or group-quantised (4-bit or 8-bit codes, one
// bf16 scale per 64 consecutive k). Quantised weights are dequantised one
// K-tile at a time while being staged into LDS, so the MFMA loop is the same
// for every format (stable-diffusion.rs README: weights held as packed bits
// and dequantised inside the matmul a tile at a time).
//
// Structure: BM x BN block tile, K-tile 64, 4 wavefronts in a WM x WN grid,
// LDS double buffer with one barrier per K-tile; global loads for tile k+1
// are issued before the MFMAs of tile k. LDS rows are padded to 72 elements
// (144 bytes) so the 16-byte fragment reads of 8 consecutive rows hit
// distinct banks.
#include "gemm_common.h"

namespace mmdit {

constexpr int kBK = 64;
constexpr int kLDK = kBK + 8;

template <int BM, int BN, int WM, int WN, int EPI, int FMT>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmBatch gb) {
  if (guard_skip(gb.p[0].skip)) return;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_CH = BM * 8 / 256;                                  // 16-byte A chunks per thread
  // 16-byte B chunks per thread; sub-byte formats (3, 4): pieces of 32 weights
  constexpr bool SUB = FMT == 3 || FMT == 4;
  constexpr int B_CH = FMT == 0 ? BN * 8 / 256 : (FMT == 2 ? BN * 4 / 256 : BN * 2 / 256);
  static_assert(WM * WN == 4, "4 wavefronts");
  static_assert(B_CH >= 1, "tile too small for this weight format");
  __shared__ bf16 As[2][BM * kLDK];
  __shared__ bf16 Bs[2][BN * kLDK];

  int prob, tm, tn;
  tile_of(gb, prob, tm, tn);
  const GemmProblem& P = gb.p[prob];
  const int M = P.M, N = P.N, K = P.K;
  const int m0 = tm * BM, n0 = tn * BN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm0 = (wave / WN) * TM, wn0 = (wave % WN) * TN;
  const bf16* A = reinterpret_cast<const bf16*>(P.A);

  bf16x8 ra[A_CH];
  u32x4 rb[B_CH];
  float rs[B_CH];
  uint32_t rq[B_CH][2], rqs[B_CH];  // sub-byte piece i: row c / 2, weights 32 (c % 2) ..

  auto load_tile = [&](int kt) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * 256;
      const int row = c >> 3, kc = c & 7;
      const int gm = m0 + row;
      ra[i] = gm < M ? *reinterpret_cast<const bf16x8*>(A + (int64_t)gm * P.lda + k0 + kc * 8) : (bf16x8){};
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * 256;
      if constexpr (SUB) {
        const int gn = n0 + (c >> 1), half = c & 1;
        const uint8_t* wq = reinterpret_cast<const uint8_t*>(P.W);
        if (gn < N) {
          rqs[i] = reinterpret_cast<const uint16_t*>(P.scales)[(int64_t)gn * (K / 128) + kt / 2];
          if constexpr (FMT == 3) {
            rq[i][0] = *reinterpret_cast<const uint32_t*>(wq + (int64_t)gn * (K / 8) + k0 / 8 + half * 4);
            rq[i][1] = 0;
          } else {
            const uint2 v = *reinterpret_cast<const uint2*>(wq + (int64_t)gn * (K / 4) + k0 / 4 + half * 8);
            rq[i][0] = v.x;
            rq[i][1] = v.y;
          }
        } else {
          rqs[i] = 0;
          rq[i][0] = rq[i][1] = 0;
        }
      } else if constexpr (FMT == 0) {
        const int row = c >> 3, kc = c & 7;
        const int gn = n0 + row;
        rb[i] = gn < N ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16*>(P.W) + (int64_t)gn * K + k0 + kc * 8)
                       : (u32x4){0, 0, 0, 0};
      } else if constexpr (FMT == 2) {
        const int row = c >> 2, part = c & 3;
        const int gn = n0 + row;
        if (gn < N) {
          rb[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const int8_t*>(P.W) + (int64_t)gn * K + k0 + part * 16);
          rs[i] = (float)reinterpret_cast<const bf16*>(P.scales)[(int64_t)gn * (K / 64) + kt];
        } else {
          rb[i] = (u32x4){0, 0, 0, 0};
          rs[i] = 0.f;
        }
      } else {
        const int row = c >> 1, part = c & 1;
        const int gn = n0 + row;
        if (gn < N) {
          rb[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(P.W) + (int64_t)gn * (K / 2) + k0 / 2 + part * 16);
          rs[i] = (float)reinterpret_cast<const bf16*>(P.scales)[(int64_t)gn * (K / 64) + kt];
        } else {
          rb[i] = (u32x4){0, 0, 0, 0};
          rs[i] = 0.f;
        }
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = tid + i * 256;
      *reinterpret_cast<bf16x8*>(&As[buf][(c >> 3) * kLDK + (c & 7) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = tid + i * 256;
      if constexpr (SUB) {
        bf16x8 o[4];
        if constexpr (FMT == 3) deq_q1_32(rq[i][0], rqs[i], o);
        else deq_tq2_32(rq[i][0], rq[i][1], rqs[i], o);
        bf16* d = &Bs[buf][(c >> 1) * kLDK + (c & 1) * 32];
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<bf16x8*>(d + 8 * j) = o[j];
      } else if constexpr (FMT == 0) {
        *reinterpret_cast<u32x4*>(&Bs[buf][(c >> 3) * kLDK + (c & 7) * 8]) = rb[i];
      } else if constexpr (FMT == 2) {
        bf16x8 lo, hi;
        deq8(rb[i], rs[i], lo, hi);
        bf16* d = &Bs[buf][(c >> 2) * kLDK + (c & 3) * 16];
        *reinterpret_cast<bf16x8*>(d) = lo;
        *reinterpret_cast<bf16x8*>(d + 8) = hi;
      } else {
        bf16x8 o[4];
        deq4(rb[i], rs[i], o);
        bf16* d = &Bs[buf][(c >> 1) * kLDK + (c & 1) * 32];
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<bf16x8*>(d + 8 * j) = o[j];
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = (f32x16){};

  const int nk = K / kBK;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tile(kt + 1);
    const bf16* as = As[cur];
    const bf16* bs = Bs[cur];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 af[FM], bfr[FN];
      const int koff = kk * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&as[(wm0 + i * 32 + (lane & 31)) * kLDK + koff]);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&bs[(wn0 + j * 32 + (lane & 31)) * kLDK + koff]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tile(cur ^ 1);
    __syncthreads();
  }

  // acc[i][j][r] holds C[m0 + wm0 + 32i + 8(r/4) + 4(lane/32) + r%4][n0 + wn0 + 32j + lane%32]
  const int bu = EPI == EPI_GATE_RES ? tile_batch(P, m0, BM) : 0;
  const int side = EPI == EPI_SPLIT ? split_side_of(P, n0, BN) : 0;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn0 + j * 32 + (lane & 31);
    const bool n_ok = n < N;
    const int nc = n_ok ? n : N - 1;
    const float bias = P.bias ? (float)reinterpret_cast<const bf16*>(P.bias)[nc] : 0.f;
    const float gate = (EPI == EPI_GATE_RES && bu >= 0) ? P.gate[(int64_t)bu * P.gate_bstride + nc] : 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (n_ok) epi_block_bf16<EPI, true>(P, m0 + wm0 + i * 32 + 4 * (lane >> 5), n, acc[i][j], bias, gate, bu >= 0, side);
  }
}

// ------------------------------------------------------------------ launch --
template <int BM, int BN, int WM, int WN, int EPI, int FMT>
static hipError_t launch_cfg(const GemmProblem* p, int nprob, hipStream_t s) {
  GemmBatch gb{};
  int total = 0;
  gb.tile_start[0] = 0;
  for (int i = 0; i < 2; ++i) {
    if (i < nprob) {
      gb.p[i] = p[i];
      gb.tiles_m[i] = (p[i].M + BM - 1) / BM;
      gb.tiles_n[i] = (p[i].N + BN - 1) / BN;
      total += gb.tiles_m[i] * gb.tiles_n[i];
    } else {
      gb.tiles_m[i] = 1;
      gb.tiles_n[i] = 1;
    }
    gb.tile_start[i + 1] = total;
  }
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm_bf16<BM, BN, WM, WN, EPI, FMT>), dim3(total), dim3(256), 0, s, gb);
  return hipGetLastError();
}

template <int EPI, int FMT>
static hipError_t launch_epi_fmt(const GemmProblem* p, int nprob, hipStream_t s) {
  // dense weights take 64 x 64 tiles for narrow outputs and whenever 128 x 128
  // tiles would leave CUs idle (e.g. the text projection: 512 x 3072 is 96
  // tiles of 128 x 128 but 384 of 64 x 64)
  int64_t tiles128 = 0;
  int maxN = 0;
  for (int i = 0; i < nprob; ++i) {
    tiles128 += (int64_t)((p[i].M + 127) / 128) * ((p[i].N + 127) / 128);
    if (p[i].N > maxN) maxN = p[i].N;
  }
  if constexpr (FMT == 0) {
    if (maxN <= 64 || tiles128 < 256) return launch_cfg<64, 64, 2, 2, EPI, FMT>(p, nprob, s);
  }
  return launch_cfg<128, 128, 2, 2, EPI, FMT>(p, nprob, s);
}

// One weight format per launch: the format of the first problem with rows
// (a problem without rows launches no tiles, whatever its format).
template <int EPI>
static hipError_t launch_epi(const GemmProblem* p, int nprob, hipStream_t s) {
  int fmt = p[0].fmt;
  if (nprob > 1 && p[0].M == 0) fmt = p[1].fmt;
  switch (fmt) {
    case 0: return launch_epi_fmt<EPI, 0>(p, nprob, s);
    case 1: return launch_epi_fmt<EPI, 1>(p, nprob, s);
    case 3: return launch_epi_fmt<EPI, 3>(p, nprob, s);
    case 4: return launch_epi_fmt<EPI, 4>(p, nprob, s);
    default: return launch_epi_fmt<EPI, 2>(p, nprob, s);
  }
}

hipError_t launch_gemm_bf16(const GemmProblem* p, int nprob, int epi, hipStream_t s) {
  // problems with rows in different weight formats (e.g. a dense text stream
  // beside a quantised image stream) run as one launch each
  if (nprob == 2 && p[0].M > 0 && p[1].M > 0 && p[0].fmt != p[1].fmt) {
    const hipError_t e = launch_gemm_bf16(p, 1, epi, s);
    return e != hipSuccess ? e : launch_gemm_bf16(p + 1, 1, epi, s);
  }
  switch (epi) {
    case EPI_STORE: return launch_epi<EPI_STORE>(p, nprob, s);
    case EPI_GELU: return launch_epi<EPI_GELU>(p, nprob, s);
    case EPI_GATE_RES: return launch_epi<EPI_GATE_RES>(p, nprob, s);
    case EPI_SPLIT: return launch_epi<EPI_SPLIT>(p, nprob, s);
    case EPI_EULER: return launch_epi<EPI_EULER>(p, nprob, s);
    default: return hipErrorInvalidValue;  // fused QK epilogues: direct-to-LDS kernel only
  }
}

}  // namespace mmdit
