// Launchers of the gfx950 kernels (host side). Each returns the hipError_t
// of its launch. Sizes are validated by the callers in api.cpp before any
// launch; the launchers themselves assume valid arguments.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace mmdit {

// Raises the dynamic-LDS limit of kernel `fn` to `bytes` on the current
// device, once per device (`done` holds one bit per device id). Safe to call
// from several threads: a thread that races another repeats the call, which
// is harmless.
inline hipError_t ensure_lds_limit(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  done.fetch_or(bit, std::memory_order_release);
  return hipSuccess;
}

// A set of activation rows split in up to two segments (text rows, then
// image rows). Row r of segment s belongs to batch r / rows_per_batch and
// sits at base + (r / rows_per_batch) * batch_stride + (r % rows_per_batch) * ld
// (strides in elements).
struct RowSeg {
  void* base;
  int64_t batch_stride;
  int32_t rows_per_batch;
  int32_t ld;
};

// ---- adaLN modulated LayerNorm -------------------------------------------
// y[r, :] = (1 + scale_b) * LN(x[r, :]) + shift_b for r in [0, rows) where the
// first seg_rows[0] rows come from seg[0] and the rest from seg[1]; y is
// contiguous [rows, h]. shift/scale for row r of segment s:
// mod[s] + b * mod_bstride + shift_off / scale_off.
struct LnArgs {
  RowSeg seg[2];
  int32_t seg_rows[2];
  const float* mod[2];
  int32_t mod_bstride;
  int32_t shift_off, scale_off;
  void* y;
  int32_t h;
  float eps;
  const int* skip = nullptr;  // step-cache guard (see guard_skip), null: always run
};
// x_f32: residual rows are float32 (else the activation type);
// y_bf16: output bf16 (else float32).
hipError_t launch_adaln_ln(const LnArgs& a, int rows, bool x_f32, bool y_bf16, hipStream_t s);

// ---- step-cache indicator -------------------------------------------------------
// For each of `rows` contiguous float32 rows x[r, :] (batch r / rows_per_batch):
// a = (1 + scale_b) * LN(x[r, :]) + shift_b with shift_b = mod + b * mod_bstride,
// scale_b = shift_b + h; part[2r] = sum |a - prev[r, :]|, part[2r + 1] =
// sum |prev[r, :]| (not written when first != 0); then prev[r, :] = a.
struct CacheDeltaArgs {
  const float* x;
  const float* mod;
  int32_t mod_bstride;
  int32_t rows_per_batch;
  float* prev;
  float* part;
  int32_t rows, h;
  float eps;
  int32_t first;
};
hipError_t launch_cache_delta(const CacheDeltaArgs& a, hipStream_t s);
// y[i] = alpha * y[i] + beta * x[i] over n floats (n % 4 == 0, 16-byte aligned);
// alpha == 0 writes beta * x[i] without reading y.
hipError_t launch_axpby(float* y, const float* x, float alpha, float beta, int64_t n, hipStream_t s);

// Device-side cache decision, one block: num = sum part[2r], den = sum
// part[2r + 1] over `rows` rows (float64, fixed order); rel = num / den (inf
// when den == 0 < num, 0 when both are 0); acc = st->acc + rel; the step
// reuses the residual (st->skip = 1) while acc < threshold, else runs the
// blocks (st->skip = 0) and acc restarts at 0. first != 0: a generation's
// first step (runs the blocks, acc = rel = 0).
struct CacheState {
  int32_t skip;        // 1: this step reuses the residual
  int32_t ran_blocks;  // !skip
  int32_t steps;       // steps decided since the generation started
  int32_t pad;
  double acc, rel;
};
hipError_t launch_cache_decide(const float* part, int rows, int first, double threshold, CacheState* st,
                               hipStream_t s);
// n floats (n % 4 == 0, 16-byte aligned): img += resid when *skip, else
// resid = img (the residual base img0 of a step that runs the blocks).
hipError_t launch_cache_apply(float* img, float* resid, int64_t n, const int* skip, hipStream_t s);
// resid = img - resid unless *skip (the image-stream residual of the blocks).
hipError_t launch_cache_store(float* resid, const float* img, int64_t n, const int* skip, hipStream_t s);

// ---- QK RMSNorm + RoPE + attention layout ------------------------------------
// Token t of batch b reads q|k|v from row (b, t) of seg[0] when t < seg_len0,
// else row (b, t - seg_len0) of seg[1] (q at col 0, k at h, v at 2h).
// Writes Q, K [B, H, Lpad, d] and V either [B, H, d, Lpad] (v_trans, bf16
// MFMA path) or [B, H, Lpad, d]; positions t in [L, Lpad) are zero-filled.
struct QkNormArgs {
  RowSeg seg[2];
  int32_t seg_len0;  // tokens in segment 0 per batch
  const void* qn[2];
  const void* kn[2];
  const float* table;  // [L, 64, 2] cos, sin
  void* Q;
  void* K;
  void* V;
  int32_t B, H, L, Lpad;
  float eps;
  float qscale;  // Q is written times qscale (the bf16 attention's score scale)
  const int* skip = nullptr;  // step-cache guard (see guard_skip), null: always run
};
hipError_t launch_qk_norm_rope(const QkNormArgs& a, bool bf16, bool v_trans, hipStream_t s);
// bf16 only, after the fused QKV epilogue: zeroes rows t in [L, Lpad) of Q
// and K and the positions of V^T that hold no token (vkey_pos(p) >= L).
hipError_t launch_qkv_pad_zero(const QkNormArgs& a, hipStream_t s);

// ---- RoPE table -------------------------------------------------------------
hipError_t launch_rope_table(const int32_t* ids, int L, int a0, int a1, int a2, double theta,
                             float* table, hipStream_t s);

// ---- GEMV: y[b, n] (+)= bias[n] + sum_k W[n, k] f(x[b, k]) --------------------
// W dense [N, K] in w_bf16 ? bf16 : float; x [B, K] float32 or activation
// dtype; f = SiLU when silu_in; y [B, N] float32 (accumulate adds to y).
struct GemvArgs {
  const void* W;
  const void* bias;
  const void* x;
  float* y;
  int32_t N, K, B;
  int32_t x_bstride, y_bstride;
  bool silu_in, accumulate;
  const int* skip = nullptr;  // step-cache guard (see guard_skip), null: always run
};
hipError_t launch_gemv(const GemvArgs& a, bool w_bf16, bool x_f32, hipStream_t s);
// Up to kGemvMaxSeg GEMVs sharing one float32 input (SiLU applied), B <= 4
// batch rows, one launch: y_s[b, :] = bias_s + W_s SiLU(x[b, :]).
constexpr int kGemvMaxSeg = 24;
constexpr int kGemvMaxB = 4;  // batch rows per GEMV launch
struct GemvSeg {
  const void* W;
  const void* bias;
  float* y;  // [B, y_bstride]
  int32_t N, y_bstride;
  int32_t block0;  // set by the launcher
};
struct GemvMultiArgs {
  const void* x;  // [B, x_bstride], float32 (bf16 when x_bf16)
  int32_t K, B, x_bstride;
  int32_t nseg;
  bool x_bf16 = false;
  GemvSeg seg[kGemvMaxSeg];
  const int* skip = nullptr;  // step-cache guard (see guard_skip), null: always run
};
hipError_t launch_gemv_multi(const GemvMultiArgs& a, bool w_bf16, hipStream_t s);

// ---- sinusoidal timestep embedding: t[b, i], tau = 1000 * sigma ---------------
hipError_t launch_timestep_embedding(float* out, int B, int dim, double sigma, hipStream_t s);

// ---- latent packing ---------------------------------------------------------
hipError_t launch_pack(const void* src, void* dst, int B, int C, int H, int W, int elem_bytes,
                       bool unpack, hipStream_t s);

// ---- elementwise cast/copy: dst[i] = src[i] (float <-> activation type) --------
hipError_t launch_convert(const void* src, bool src_f32, void* dst, bool dst_f32, int64_t n,
                          hipStream_t s);

// ---- GEMM: C = A W^T with a fused epilogue ---------------------------------------
enum Epi : int {
  EPI_STORE = 0,     // out = acc + bias                      (activation type or f32)
  EPI_GELU = 1,      // out = GELU(acc + bias)
  EPI_GATE_RES = 2,  // res_out = res_in + gate[b, n] * (acc + bias)
  EPI_SPLIT = 3,     // n < split_n: out = acc + bias; else out2[n - split_n] = GELU(acc + bias)
  EPI_EULER = 4,     // x[r, n] += dsigma * (acc + bias); v_out (if set) = acc + bias  (f32)
  // as EPI_STORE / EPI_SPLIT, except that columns [0, 2 qk_h) (q | k) go
  // through QK RMSNorm + RoPE into Q / K [B, H, Lpad, 128] and columns
  // [2 qk_h, 3 qk_h) (v) into V^T [B, H, 128, Lpad] in vkey_pos order,
  // instead of `out` (256x256 direct-to-LDS kernel, dense bf16 weights only)
  EPI_QKV = 5,
  EPI_SPLIT_QKV = 6,
  // internal to split-K: the float32 sums over one k-range go to part
  // [ksplit, M, N]; a second kernel applies the real epilogue
  EPI_PARTIAL = 7,
};

struct GemmProblem {
  const void* A;  // [M, K] activation type, row stride lda
  int64_t lda;
  const void* W;  // weights per fmt
  const void* scales;
  const void* bias;
  int32_t fmt;  // 0 dense, 1 q4g64, 2 q8g64
  int32_t M, N, K;
  // outputs
  void* out;  // EPI_STORE/GELU/SPLIT: rows contiguous, stride ldo
  int64_t ldo;
  bool out_f32;
  void* out2;  // EPI_SPLIT: GELU part
  int64_t ldo2;
  int32_t split_n;
  RowSeg res_in, res_out;  // EPI_GATE_RES / EPI_EULER (res_out = x); single segment
  bool res_f32;
  const float* gate;  // [B, gate_bstride] at column offset already applied
  int32_t gate_bstride;
  float dsigma;
  float* v_out;  // EPI_EULER, contiguous [M, N], may be null
  // EPI_QKV / EPI_SPLIT_QKV: row m is token qk_tok0 + m % qk_rows of batch
  // m / qk_rows in the joint sequence; head hh of q (k) is columns
  // hh * 128 .. + 127 (qk_h + ...): RMS over those columns (after the bias),
  // times qn (kn), rotated by rope[token] pairs, written as bf16 to
  // Q (K) [B, H, qk_Lpad, 128].
  void* qk_Q;
  void* qk_K;
  void* qk_V;  // V^T
  const void* qn;
  const void* kn;
  const float* rope;  // [L, 64, 2] cos, sin
  int32_t qk_h, qk_rows, qk_tok0, qk_Lpad;
  float qk_eps;
  float qk_qscale;  // Q is written times qk_qscale
  // split-K partial sums [ksplit, M, N] float32 (set by the split-K launcher)
  float* part = nullptr;
  // step-cache guard of the launch (read from the first problem), null: run
  const int* skip = nullptr;
};

// Up to two problems with the same epilogue in one launch (text and image
// streams of a dual block). bf16 operands, MFMA.
hipError_t launch_gemm_bf16(const GemmProblem* p, int nprob, int epi, hipStream_t s);
// Dense bf16 with direct-to-LDS staging, 256x256 tiles (large problems).
bool gemm_dma_eligible(const GemmProblem* p, int nprob, int epi);
hipError_t launch_gemm_dma(const GemmProblem* p, int nprob, int epi, hipStream_t s);
// Split-K on the direct-to-LDS kernel for gated-residual launches with too
// few 256x256 tiles to fill the chip: each tile's k-tiles are cut into
// `ways` ranges, one workgroup per (range, tile) writes float32 partial sums,
// and a second kernel adds them in range order and applies the epilogue.
// gemm_splitk_ways: the number of ranges for this launch (1: no split);
// splitk_ways: the same rule from the launch's tile count and k depth.
int splitk_ways(int64_t tiles, int K);
int64_t gemm_dma_tiles(int M, int N);
int gemm_splitk_ways(const GemmProblem* p, int nprob, int epi);
// part: float32 scratch of ways * sum(M N) values, 16-byte aligned
hipError_t launch_gemm_dma_splitk(const GemmProblem* p, int nprob, int epi, int ways, float* part, hipStream_t s);
// float32 operands and accumulation (VALU), dense weights only.
hipError_t launch_gemm_f32(const GemmProblem* p, int nprob, int epi, hipStream_t s);
// Quantised weights (fmt 1-4, layouts as the GEMM kernels read them) decoded
// into dense bf16 [N, K] at `out` (16-byte aligned): the same bf16 values the
// GEMM kernels stage when they dequantise a tile.
hipError_t launch_dequant(const void* w, const void* scales, int fmt, int N, int K, void* out, hipStream_t s,
                          const int* skip = nullptr);

// y [M, N] (float32 when y_f32, else bf16) = x [M, K] (bf16, row stride K)
// W^T + bias for M <= 16 rows, weights in format fmt (0 dense bf16, 1-4
// quantised, layouts as the GEMMs read them), decoded in registers;
// K % 128 == 0; x, W 16-byte aligned.
hipError_t launch_linear_skinny(const void* x, int M, const void* W, const void* scales, const void* bias, int fmt,
                                void* y, bool y_f32, int N, int K, hipStream_t s);

// ---- joint attention ------------------------------------------------------------
// O rows: token t of batch b goes to seg[0] row (b, t) if t < seg_len0 else
// seg[1] row (b, t - seg_len0), at column offset head * d.
// Token order inside V^T rows (bf16 path): within each aligned group of 16
// tokens, position p holds token vkey_pos(p) (bits 2 and 3 of the index
// swapped; the map is its own inverse), so that the 8 keys one lane feeds to
// the P.V MFMA (keys 4g..4g+3 and 8+4g..8+4g+3 of a 16-key step) are
// contiguous.
__host__ __device__ inline int vkey_pos(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

struct AttnArgs {
  const void* Q;  // [B, H, Lpad, 128]
  const void* K;  // [B, H, Lpad, 128]
  const void* V;  // bf16: V^T [B, H, 128, Lpad] in vkey_pos token order; f32: [B, H, Lpad, 128]
  RowSeg out[2];
  int32_t seg_len0;
  int32_t B, H, L, Lpad;
  float scale;  // 1/sqrt(d) (float32 path; the bf16 path takes Q already
                // multiplied by scale * log2(e), see kAttnQScale)
  // bf16 path: scratch for the partial results of split units (at least
  // kAttnPartBytes, 16-byte aligned), or null to run every unit whole.
  // full_units and workers are set by the launcher.
  float* part;
  int32_t full_units, workers;
  const int* skip = nullptr;  // step-cache guard (see guard_skip), null: always run
};
// bf16 attention blocks: kAttnWaves wavefronts of 32 queries each, one
// block per CU. A unit is 32 * kAttnWaves queries of one (batch, head)
// against all keys. When the unit count leaves the last round of blocks
// short of a full round of kAttnTailWorkers (the CU count), the units of
// that round are cut along the keys: kAttnTailWorkers worker blocks each
// take an equal contiguous share of those units' 64-key tiles (at most two
// pieces of two units), write unnormalised partial results, and a merge
// kernel combines the pieces of each unit.
constexpr int kAttnWaves = 8;
constexpr int kAttnTailWorkers = 256;
// The bf16 attention reads Q multiplied by 1/sqrt(128) * log2(e), applied
// where Q is written (the QK RMSNorm + RoPE epilogue or kernel), so that the
// score MFMA yields exp2 arguments directly.
constexpr float kAttnQScale = 0.08838834764831845f * 1.4426950408889634f;
// one record per piece: O [256][128] float32, then m [256], l [256]
constexpr size_t kAttnRecFloats = (size_t)32 * kAttnWaves * 130;
constexpr size_t kAttnPartBytes = 2 * (size_t)kAttnTailWorkers * kAttnRecFloats * 4;
hipError_t launch_attention_bf16(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_f32(const AttnArgs& a, hipStream_t s);

}  // namespace mmdit
