// C ABI of the MMDiT denoising step: argument validation, workspace layout
// and the order of kernel launches for the dual-stream block, the
// single-stream block and the whole step. All arithmetic runs in the HIP
// kernels (k_*.hip); this file only checks, carves buffers and enqueues.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mmdit.h"
#include "api_internal.h"
#include "kernels.h"

using namespace mmdit;

namespace {
thread_local std::string g_err;
}  // namespace

int mmdit::fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

namespace {

#define HIP_TRY(expr)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(MMDIT_ERR_HIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

size_t align_up(size_t x) { return (x + 255) & ~(size_t)255; }

// ------------------------------------------------------------------ profiling --
// Kernel timing (mmdit_profile_begin/end). Every access to the state holds
// the mutex; `gen` tells a scope whose profiling session has since ended not
// to record its stop event (its launch is then not counted).
struct Prof {
  std::mutex mu;
  bool active = false;
  int cls = 0;
  int cap = 0;
  int used = 0;
  uint64_t gen = 0;
  double work = 0;
  std::vector<hipEvent_t> ev;
};
Prof g_prof;

enum { PC_GEMM = 1, PC_ATTN = 2, PC_LN = 3, PC_QKNORM = 4, PC_GEMV = 5, PC_GEMM_LIN1 = 6, PC_GEMM_RES = 7, PC_DEQUANT = 8,
       PC_GEMM_QKV = 9, PC_GEMM_FC1 = 10, PC_STREAM = 11 };

struct ProfScope {
  hipEvent_t stop = nullptr;
  hipStream_t s;
  uint64_t gen = 0;
  // records when the active class is `cls` or `cls2`
  ProfScope(int cls, double work, hipStream_t st, int cls2 = -1) : s(st) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (!g_prof.active || (g_prof.cls != cls && g_prof.cls != cls2) || g_prof.used >= g_prof.cap) return;
    hipEvent_t start = g_prof.ev[2 * g_prof.used];
    stop = g_prof.ev[2 * g_prof.used + 1];
    gen = g_prof.gen;
    g_prof.used++;
    g_prof.work += work;
    (void)hipEventRecord(start, s);
  }
  ~ProfScope() {
    if (!stop) return;
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (g_prof.active && g_prof.gen == gen) (void)hipEventRecord(stop, s);
  }
};

// ------------------------------------------------------------------ checks --
struct Geo {
  int B, h, H, m, Lt, Li, L, Lpad;
  bool bf16;
  int esz;
  int resid;  // mmdit_dims.resid (MMDIT_RESID_*)
};

int check_dims(const mmdit_dims* d, Geo& g) {
  if (!d) return fail(MMDIT_ERR_NULL, "dims is NULL");
  if (d->act_dtype != MMDIT_F32 && d->act_dtype != MMDIT_BF16)
    return fail(MMDIT_ERR_DTYPE, "act_dtype %d is not MMDIT_F32 or MMDIT_BF16", d->act_dtype);
  if (d->head_dim != 128) return fail(MMDIT_ERR_UNSUPPORTED, "head_dim %d: only 128 is implemented", d->head_dim);
  if (d->batch < 1 || d->heads < 1) return fail(MMDIT_ERR_SHAPE, "batch and heads must be >= 1");
  if ((int64_t)d->heads * 128 != d->hidden) return fail(MMDIT_ERR_SHAPE, "hidden %d != heads*head_dim", d->hidden);
  if (d->hidden % 256 != 0 || d->hidden > 4096)
    return fail(MMDIT_ERR_SHAPE, "hidden %d must be a multiple of 256 and at most 4096", d->hidden);
  if (d->mlp_hidden < 64 || d->mlp_hidden % 64 != 0) return fail(MMDIT_ERR_SHAPE, "mlp_hidden %d must be a positive multiple of 64", d->mlp_hidden);
  if (d->txt_len < 0 || d->img_len < 1) return fail(MMDIT_ERR_SHAPE, "need txt_len >= 0 and img_len >= 1");
  int sum = 0;
  for (int a = 0; a < 3; ++a) {
    if (d->axes_dim[a] < 0 || d->axes_dim[a] % 2) return fail(MMDIT_ERR_SHAPE, "axes_dim[%d] must be even and >= 0", a);
    sum += d->axes_dim[a];
  }
  if (sum != d->head_dim) return fail(MMDIT_ERR_SHAPE, "axes_dim sum %d != head_dim", sum);
  if (!(d->theta > 0) || !(d->ln_eps > 0) || !(d->rms_eps > 0)) return fail(MMDIT_ERR_SHAPE, "theta and eps must be > 0");
  if (d->resid != MMDIT_RESID_DEFAULT && d->resid != MMDIT_RESID_F32 && d->resid != MMDIT_RESID_BF16)
    return fail(MMDIT_ERR_DTYPE, "resid %d is not one of MMDIT_RESID_DEFAULT, _F32, _BF16", d->resid);
  if (d->resid == MMDIT_RESID_BF16 && d->act_dtype != MMDIT_BF16)
    return fail(MMDIT_ERR_DTYPE, "a bf16 residual stream needs bf16 activations");
  g.B = d->batch; g.h = d->hidden; g.H = d->heads; g.m = d->mlp_hidden;
  g.Lt = d->txt_len; g.Li = d->img_len; g.L = g.Lt + g.Li;
  g.Lpad = (g.L + 127) / 128 * 128;
  g.bf16 = d->act_dtype == MMDIT_BF16;
  g.esz = g.bf16 ? 2 : 4;
  g.resid = d->resid;
  const int64_t widest = 3 * (int64_t)g.h + g.m;
  if ((int64_t)g.B * g.Lpad * widest >= (int64_t(1) << 31) || (int64_t)g.B * g.H * g.Lpad * 128 >= (int64_t(1) << 31))
    return fail(MMDIT_ERR_SHAPE, "batch * tokens too large for 32-bit row indexing");
  return MMDIT_OK;
}

// GEMM linear: dense (any K for f32; K % 64 for bf16) or quantised (bf16 only).
int check_linear(const mmdit_linear& l, int n, int k, const Geo& g, const char* name) {
  if (!l.w) return fail(MMDIT_ERR_NULL, "%s.w is NULL", name);
  if (l.n_out != n || l.k_in != k) return fail(MMDIT_ERR_SHAPE, "%s is [%d, %d], expected [%d, %d]", name, l.n_out, l.k_in, n, k);
  if (l.fmt == MMDIT_W_DENSE) {
    if (g.bf16 && k % 64) return fail(MMDIT_ERR_SHAPE, "%s: k_in %d must be a multiple of 64 for bf16", name, k);
    return MMDIT_OK;
  }
  const bool sub = l.fmt == MMDIT_W_Q1G128 || l.fmt == MMDIT_W_TQ2G128;
  if (l.fmt != MMDIT_W_Q4G64 && l.fmt != MMDIT_W_Q8G64 && !sub)
    return fail(MMDIT_ERR_DTYPE, "%s: unknown weight format %d", name, l.fmt);
  if (!g.bf16) return fail(MMDIT_ERR_DTYPE, "%s: quantised weights need bf16 activations", name);
  if (k % (sub ? 128 : 64)) return fail(MMDIT_ERR_SHAPE, "%s: quantised k_in %d must be a multiple of %d", name, k, sub ? 128 : 64);
  if (!l.scales) return fail(MMDIT_ERR_NULL, "%s.scales is NULL", name);
  return MMDIT_OK;
}

// GEMV linear (modulation, conditioning MLPs): dense, K % 8, K <= 4096.
int check_gemv(const mmdit_linear& l, int n, int k, const char* name) {
  if (!l.w) return fail(MMDIT_ERR_NULL, "%s.w is NULL", name);
  if (l.n_out != n || l.k_in != k) return fail(MMDIT_ERR_SHAPE, "%s is [%d, %d], expected [%d, %d]", name, l.n_out, l.k_in, n, k);
  if (l.fmt != MMDIT_W_DENSE) return fail(MMDIT_ERR_DTYPE, "%s must be dense", name);
  if (k % 8 || k > 4096) return fail(MMDIT_ERR_SHAPE, "%s: k_in %d must be a multiple of 8 and <= 4096", name, k);
  return MMDIT_OK;
}

int check_stream(const mmdit_stream_w& s, const Geo& g, const char* name) {
  char nm[64];
  int r;
  snprintf(nm, sizeof nm, "%s.mod", name);
  if ((r = check_gemv(s.mod, 6 * g.h, g.h, nm))) return r;
  snprintf(nm, sizeof nm, "%s.qkv", name);
  if ((r = check_linear(s.qkv, 3 * g.h, g.h, g, nm))) return r;
  snprintf(nm, sizeof nm, "%s.proj", name);
  if ((r = check_linear(s.proj, g.h, g.h, g, nm))) return r;
  snprintf(nm, sizeof nm, "%s.fc1", name);
  if ((r = check_linear(s.fc1, g.m, g.h, g, nm))) return r;
  snprintf(nm, sizeof nm, "%s.fc2", name);
  if ((r = check_linear(s.fc2, g.h, g.m, g, nm))) return r;
  if (!s.q_norm || !s.k_norm) return fail(MMDIT_ERR_NULL, "%s q_norm/k_norm is NULL", name);
  return MMDIT_OK;
}

int check_single(const mmdit_single_w& s, const Geo& g) {
  int r;
  if ((r = check_gemv(s.mod, 3 * g.h, g.h, "single.mod"))) return r;
  if ((r = check_linear(s.lin1, 3 * g.h + g.m, g.h, g, "single.lin1"))) return r;
  if ((r = check_linear(s.lin2, g.h, g.h + g.m, g, "single.lin2"))) return r;
  if (!s.q_norm || !s.k_norm) return fail(MMDIT_ERR_NULL, "single q_norm/k_norm is NULL");
  return MMDIT_OK;
}

// ---------------------------------------------------------------- workspace --
// Block scratch (activation dtype unless noted):
//   xn [rows, h], qkv [rows, 3h], Q/K/V [B, H, Lpad, 128],
//   o   [rows, h] (dual) or cat [rows, h + m] (single), mlp [rows, m] (dual).
//   attn  partial results of key-split attention units (bf16 path).
//   xw  bf16 weights decoded from a quantised layer (only when expanding).
// Laid out as o, xn, qkv, Q, K, V, mlp, attn, xw, so that the float32
// partial sums of a split-K gated-residual GEMM fit in scratch that is dead
// during it: [xn, mlp end) when the GEMM reads o (out-projection, linear2),
// [o, V end) when it reads mlp (fc2).
struct BlockWs {
  size_t o, xn, qkv, q, k, v, mlp, attn, xw, xw_bytes, total;
};

// Quantised layers of launches with at least this many rows are decoded into
// bf16 scratch once and run on the dense kernels. Dequantising inside the GEMM
// decodes each weight tile once per output row-tile (rows / 256 times); from
// four row-tiles on, that repeated VALU work (which the MFMAs of the same SIMD
// do not hide) costs more than one HBM-bound decoding pass.
constexpr int64_t kExpandMinRows = 1024;

// Bytes of the decoded-weight scratch for geometry g when the largest
// quantised launch holds nk weights (0 when the launches do not expand).
size_t expand_bytes(const Geo& g, size_t nk) {
  return g.bf16 && (int64_t)g.B * g.L >= kExpandMinRows ? align_up(nk * 2) : 0;
}

// Largest weight count of one block GEMM launch: both streams' qkv or fc1 /
// fc2 (dual), or linear1 (single).
size_t block_launch_weights(const Geo& g) {
  const size_t h = g.h, m = g.m;
  const size_t dual = 2 * h * (3 * h > m ? 3 * h : m);
  const size_t single = h * (3 * h + m);
  return dual > single ? dual : single;
}

BlockWs plan_block(const Geo& g, size_t base, size_t xw_bytes) {
  BlockWs w;
  const size_t rows = (size_t)g.B * g.L;
  const size_t qkvh = (size_t)g.B * g.H * g.Lpad * 128;
  size_t at = base;
  w.o = at; at = align_up(at + rows * (size_t)(g.h + g.m) * g.esz);
  w.xn = at; at = align_up(at + rows * g.h * g.esz);
  w.qkv = at; at = align_up(at + rows * 3 * g.h * g.esz);
  w.q = at; at = align_up(at + qkvh * g.esz);
  w.k = at; at = align_up(at + qkvh * g.esz);
  w.v = at; at = align_up(at + qkvh * g.esz);
  w.mlp = at; at = align_up(at + rows * g.m * g.esz);
  w.attn = at; at = align_up(at + (g.bf16 ? kAttnPartBytes : 0));
  w.xw = at; w.xw_bytes = xw_bytes; at = align_up(at + xw_bytes);
  w.total = at;
  return w;
}

// Block-call workspace: RoPE table [L, 64, 2] f32, modulation f32, scratch.
struct BlockCallWs {
  size_t table, mod;
  BlockWs blk;
};

// xw: room for decoded weights (needed only when a quantised layer is
// decoded, see kExpandMinRows; the queries without weights assume it is).
BlockCallWs plan_block_call(const Geo& g, int mod_width, bool xw = true) {
  BlockCallWs w;
  size_t at = 0;
  w.table = at; at = align_up(at + (size_t)g.L * 64 * 2 * 4);
  w.mod = at; at = align_up(at + (size_t)g.B * mod_width * 4);
  w.blk = plan_block(g, at, xw ? expand_bytes(g, block_launch_weights(g)) : 0);
  return w;
}

// Step workspace.
struct StepWs {
  size_t x, vec, temb, hid, mods, table, xin;
  BlockWs blk;
  size_t mod_dual, mod_single, mod_final;  // offsets inside mods (floats)
};

// Where the modulation vectors of a step sit. Each modulation matrix (dual
// block i stream s, single block i, the final layer) holds its rows for n
// timesteps of B batch rows each, [n B, width], timestep j first; a step
// reads the rows of timestep j. Inside the step workspace n = 1, j = 0;
// mmdit_step_modulations fills n timesteps at once.
struct ModLay {
  float* base;
  size_t B, h, nd, ns, n, j;
  float* dual(int i, int s) const { return base + (((size_t)i * 2 + s) * n + j) * B * 6 * h; }
  float* single(int i) const { return base + nd * 2 * n * B * 6 * h + ((size_t)i * n + j) * B * 3 * h; }
  float* fin() const { return base + nd * 2 * n * B * 6 * h + ns * n * B * 3 * h + j * B * 2 * h; }
  static size_t floats(size_t B, size_t h, size_t nd, size_t ns, size_t n) {
    return n * B * h * (nd * 12 + ns * 3 + 2);
  }
};

// Residual bytes per element inside mmdit_step.
int step_resid_esz(const Geo& g) { return g.resid == MMDIT_RESID_BF16 ? 2 : 4; }

StepWs plan_step(const mmdit_config* c, const Geo& g, bool xw = true) {
  StepWs w;
  size_t at = 0;
  const size_t B = g.B;
  w.x = at; at = align_up(at + B * g.L * g.h * step_resid_esz(g));
  w.vec = at; at = align_up(at + B * g.h * 4);
  w.temb = at; at = align_up(at + B * c->temb_dim * 4);
  w.hid = at; at = align_up(at + B * g.h * 4);
  w.mod_dual = 0;
  w.mod_single = (size_t)c->n_double * 2 * B * 6 * g.h;
  w.mod_final = w.mod_single + (size_t)c->n_single * B * 3 * g.h;
  w.mods = at; at = align_up(at + (w.mod_final + B * 2 * g.h) * 4);
  w.table = at; at = align_up(at + (size_t)g.L * 64 * 2 * 4);
  w.xin = at; at = align_up(at + B * g.Li * c->in_ch * g.esz);
  // the input and final projections may be quantised too
  size_t nk = block_launch_weights(g);
  const size_t nk_io = (size_t)g.h * (c->txt_in_dim > c->in_ch ? c->txt_in_dim : c->in_ch);
  nk = nk > nk_io ? nk : nk_io;
  w.blk = plan_block(g, at, xw ? expand_bytes(g, nk) : 0);
  return w;
}

bool is_quantised(const mmdit_linear& l) { return l.fmt != MMDIT_W_DENSE; }
bool stream_quantised(const mmdit_stream_w& s) {
  return is_quantised(s.qkv) || is_quantised(s.proj) || is_quantised(s.fc1) || is_quantised(s.fc2);
}
bool single_quantised(const mmdit_single_w& s) { return is_quantised(s.lin1) || is_quantised(s.lin2); }

// Whether a step with these weights decodes a quantised layer into the
// workspace (automatic route, at least kExpandMinRows rows).
bool step_decodes(const mmdit_config* c, const mmdit_model_w* w, const mmdit_step_opts* o, const Geo& g) {
  if (!g.bf16 || (o && o->dequant == 1) || (int64_t)g.B * g.L < kExpandMinRows) return false;
  bool q = is_quantised(w->img_in) || is_quantised(w->txt_in) || is_quantised(w->final_lin);
  for (int i = 0; i < c->n_double && !q; ++i) q = stream_quantised(w->dbl[i].txt) || stream_quantised(w->dbl[i].img);
  for (int i = 0; i < c->n_single && !q; ++i) q = single_quantised(w->sgl[i]);
  return q;
}

// --------------------------------------------------------------- launches --
struct Ctx {
  hipStream_t s;
  Geo g;
  float ln_eps, rms_eps;
  void* xw = nullptr;  // decoded-weight scratch (null: quantised layers stay fused)
  size_t xw_bytes = 0;
  // dead scratch for split-K partial sums of the next gated-residual launch
  // (null: it runs whole)
  float* part = nullptr;
  size_t part_bytes = 0;
  // step-cache guard passed to every launch (null: unguarded): the launches
  // do nothing when the device-side cache decision reuses the residual
  const int* skip = nullptr;
};

char* ptr(void* base, size_t off) { return reinterpret_cast<char*>(base) + off; }

// Decodes the quantised weights of a launch into the scratch (when the
// geometry expands, see kExpandMinRows) and points the problems at the dense
// copies. Problems sharing one weight matrix share one copy. Later launches on
// the stream reuse the scratch, after this launch's reads.
int expand_quantised(const Ctx& c, GemmProblem* p, int np) {
  if (!c.xw) return MMDIT_OK;
  const void* src[2] = {nullptr, nullptr};
  void* dst[2] = {nullptr, nullptr};
  size_t at = 0;
  for (int i = 0; i < np; ++i) {
    if (p[i].fmt == MMDIT_W_DENSE) continue;
    void* d = nullptr;
    for (int j = 0; j < i; ++j)
      if (src[j] == p[i].W) d = dst[j];
    if (!d) {
      const size_t bytes = (size_t)p[i].N * p[i].K * 2;
      if (at + bytes > c.xw_bytes)
        return fail(MMDIT_ERR_WORKSPACE, "decoded-weight scratch %zu bytes, need %zu", c.xw_bytes, at + bytes);
      d = ptr(c.xw, at);
      at = align_up(at + bytes);
      const double wb = p[i].fmt == MMDIT_W_Q4G64 ? 0.5 : p[i].fmt == MMDIT_W_Q8G64 ? 1.0
                        : p[i].fmt == MMDIT_W_Q1G128 ? 0.125 : 0.25;
      ProfScope ps(PC_DEQUANT, (double)p[i].N * p[i].K * (wb + 2.0), c.s);
      HIP_TRY(launch_dequant(p[i].W, p[i].scales, p[i].fmt, p[i].N, p[i].K, d, c.s, c.skip));
    }
    src[i] = p[i].W;
    dst[i] = d;
    p[i].W = d;
    p[i].fmt = MMDIT_W_DENSE;
    p[i].scales = nullptr;
  }
  return MMDIT_OK;
}

int gemm(const Ctx& c, GemmProblem* p, int np, int epi) {
  for (int i = 0; i < np; ++i) p[i].skip = c.skip;
  if (int r = expand_quantised(c, p, np)) return r;
  double flops = 0;
  for (int i = 0; i < np; ++i) flops += 2.0 * p[i].M * (double)p[i].N * p[i].K;
  ProfScope ps(PC_GEMM, flops, c.s,
               epi == EPI_SPLIT || epi == EPI_SPLIT_QKV ? PC_GEMM_LIN1
               : epi == EPI_GATE_RES                   ? PC_GEMM_RES
               : epi == EPI_QKV                        ? PC_GEMM_QKV
               : epi == EPI_GELU                       ? PC_GEMM_FC1
                                                       : -1);
  if (!c.g.bf16) {
    HIP_TRY(launch_gemm_f32(p, np, epi, c.s));
    return MMDIT_OK;
  }
  if (gemm_dma_eligible(p, np, epi)) {
    HIP_TRY(launch_gemm_dma(p, np, epi, c.s));
    return MMDIT_OK;
  }
  int ways = c.part && (uintptr_t)c.part % 16 == 0 ? gemm_splitk_ways(p, np, epi) : 1;
  size_t mn = 0;
  for (int i = 0; i < np; ++i) mn += (size_t)p[i].M * p[i].N;
  while (ways > 1 && (size_t)ways * mn * 4 > c.part_bytes) --ways;
  if (ways > 1) HIP_TRY(launch_gemm_dma_splitk(p, np, epi, ways, c.part, c.s));
  else HIP_TRY(launch_gemm_bf16(p, np, epi, c.s));
  return MMDIT_OK;
}

int gemv(const Ctx& c, const mmdit_linear& l, const void* x, bool x_f32, int x_bstride, float* y,
         int y_bstride, bool silu, bool accumulate) {
  GemvArgs a;
  a.W = l.w; a.bias = l.bias; a.x = x; a.y = y;
  a.N = l.n_out; a.K = l.k_in; a.B = c.g.B;
  a.x_bstride = x_bstride; a.y_bstride = y_bstride;
  a.silu_in = silu; a.accumulate = accumulate;
  a.skip = c.skip;
  ProfScope ps(PC_GEMV, (double)l.n_out * l.k_in * c.g.esz, c.s);
  HIP_TRY(launch_gemv(a, c.g.bf16, x_f32 || !c.g.bf16, c.s));
  return MMDIT_OK;
}

// The modulation GEMVs of one block call, SiLU(vec) times each matrix: one
// launch over all matrices when the batch fits one pass of the multi-GEMV.
int mod_gemvs(const Ctx& c, const mmdit_linear* const* l, float* const* y, int n, const void* vec) {
  const Geo& g = c.g;
  if (g.B > kGemvMaxB) {
    for (int i = 0; i < n; ++i)
      if (int r = gemv(c, *l[i], vec, false, g.h, y[i], l[i]->n_out, true, false)) return r;
    return MMDIT_OK;
  }
  GemvMultiArgs ga{};
  ga.x = vec; ga.K = g.h; ga.B = g.B; ga.x_bstride = g.h; ga.x_bf16 = g.bf16;
  ga.skip = c.skip;
  double bytes = 0;
  for (int i = 0; i < n; ++i) {
    GemvSeg& sg = ga.seg[ga.nseg++];
    sg.W = l[i]->w; sg.bias = l[i]->bias; sg.y = y[i]; sg.N = l[i]->n_out; sg.y_bstride = l[i]->n_out;
    bytes += (double)l[i]->n_out * l[i]->k_in * g.esz;
  }
  ProfScope ps(PC_GEMV, bytes, c.s);
  HIP_TRY(launch_gemv_multi(ga, g.bf16, c.s));
  return MMDIT_OK;
}

// A block operates on up to two parts: the text rows and the image rows.
// Part p has len tokens per batch; its rows in the contiguous scratch buffers
// start at row0 (row = row0 + b * len + t_local); its residual rows are x_in /
// x_out (activation dtype, or f32 when res_f32).
struct Part {
  int len;
  int64_t row0;
  RowSeg x_in, x_out;
  const float* mod;
};

RowSeg rows_of(void* buf, int64_t row0, int len, int ld, int esz) {
  RowSeg r;
  r.base = ptr(buf, (size_t)row0 * ld * esz);
  r.batch_stride = (int64_t)len * ld;
  r.rows_per_batch = len > 0 ? len : 1;
  r.ld = ld;
  return r;
}

int run_ln(const Ctx& c, const Part* parts, int np, int mod_bstride, int shift_off, int scale_off,
           bool res_f32, void* y) {
  const Geo& g = c.g;
  LnArgs a{};
  int rows = 0;
  for (int p = 0; p < 2; ++p) {
    if (p < np) {
      a.seg[p] = parts[p].x_in;
      a.seg_rows[p] = g.B * parts[p].len;
      a.mod[p] = parts[p].mod;
    } else {
      a.seg[p] = parts[0].x_in;
      a.seg_rows[p] = 0;
      a.mod[p] = parts[0].mod;
    }
    rows += a.seg_rows[p];
  }
  a.mod_bstride = mod_bstride; a.shift_off = shift_off; a.scale_off = scale_off;
  a.y = y; a.h = g.h; a.eps = c.ln_eps;
  a.skip = c.skip;
  if (rows == 0) return MMDIT_OK;
  ProfScope ps(PC_LN, (double)rows * g.h * ((res_f32 ? 4 : g.esz) + g.esz), c.s);
  HIP_TRY(launch_adaln_ln(a, rows, res_f32 || !g.bf16, g.bf16, c.s));
  return MMDIT_OK;
}

// Points the q | k | v columns of a QKV projection at the fused epilogues
// (RMSNorm + RoPE into Q and K, V transposed into V^T; part p's rows start
// at joint token tok0) and reports whether the direct-to-LDS kernel takes
// the launch; otherwise the separate QK-norm kernel runs after a plain store.
bool fuse_qk(const Ctx& c, GemmProblem* gp, int np, const Part* parts, const void* const qn[2],
             const void* const kn[2], const float* table, const BlockWs& w, void* ws, int epi) {
  const Geo& g = c.g;
  if (!g.bf16) return false;
  int tok0 = 0;
  for (int p = 0; p < np; ++p) {
    gp[p].qk_Q = ptr(ws, w.q); gp[p].qk_K = ptr(ws, w.k); gp[p].qk_V = ptr(ws, w.v);
    gp[p].qn = qn[p]; gp[p].kn = kn[p];
    gp[p].rope = table;
    gp[p].qk_h = g.h; gp[p].qk_rows = parts[p].len; gp[p].qk_tok0 = tok0; gp[p].qk_Lpad = g.Lpad;
    gp[p].qk_eps = c.rms_eps;
    gp[p].qk_qscale = kAttnQScale;
    tok0 += parts[p].len;
  }
  return gemm_dma_eligible(gp, np, epi);
}

int run_qk_attn(const Ctx& c, const Part* parts, int np, void* qkv, const void* const qn[2],
                const void* const kn[2], const float* table, const BlockWs& w, void* ws, void* obuf, int o_ld,
                bool qk_fused) {
  const Geo& g = c.g;
  QkNormArgs q{};
  AttnArgs at{};
  for (int p = 0; p < 2; ++p) {
    const int pp = p < np ? p : 0;
    q.seg[p] = rows_of(qkv, parts[pp].row0, parts[pp].len, 3 * g.h, g.esz);
    q.qn[p] = qn[pp];
    q.kn[p] = kn[pp];
    at.out[p] = rows_of(obuf, parts[pp].row0, parts[pp].len, o_ld, g.esz);
  }
  q.seg_len0 = np == 2 ? parts[0].len : g.L;
  q.table = table;
  q.Q = ptr(ws, w.q); q.K = ptr(ws, w.k); q.V = ptr(ws, w.v);
  q.B = g.B; q.H = g.H; q.L = g.L; q.Lpad = g.Lpad; q.eps = c.rms_eps;
  q.qscale = g.bf16 ? kAttnQScale : 1.0f;
  q.skip = c.skip;
  if (qk_fused) {  // Q, K and V^T are written; only the pad rows remain
    if (g.Lpad > g.L) HIP_TRY(launch_qkv_pad_zero(q, c.s));
  } else {
    ProfScope ps(PC_QKNORM, (double)g.B * g.L * 3 * g.h * g.esz * 2, c.s);
    HIP_TRY(launch_qk_norm_rope(q, g.bf16, g.bf16, c.s));
  }
  at.Q = q.Q; at.K = q.K; at.V = q.V;
  at.part = g.bf16 ? (float*)ptr(ws, w.attn) : nullptr;
  at.seg_len0 = q.seg_len0;
  at.B = g.B; at.H = g.H; at.L = g.L; at.Lpad = g.Lpad;
  at.scale = 1.0f / sqrtf(128.0f);
  at.skip = c.skip;
  {
    ProfScope ps(PC_ATTN, 4.0 * g.B * g.H * (double)g.L * g.L * 128, c.s);
    HIP_TRY(g.bf16 ? launch_attention_bf16(at, c.s) : launch_attention_f32(at, c.s));
  }
  return MMDIT_OK;
}

GemmProblem base_problem(const mmdit_linear& l) {
  GemmProblem p{};
  p.W = l.w; p.scales = l.scales; p.bias = l.bias; p.fmt = l.fmt;
  p.N = l.n_out; p.K = l.k_in;
  return p;
}

// The context of a gated-residual launch whose split-K partial sums may use
// the dead block scratch [from, to) (bf16 path).
Ctx with_part(const Ctx& c, void* ws, size_t from, size_t to) {
  Ctx r = c;
  if (c.g.bf16 && to > from) {
    r.part = (float*)ptr(ws, from);
    r.part_bytes = to - from;
  }
  return r;
}

// Dual-stream block; parts[0] text, parts[1] image; sw[p] the stream weights.
int run_double(const Ctx& c, const mmdit_stream_w* const sw[2], const Part* parts, bool res_f32,
               const float* table, void* ws, const BlockWs& w) {
  const Geo& g = c.g;
  const int h = g.h, m = g.m;
  int r;
  void* xn = ptr(ws, w.xn);
  void* qkv = ptr(ws, w.qkv);
  void* o = ptr(ws, w.o);
  void* mlp = ptr(ws, w.mlp);
  // adaLN LayerNorm 1
  if ((r = run_ln(c, parts, 2, 6 * h, 0, h, res_f32, xn))) return r;
  // QKV projection (both streams, one launch)
  GemmProblem gp[2];
  for (int p = 0; p < 2; ++p) {
    gp[p] = base_problem(sw[p]->qkv);
    gp[p].A = ptr(xn, (size_t)parts[p].row0 * h * g.esz); gp[p].lda = h;
    gp[p].M = g.B * parts[p].len;
    gp[p].out = ptr(qkv, (size_t)parts[p].row0 * 3 * h * g.esz); gp[p].ldo = 3 * h;
  }
  // QK RMSNorm + RoPE (fused into the projection's epilogue when the
  // direct-to-LDS kernel runs it), joint attention
  const void* qn[2] = {sw[0]->q_norm, sw[1]->q_norm};
  const void* kn[2] = {sw[0]->k_norm, sw[1]->k_norm};
  if ((r = expand_quantised(c, gp, 2))) return r;
  const bool fused = fuse_qk(c, gp, 2, parts, qn, kn, table, w, ws, EPI_QKV);
  if ((r = gemm(c, gp, 2, fused ? EPI_QKV : EPI_STORE))) return r;
  if ((r = run_qk_attn(c, parts, 2, qkv, qn, kn, table, w, ws, o, h, fused))) return r;
  // out-projection, x += gate1 * (.)
  for (int p = 0; p < 2; ++p) {
    gp[p] = base_problem(sw[p]->proj);
    gp[p].A = ptr(o, (size_t)parts[p].row0 * h * g.esz); gp[p].lda = h;
    gp[p].M = g.B * parts[p].len;
    gp[p].res_in = parts[p].x_in; gp[p].res_out = parts[p].x_out; gp[p].res_f32 = res_f32;
    gp[p].gate = parts[p].mod + 2 * h; gp[p].gate_bstride = 6 * h;
  }
  if ((r = gemm(with_part(c, ws, w.xn, w.attn), gp, 2, EPI_GATE_RES))) return r;
  // adaLN LayerNorm 2 on the updated residual
  Part p2[2] = {parts[0], parts[1]};
  for (int p = 0; p < 2; ++p) p2[p].x_in = parts[p].x_out;
  if ((r = run_ln(c, p2, 2, 6 * h, 3 * h, 4 * h, res_f32, xn))) return r;
  // fc1 + GELU
  for (int p = 0; p < 2; ++p) {
    gp[p] = base_problem(sw[p]->fc1);
    gp[p].A = ptr(xn, (size_t)parts[p].row0 * h * g.esz); gp[p].lda = h;
    gp[p].M = g.B * parts[p].len;
    gp[p].out = ptr(mlp, (size_t)parts[p].row0 * m * g.esz); gp[p].ldo = m;
  }
  if ((r = gemm(c, gp, 2, EPI_GELU))) return r;
  // fc2, x += gate2 * (.)
  for (int p = 0; p < 2; ++p) {
    gp[p] = base_problem(sw[p]->fc2);
    gp[p].A = ptr(mlp, (size_t)parts[p].row0 * m * g.esz); gp[p].lda = m;
    gp[p].M = g.B * parts[p].len;
    gp[p].res_in = parts[p].x_out; gp[p].res_out = parts[p].x_out; gp[p].res_f32 = res_f32;
    gp[p].gate = parts[p].mod + 5 * h; gp[p].gate_bstride = 6 * h;
  }
  return gemm(with_part(c, ws, w.o, w.mlp), gp, 2, EPI_GATE_RES);
}

// Single-stream block over np parts sharing the weights.
int run_single(const Ctx& c, const mmdit_single_w& sw, const Part* parts, int np, bool res_f32,
               const float* table, void* ws, const BlockWs& w) {
  const Geo& g = c.g;
  const int h = g.h, m = g.m;
  int r;
  void* xn = ptr(ws, w.xn);
  void* qkv = ptr(ws, w.qkv);
  void* cat = ptr(ws, w.o);
  if ((r = run_ln(c, parts, np, 3 * h, 0, h, res_f32, xn))) return r;
  GemmProblem gp[2];
  for (int p = 0; p < np; ++p) {
    gp[p] = base_problem(sw.lin1);
    gp[p].A = ptr(xn, (size_t)parts[p].row0 * h * g.esz); gp[p].lda = h;
    gp[p].M = g.B * parts[p].len;
    gp[p].out = ptr(qkv, (size_t)parts[p].row0 * 3 * h * g.esz); gp[p].ldo = 3 * h;
    gp[p].split_n = 3 * h;
    gp[p].out2 = ptr(cat, ((size_t)parts[p].row0 * (h + m) + h) * g.esz); gp[p].ldo2 = h + m;
  }
  const void* qn[2] = {sw.q_norm, sw.q_norm};
  const void* kn[2] = {sw.k_norm, sw.k_norm};
  if ((r = expand_quantised(c, gp, np))) return r;
  const bool fused = fuse_qk(c, gp, np, parts, qn, kn, table, w, ws, EPI_SPLIT_QKV);
  if ((r = gemm(c, gp, np, fused ? EPI_SPLIT_QKV : EPI_SPLIT))) return r;
  if ((r = run_qk_attn(c, parts, np, qkv, qn, kn, table, w, ws, cat, h + m, fused))) return r;
  for (int p = 0; p < np; ++p) {
    gp[p] = base_problem(sw.lin2);
    gp[p].A = ptr(cat, (size_t)parts[p].row0 * (h + m) * g.esz); gp[p].lda = h + m;
    gp[p].M = g.B * parts[p].len;
    gp[p].res_in = parts[p].x_in; gp[p].res_out = parts[p].x_out; gp[p].res_f32 = res_f32;
    gp[p].gate = parts[p].mod + 2 * h; gp[p].gate_bstride = 3 * h;
  }
  return gemm(with_part(c, ws, w.xn, w.attn), gp, np, EPI_GATE_RES);
}

int rope(const Ctx& c, const mmdit_dims* d, const int32_t* ids, float* table) {
  HIP_TRY(launch_rope_table(ids, c.g.L, d->axes_dim[0], d->axes_dim[1], d->axes_dim[2], d->theta, table, c.s));
  return MMDIT_OK;
}

}  // namespace

// ===================================================================== C ABI ==
extern "C" {

int mmdit_double_block_workspace(const mmdit_dims* dims, size_t* bytes) {
  Geo g;
  int r;
  if (!bytes) return fail(MMDIT_ERR_NULL, "bytes is NULL");
  if ((r = check_dims(dims, g))) return r;
  *bytes = plan_block_call(g, 2 * 6 * g.h).blk.total;
  return MMDIT_OK;
}

int mmdit_single_block_workspace(const mmdit_dims* dims, size_t* bytes) {
  Geo g;
  int r;
  if (!bytes) return fail(MMDIT_ERR_NULL, "bytes is NULL");
  if ((r = check_dims(dims, g))) return r;
  *bytes = plan_block_call(g, 3 * g.h).blk.total;
  return MMDIT_OK;
}

int mmdit_double_block_fwd(const mmdit_dims* dims, const mmdit_double_w* w, const void* img_in,
                           const void* txt_in, void* img_out, void* txt_out, const void* vec,
                           const int32_t* ids, void* ws, size_t ws_bytes, void* hip_stream) {
  Geo g;
  int r;
  if ((r = check_dims(dims, g))) return r;
  if (!w || !img_in || !img_out || !vec || !ids) return fail(MMDIT_ERR_NULL, "NULL weights, image, vec or ids");
  if (g.Lt > 0 && (!txt_in || !txt_out)) return fail(MMDIT_ERR_NULL, "NULL text buffers with txt_len > 0");
  if ((r = check_stream(w->txt, g, "txt"))) return r;
  if ((r = check_stream(w->img, g, "img"))) return r;
  const bool xw = stream_quantised(w->txt) || stream_quantised(w->img);
  const BlockCallWs lay = plan_block_call(g, 2 * 6 * g.h, xw);
  if (!ws || ws_bytes < lay.blk.total)
    return fail(MMDIT_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, lay.blk.total);
  Ctx c{(hipStream_t)hip_stream, g, dims->ln_eps, dims->rms_eps};
  c.xw = lay.blk.xw_bytes ? ptr(ws, lay.blk.xw) : nullptr;
  c.xw_bytes = lay.blk.xw_bytes;
  float* table = (float*)ptr(ws, lay.table);
  float* mod = (float*)ptr(ws, lay.mod);
  float* mod_txt = mod;
  float* mod_img = mod + (size_t)g.B * 6 * g.h;
  if ((r = rope(c, dims, ids, table))) return r;
  {
    const mmdit_linear* ml[2] = {&w->txt.mod, &w->img.mod};
    float* const my[2] = {mod_txt, mod_img};
    if ((r = mod_gemvs(c, ml, my, 2, vec))) return r;
  }
  Part parts[2];
  void* tin = const_cast<void*>(txt_in ? txt_in : img_in);
  void* tout = txt_out ? txt_out : img_out;
  const bool rf = g.resid == MMDIT_RESID_F32;
  const int re = rf ? 4 : g.esz;
  parts[0] = {g.Lt, 0, rows_of(tin, 0, g.Lt, g.h, re), rows_of(tout, 0, g.Lt, g.h, re), mod_txt};
  parts[1] = {g.Li, (int64_t)g.B * g.Lt, rows_of(const_cast<void*>(img_in), 0, g.Li, g.h, re),
              rows_of(img_out, 0, g.Li, g.h, re), mod_img};
  const mmdit_stream_w* sw[2] = {&w->txt, &w->img};
  return run_double(c, sw, parts, rf, table, ws, lay.blk);
}

int mmdit_single_block_fwd(const mmdit_dims* dims, const mmdit_single_w* w, const void* x_in,
                           void* x_out, const void* vec, const int32_t* ids, void* ws,
                           size_t ws_bytes, void* hip_stream) {
  Geo g;
  int r;
  if ((r = check_dims(dims, g))) return r;
  if (!w || !x_in || !x_out || !vec || !ids) return fail(MMDIT_ERR_NULL, "NULL weights, x, vec or ids");
  if ((r = check_single(*w, g))) return r;
  const BlockCallWs lay = plan_block_call(g, 3 * g.h, single_quantised(*w));
  if (!ws || ws_bytes < lay.blk.total)
    return fail(MMDIT_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, lay.blk.total);
  Ctx c{(hipStream_t)hip_stream, g, dims->ln_eps, dims->rms_eps};
  c.xw = lay.blk.xw_bytes ? ptr(ws, lay.blk.xw) : nullptr;
  c.xw_bytes = lay.blk.xw_bytes;
  float* table = (float*)ptr(ws, lay.table);
  float* mod = (float*)ptr(ws, lay.mod);
  if ((r = rope(c, dims, ids, table))) return r;
  {
    const mmdit_linear* ml[1] = {&w->mod};
    float* const my[1] = {mod};
    if ((r = mod_gemvs(c, ml, my, 1, vec))) return r;
  }
  const bool rf = g.resid == MMDIT_RESID_F32;
  const int re = rf ? 4 : g.esz;
  Part part = {g.L, 0, rows_of(const_cast<void*>(x_in), 0, g.L, g.h, re), rows_of(x_out, 0, g.L, g.h, re), mod};
  return run_single(c, *w, &part, 1, rf, table, ws, lay.blk);
}

static int check_config(const mmdit_config* cfg, Geo& g) {
  if (!cfg) return fail(MMDIT_ERR_NULL, "config is NULL");
  int r;
  if ((r = check_dims(&cfg->dims, g))) return r;
  if (cfg->n_double < 0 || cfg->n_single < 0) return fail(MMDIT_ERR_SHAPE, "negative block count");
  if (cfg->in_ch < 64 || cfg->in_ch % 64) return fail(MMDIT_ERR_SHAPE, "in_ch %d must be a positive multiple of 64", cfg->in_ch);
  if (cfg->txt_in_dim < 64 || cfg->txt_in_dim % 64) return fail(MMDIT_ERR_SHAPE, "txt_in_dim must be a positive multiple of 64");
  if (cfg->vec_in_dim < 8 || cfg->vec_in_dim % 8 || cfg->vec_in_dim > 4096) return fail(MMDIT_ERR_SHAPE, "vec_in_dim must be a multiple of 8 in [8, 4096]");
  if (cfg->temb_dim < 8 || cfg->temb_dim % 8 || cfg->temb_dim > 4096) return fail(MMDIT_ERR_SHAPE, "temb_dim must be a multiple of 8 in [8, 4096]");
  return MMDIT_OK;
}

int mmdit_dequantise(const void* w, const void* scales, int32_t fmt, int32_t n_out, int32_t k_in, void* out,
                     void* hip_stream) {
  if (!w || !scales || !out) return fail(MMDIT_ERR_NULL, "NULL weights, scales or output");
  if (fmt != MMDIT_W_Q4G64 && fmt != MMDIT_W_Q8G64 && fmt != MMDIT_W_Q1G128 && fmt != MMDIT_W_TQ2G128)
    return fail(MMDIT_ERR_DTYPE, "fmt %d is not a quantised weight format", fmt);
  const int group = fmt == MMDIT_W_Q1G128 || fmt == MMDIT_W_TQ2G128 ? 128 : 64;
  if (n_out < 0 || k_in < group || k_in % group)
    return fail(MMDIT_ERR_SHAPE, "need n_out >= 0 and k_in a positive multiple of %d (got %d, %d)", group, n_out, k_in);
  const uintptr_t wa = fmt == MMDIT_W_Q1G128 ? 4 : fmt == MMDIT_W_TQ2G128 ? 8 : 16;
  if ((uintptr_t)w % wa || (uintptr_t)scales % 2 || (uintptr_t)out % 16)
    return fail(MMDIT_ERR_SHAPE, "misaligned pointer (w %zu, scales 2, out 16 bytes)", (size_t)wa);
  HIP_TRY(launch_dequant(w, scales, fmt, n_out, k_in, out, (hipStream_t)hip_stream));
  return MMDIT_OK;
}

int mmdit_step_workspace(const mmdit_config* cfg, size_t* bytes) {
  Geo g;
  int r;
  if (!bytes) return fail(MMDIT_ERR_NULL, "bytes is NULL");
  if ((r = check_config(cfg, g))) return r;
  *bytes = plan_step(cfg, g).blk.total;
  return MMDIT_OK;
}

int mmdit_step_workspace_ex(const mmdit_config* cfg, const mmdit_model_w* w, const mmdit_step_opts* opts,
                            size_t* bytes) {
  Geo g;
  int r;
  if (!bytes) return fail(MMDIT_ERR_NULL, "bytes is NULL");
  if ((r = check_config(cfg, g))) return r;
  if (!w) return fail(MMDIT_ERR_NULL, "weights are NULL");
  if ((cfg->n_double > 0 && !w->dbl) || (cfg->n_single > 0 && !w->sgl)) return fail(MMDIT_ERR_NULL, "block weight arrays are NULL");
  *bytes = plan_step(cfg, g, step_decodes(cfg, w, opts, g)).blk.total;
  return MMDIT_OK;
}

// Step-cache buffer: a_prev [B Li h], residual [B Li h] (float32), per-row
// partial sums [B Li 2], the device-side decision state (CacheState).
struct CacheLay {
  size_t prev, resid, part, state, total;
};
static CacheLay plan_cache(const Geo& g) {
  CacheLay c;
  const size_t n = (size_t)g.B * g.Li * g.h;
  c.prev = 0;
  c.resid = align_up(n * 4);
  c.part = align_up(c.resid + n * 4);
  c.state = align_up(c.part + (size_t)g.B * g.Li * 2 * 4);
  c.total = align_up(c.state + sizeof(CacheState));
  return c;
}

int mmdit_step_cache_bytes(const mmdit_config* cfg, size_t* bytes) {
  Geo g;
  int r;
  if (!bytes) return fail(MMDIT_ERR_NULL, "bytes is NULL");
  if ((r = check_config(cfg, g))) return r;
  *bytes = plan_cache(g).total;
  return MMDIT_OK;
}

int mmdit_step_modulations_bytes(const mmdit_config* cfg, int32_t n_sigma, size_t* bytes) {
  Geo g;
  int r;
  if (!bytes) return fail(MMDIT_ERR_NULL, "bytes is NULL");
  if ((r = check_config(cfg, g))) return r;
  if (n_sigma < 1 || (int64_t)n_sigma * g.B > kGemvMaxB)
    return fail(MMDIT_ERR_SHAPE, "n_sigma %d times batch %d must be in [1, %d]", n_sigma, g.B, kGemvMaxB);
  const size_t rows = (size_t)n_sigma * g.B;
  // the modulation matrices, then scratch for the timestep embeddings, the
  // conditioning MLPs' hidden rows, the conditioning vectors and the pooled
  // text vectors repeated per timestep
  *bytes = align_up(ModLay::floats(g.B, g.h, cfg->n_double, cfg->n_single, n_sigma) * 4) +
           align_up(rows * cfg->temb_dim * 4) + 2 * align_up(rows * g.h * 4) +
           align_up(rows * cfg->vec_in_dim * g.esz);
  return MMDIT_OK;
}

int mmdit_step_modulations(const mmdit_config* cfg, const mmdit_model_w* w, const void* y, const double* sigmas,
                           int32_t n_sigma, const mmdit_step_opts* opts, void* mods, size_t mods_bytes,
                           void* hip_stream) {
  Geo g;
  int r;
  size_t need = 0;
  if ((r = mmdit_step_modulations_bytes(cfg, n_sigma, &need))) return r;
  g = Geo{};
  if ((r = check_config(cfg, g))) return r;
  if (!w || !y || !sigmas || !mods) return fail(MMDIT_ERR_NULL, "NULL weights, y, sigmas or mods");
  if ((uintptr_t)mods % 16) return fail(MMDIT_ERR_SHAPE, "mods must be 16-byte aligned");
  if (mods_bytes < need) return fail(MMDIT_ERR_WORKSPACE, "mods buffer %zu bytes, need %zu", mods_bytes, need);
  for (int j = 0; j < n_sigma; ++j)
    if (!std::isfinite(sigmas[j])) return fail(MMDIT_ERR_SHAPE, "sigma values must be finite");
  const mmdit_step_opts none{};
  if (!opts) opts = &none;
  const bool guided = w->guidance_in0.w != nullptr;
  if (guided) {
    if (!opts->has_guidance)
      return fail(MMDIT_ERR_NULL, "the model has a guidance embedder: pass a guidance value");
    if (!std::isfinite(opts->guidance)) return fail(MMDIT_ERR_SHAPE, "guidance must be finite");
  }
  if ((cfg->n_double > 0 && !w->dbl) || (cfg->n_single > 0 && !w->sgl)) return fail(MMDIT_ERR_NULL, "block weight arrays are NULL");
  const int h = g.h, B = g.B;
  if ((r = check_gemv(w->time_in0, h, cfg->temb_dim, "time_in0"))) return r;
  if ((r = check_gemv(w->time_in1, h, h, "time_in1"))) return r;
  if ((r = check_gemv(w->vec_in0, h, cfg->vec_in_dim, "vec_in0"))) return r;
  if ((r = check_gemv(w->vec_in1, h, h, "vec_in1"))) return r;
  if (guided) {
    if ((r = check_gemv(w->guidance_in0, h, cfg->temb_dim, "guidance_in0"))) return r;
    if ((r = check_gemv(w->guidance_in1, h, h, "guidance_in1"))) return r;
  }
  if ((r = check_gemv(w->final_mod, 2 * h, h, "final_mod"))) return r;
  for (int i = 0; i < cfg->n_double; ++i) {
    if ((r = check_gemv(w->dbl[i].txt.mod, 6 * h, h, "dbl.txt.mod"))) return fail(r, "dbl[%d]: %s", i, g_err.c_str());
    if ((r = check_gemv(w->dbl[i].img.mod, 6 * h, h, "dbl.img.mod"))) return fail(r, "dbl[%d]: %s", i, g_err.c_str());
  }
  for (int i = 0; i < cfg->n_single; ++i)
    if ((r = check_gemv(w->sgl[i].mod, 3 * h, h, "sgl.mod"))) return fail(r, "sgl[%d]: %s", i, g_err.c_str());

  // rows j B + b: timestep j, batch row b
  const int rows = n_sigma * B;
  Geo gr = g;
  gr.B = rows;
  Ctx c{(hipStream_t)hip_stream, gr, cfg->dims.ln_eps, cfg->dims.rms_eps};
  const ModLay ml{(float*)mods, (size_t)B, (size_t)h, (size_t)cfg->n_double, (size_t)cfg->n_single,
                  (size_t)n_sigma, 0};
  size_t at = align_up(ModLay::floats(B, h, cfg->n_double, cfg->n_single, n_sigma) * 4);
  float* temb = (float*)ptr(mods, at);
  at += align_up((size_t)rows * cfg->temb_dim * 4);
  float* hid = (float*)ptr(mods, at);
  at += align_up((size_t)rows * h * 4);
  float* vec = (float*)ptr(mods, at);
  at += align_up((size_t)rows * h * 4);
  void* yrep = ptr(mods, at);
  // conditioning vectors, as in the step, one row per (timestep, batch row)
  for (int j = 0; j < n_sigma; ++j)
    HIP_TRY(launch_timestep_embedding(temb + (size_t)j * B * cfg->temb_dim, B, cfg->temb_dim, sigmas[j], c.s));
  if ((r = gemv(c, w->time_in0, temb, true, cfg->temb_dim, hid, h, false, false))) return r;
  if ((r = gemv(c, w->time_in1, hid, true, h, vec, h, true, false))) return r;
  if (guided) {
    HIP_TRY(launch_timestep_embedding(temb, rows, cfg->temb_dim, opts->guidance, c.s));
    if ((r = gemv(c, w->guidance_in0, temb, true, cfg->temb_dim, hid, h, false, false))) return r;
    if ((r = gemv(c, w->guidance_in1, hid, true, h, vec, h, true, true))) return r;
  }
  for (int j = 0; j < n_sigma; ++j)  // the pooled vectors, once per timestep
    HIP_TRY(launch_convert(y, !g.bf16, ptr(yrep, (size_t)j * B * cfg->vec_in_dim * g.esz), !g.bf16,
                           (int64_t)B * cfg->vec_in_dim, c.s));
  if ((r = gemv(c, w->vec_in0, yrep, false, cfg->vec_in_dim, hid, h, false, false))) return r;
  if ((r = gemv(c, w->vec_in1, hid, true, h, vec, h, true, true))) return r;
  // every modulation matrix, all timesteps in one pass over its weights
  GemvMultiArgs ga{};
  ga.x = vec; ga.K = h; ga.B = rows; ga.x_bstride = h;
  double gemv_bytes = 0;
  auto flush = [&]() -> int {
    if (ga.nseg == 0) return MMDIT_OK;
    ProfScope ps(PC_GEMV, gemv_bytes, c.s);
    HIP_TRY(launch_gemv_multi(ga, g.bf16, c.s));
    ga.nseg = 0;
    gemv_bytes = 0;
    return MMDIT_OK;
  };
  auto add = [&](const mmdit_linear& l, float* out, int y_bstride) -> int {
    GemvSeg& sg = ga.seg[ga.nseg++];
    sg.W = l.w; sg.bias = l.bias; sg.y = out; sg.N = l.n_out; sg.y_bstride = y_bstride;
    gemv_bytes += (double)l.n_out * l.k_in * g.esz;
    return ga.nseg == kGemvMaxSeg ? flush() : MMDIT_OK;
  };
  if ((r = add(w->final_mod, ml.fin(), 2 * h))) return r;
  for (int i = 0; i < cfg->n_double; ++i) {
    if ((r = add(w->dbl[i].txt.mod, ml.dual(i, 0), 6 * h))) return r;
    if ((r = add(w->dbl[i].img.mod, ml.dual(i, 1), 6 * h))) return r;
  }
  for (int i = 0; i < cfg->n_single; ++i)
    if ((r = add(w->sgl[i].mod, ml.single(i), 3 * h))) return r;
  return flush();
}

int mmdit_step_cache_read(const mmdit_config* cfg, mmdit_step_cache* cache, void* hip_stream) {
  Geo g;
  int r;
  if (!cache || !cache->buf) return fail(MMDIT_ERR_NULL, "cache or cache->buf is NULL");
  if ((r = check_config(cfg, g))) return r;
  const CacheLay cl = plan_cache(g);
  if (cache->bytes < cl.total)
    return fail(MMDIT_ERR_WORKSPACE, "cache buffer %zu bytes, need %zu", cache->bytes, cl.total);
  if (!cache->valid) return fail(MMDIT_ERR_SHAPE, "no step of this generation has run (cache->valid == 0)");
  CacheState st;
  const hipStream_t s = (hipStream_t)hip_stream;
  HIP_TRY(hipMemcpyAsync(&st, ptr(cache->buf, cl.state), sizeof st, hipMemcpyDeviceToHost, s));
  HIP_TRY(hipStreamSynchronize(s));
  cache->ran_blocks = st.ran_blocks;
  cache->acc = st.acc;
  cache->rel = st.rel;
  return MMDIT_OK;
}

// One step; the image stream holds Lg = Li - ctx_len generated tokens
// followed by ctx_len context tokens per batch (ctx_packed [B, ctx_len,
// in_ch] float32). Only the generated rows get the final layer and update.
}  // extern "C"

int mmdit::step_impl(const mmdit_config* cfg, const mmdit_model_w* w, void* x_packed, void* v_out,
                     const void* txt_emb, const void* y, const int32_t* ids, double sigma, double sigma_next,
                     const mmdit_step_opts* opts, void* ws, size_t ws_bytes, void* hip_stream) {
  Geo g;
  int r;
  if ((r = check_config(cfg, g))) return r;
  const mmdit_step_opts none{};
  if (!opts) opts = &none;
  if (!w || !x_packed || !ids || (!y && !opts->mods)) return fail(MMDIT_ERR_NULL, "NULL weights, latent, y or ids");
  const void* ctx_packed = opts->ctx_packed;
  const int ctx_len = opts->ctx_len;
  if (ctx_len < 0 || ctx_len >= g.Li)
    return fail(MMDIT_ERR_SHAPE, "ctx_len %d must be in [0, img_len %d)", ctx_len, g.Li);
  if (ctx_len > 0 && !ctx_packed) return fail(MMDIT_ERR_NULL, "ctx_packed is NULL with ctx_len > 0");
  const int Lg = g.Li - ctx_len;  // generated image tokens per batch
  const bool guided = w->guidance_in0.w != nullptr;
  if (guided && !opts->mods) {  // given modulations already hold the guidance
    if (!opts->has_guidance)
      return fail(MMDIT_ERR_NULL, "the model has a guidance embedder: pass a guidance value (mmdit_step_ex)");
    if (!std::isfinite(opts->guidance)) return fail(MMDIT_ERR_SHAPE, "guidance must be finite");
  }
  if (opts->dequant != 0 && opts->dequant != 1) return fail(MMDIT_ERR_SHAPE, "dequant %d must be 0 or 1", opts->dequant);
  if (opts->mods) {
    if (opts->mods_count < 1 || opts->mods_index < 0 || opts->mods_index >= opts->mods_count)
      return fail(MMDIT_ERR_SHAPE, "mods_index %d must be in [0, mods_count %d)", opts->mods_index, opts->mods_count);
    if ((uintptr_t)opts->mods % 16) return fail(MMDIT_ERR_SHAPE, "mods must be 16-byte aligned");
  }
  mmdit_step_cache* cache = opts->cache;
  if (cache) {
    if (std::isnan(opts->cache_threshold) || opts->cache_threshold < 0)
      return fail(MMDIT_ERR_SHAPE, "cache_threshold must be >= 0");
    if (cfg->n_double < 1) return fail(MMDIT_ERR_SHAPE, "step caching needs a dual-stream block");
    if (!cache->buf) return fail(MMDIT_ERR_NULL, "cache->buf is NULL");
    if (cache->bytes < plan_cache(g).total)
      return fail(MMDIT_ERR_WORKSPACE, "cache buffer %zu bytes, need %zu", cache->bytes, plan_cache(g).total);
  }
  if (opts->cache_on_device != 0 && opts->cache_on_device != 1)
    return fail(MMDIT_ERR_SHAPE, "cache_on_device %d must be 0 or 1", opts->cache_on_device);
  const bool dev_cache = cache && opts->cache_on_device == 1;
  if (g.Lt > 0 && !txt_emb) return fail(MMDIT_ERR_NULL, "txt_emb is NULL with txt_len > 0");
  if ((cfg->n_double > 0 && !w->dbl) || (cfg->n_single > 0 && !w->sgl)) return fail(MMDIT_ERR_NULL, "block weight arrays are NULL");
  if (!std::isfinite(sigma) || !std::isfinite(sigma_next)) return fail(MMDIT_ERR_SHAPE, "sigma values must be finite");
  const int h = g.h;
  if ((r = check_linear(w->img_in, h, cfg->in_ch, g, "img_in"))) return r;
  if ((r = check_linear(w->txt_in, h, cfg->txt_in_dim, g, "txt_in"))) return r;
  if ((r = check_gemv(w->time_in0, h, cfg->temb_dim, "time_in0"))) return r;
  if ((r = check_gemv(w->time_in1, h, h, "time_in1"))) return r;
  if ((r = check_gemv(w->vec_in0, h, cfg->vec_in_dim, "vec_in0"))) return r;
  if ((r = check_gemv(w->vec_in1, h, h, "vec_in1"))) return r;
  if (guided) {
    if ((r = check_gemv(w->guidance_in0, h, cfg->temb_dim, "guidance_in0"))) return r;
    if ((r = check_gemv(w->guidance_in1, h, h, "guidance_in1"))) return r;
  }
  if ((r = check_gemv(w->final_mod, 2 * h, h, "final_mod"))) return r;
  if ((r = check_linear(w->final_lin, cfg->in_ch, h, g, "final_lin"))) return r;
  for (int i = 0; i < cfg->n_double; ++i) {
    char nm[32];
    snprintf(nm, sizeof nm, "dbl[%d].txt", i);
    if ((r = check_stream(w->dbl[i].txt, g, nm))) return r;
    snprintf(nm, sizeof nm, "dbl[%d].img", i);
    if ((r = check_stream(w->dbl[i].img, g, nm))) return r;
  }
  for (int i = 0; i < cfg->n_single; ++i)
    if ((r = check_single(w->sgl[i], g))) return fail(r, "sgl[%d]: %s", i, g_err.c_str());
  const bool rb = g.resid == MMDIT_RESID_BF16;  // bf16 residual stream (else float32)
  if (rb && cache) return fail(MMDIT_ERR_UNSUPPORTED, "step caching needs the float32 residual stream");
  const StepWs lay = plan_step(cfg, g, step_decodes(cfg, w, opts, g));
  if (!ws || ws_bytes < lay.blk.total)
    return fail(MMDIT_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, lay.blk.total);

  Ctx c{(hipStream_t)hip_stream, g, cfg->dims.ln_eps, cfg->dims.rms_eps};
  c.xw = lay.blk.xw_bytes && opts->dequant == 0 ? ptr(ws, lay.blk.xw) : nullptr;
  c.xw_bytes = lay.blk.xw_bytes;
  const int B = g.B;
  // residual: [B*Lt text rows; B*Li image rows], float32 (bf16 when rb)
  void* x = ptr(ws, lay.x);
  const int re = rb ? 2 : 4;
  float* vec = (float*)ptr(ws, lay.vec);
  float* temb = (float*)ptr(ws, lay.temb);
  float* hid = (float*)ptr(ws, lay.hid);
  float* table = (float*)ptr(ws, lay.table);
  // modulation vectors: computed below, or given (mmdit_step_modulations)
  const bool given = opts->mods != nullptr;
  const ModLay ml{given ? (float*)opts->mods : (float*)ptr(ws, lay.mods), (size_t)B, (size_t)h,
                  (size_t)cfg->n_double, (size_t)cfg->n_single, given ? (size_t)opts->mods_count : 1,
                  given ? (size_t)opts->mods_index : 0};

  // conditioning vector: L1(SiLU(L0(temb))) + V1(SiLU(V0(y)))
  if (!given) {
    HIP_TRY(launch_timestep_embedding(temb, B, cfg->temb_dim, sigma, c.s));
    if ((r = gemv(c, w->time_in0, temb, true, cfg->temb_dim, hid, h, false, false))) return r;
    if ((r = gemv(c, w->time_in1, hid, true, h, vec, h, true, false))) return r;
    if (guided) {  // + G1(SiLU(G0(temb(guidance))))
      HIP_TRY(launch_timestep_embedding(temb, B, cfg->temb_dim, opts->guidance, c.s));
      if ((r = gemv(c, w->guidance_in0, temb, true, cfg->temb_dim, hid, h, false, false))) return r;
      if ((r = gemv(c, w->guidance_in1, hid, true, h, vec, h, true, true))) return r;
    }
    if ((r = gemv(c, w->vec_in0, y, false, cfg->vec_in_dim, hid, h, false, false))) return r;
    if ((r = gemv(c, w->vec_in1, hid, true, h, vec, h, true, true))) return r;
  }
  // every block's modulation, all from SiLU(vec): batched into launches of
  // up to kGemvMaxSeg weight matrices. The final layer's and the first dual
  // block's image modulation come first: a step that reuses the cached
  // residual needs only those two.
  GemvMultiArgs ga{};
  ga.x = vec; ga.K = h; ga.B = B; ga.x_bstride = h;
  double gemv_bytes = 0;
  auto flush = [&]() -> int {
    if (ga.nseg == 0) return MMDIT_OK;
    ProfScope ps(PC_GEMV, gemv_bytes, c.s);
    ga.skip = c.skip;
    HIP_TRY(launch_gemv_multi(ga, g.bf16, c.s));
    ga.nseg = 0;
    gemv_bytes = 0;
    return MMDIT_OK;
  };
  auto add = [&](const mmdit_linear& l, float* out, int y_bstride) -> int {
    if (given) return MMDIT_OK;
    if (B > kGemvMaxB) return gemv(c, l, vec, true, h, out, y_bstride, true, false);
    GemvSeg& sg = ga.seg[ga.nseg++];
    sg.W = l.w; sg.bias = l.bias; sg.y = out; sg.N = l.n_out; sg.y_bstride = y_bstride;
    gemv_bytes += (double)l.n_out * l.k_in * g.esz;
    return ga.nseg == kGemvMaxSeg ? flush() : MMDIT_OK;
  };
  if ((r = add(w->final_mod, ml.fin(), 2 * h))) return r;
  if (cfg->n_double > 0 && (r = add(w->dbl[0].img.mod, ml.dual(0, 1), 6 * h))) return r;
  if (cache && (r = flush())) return r;
  // the RoPE table depends on the ids only; built before a cached step's
  // decision so that the guarded launches below are the blocks' alone
  if ((r = rope(c, &cfg->dims, ids, table))) return r;

  // image input projection into the f32 residual
  const void* xa = x_packed;
  if (ctx_len > 0) {
    // per batch: [generated rows; context rows] staged in the activation dtype
    const int64_t ci = cfg->in_ch;
    for (int b = 0; b < B; ++b) {
      char* dst = ptr(ws, lay.xin + (size_t)b * g.Li * ci * g.esz);
      HIP_TRY(launch_convert((const float*)x_packed + (size_t)b * Lg * ci, true, dst, !g.bf16, (int64_t)Lg * ci, c.s));
      HIP_TRY(launch_convert((const float*)ctx_packed + (size_t)b * ctx_len * ci, true, dst + (size_t)Lg * ci * g.esz,
                             !g.bf16, (int64_t)ctx_len * ci, c.s));
    }
    xa = ptr(ws, lay.xin);
  } else if (g.bf16) {
    HIP_TRY(launch_convert(x_packed, true, ptr(ws, lay.xin), false, (int64_t)B * g.Li * cfg->in_ch, c.s));
    xa = ptr(ws, lay.xin);
  }
  void* ximg = ptr(x, (size_t)B * g.Lt * h * re);  // image rows, contiguous [B Li h]
  const int64_t nimg = (int64_t)B * g.Li * h;
  {
    GemmProblem gi = base_problem(w->img_in);
    gi.A = xa; gi.lda = cfg->in_ch; gi.M = B * g.Li;
    gi.out = ximg; gi.ldo = h; gi.out_f32 = !rb;
    if ((r = gemm(c, &gi, 1, EPI_STORE))) return r;
  }

  // step cache: indicator, decision, residual
  bool run_blocks = true;
  double rel = 0.0, acc = 0.0;
  float* resid = nullptr;
  if (cache) {
    const CacheLay cl = plan_cache(g);
    resid = (float*)ptr(cache->buf, cl.resid);
    float* part = (float*)ptr(cache->buf, cl.part);
    CacheDeltaArgs ca{};
    ca.x = (const float*)ximg;
    ca.mod = ml.dual(0, 1);  // shift1 at 0, scale1 at h
    ca.mod_bstride = 6 * h;
    ca.rows_per_batch = g.Li;
    ca.prev = (float*)ptr(cache->buf, cl.prev);
    ca.part = part;
    ca.rows = B * g.Li;
    ca.h = h;
    ca.eps = c.ln_eps;
    ca.first = cache->valid ? 0 : 1;
    HIP_TRY(launch_cache_delta(ca, c.s));
    if (dev_cache) {
      // decided on the device: every launch up to the residual store is
      // guarded by the decision's skip flag (graph-capturable, no wait)
      CacheState* st = (CacheState*)ptr(cache->buf, cl.state);
      HIP_TRY(launch_cache_decide(part, B * g.Li, ca.first, opts->cache_threshold, st, c.s));
      HIP_TRY(launch_cache_apply((float*)ximg, resid, nimg, &st->skip, c.s));
      c.skip = &st->skip;
    } else if (cache->valid) {
      std::vector<float> hp((size_t)2 * B * g.Li);
      HIP_TRY(hipMemcpyAsync(hp.data(), part, hp.size() * sizeof(float), hipMemcpyDeviceToHost, c.s));
      HIP_TRY(hipStreamSynchronize(c.s));
      double num = 0.0, den = 0.0;
      for (size_t k = 0; k < hp.size(); k += 2) {
        num += hp[k];
        den += hp[k + 1];
      }
      rel = den > 0.0 ? num / den : (num > 0.0 ? INFINITY : 0.0);
      acc = cache->acc + rel;
      run_blocks = !(acc < opts->cache_threshold);
      if (run_blocks) acc = 0.0;
    }
    if (!dev_cache) {
      if (run_blocks) HIP_TRY(launch_axpby(resid, (const float*)ximg, 0.f, 1.f, nimg, c.s));  // resid <- img0
      else HIP_TRY(launch_axpby((float*)ximg, resid, 1.f, 1.f, nimg, c.s));             // img0 + residual
    }
  }

  Part parts[2];
  parts[0] = {g.Lt, 0, rows_of(x, 0, g.Lt, h, re), rows_of(x, 0, g.Lt, h, re), nullptr};
  parts[1] = {g.Li, (int64_t)B * g.Lt, rows_of(x, (int64_t)B * g.Lt, g.Li, h, re),
              rows_of(x, (int64_t)B * g.Lt, g.Li, h, re), nullptr};
  if (run_blocks) {
    for (int i = 0; i < cfg->n_double; ++i) {
      if ((r = add(w->dbl[i].txt.mod, ml.dual(i, 0), 6 * h))) return r;
      if (i > 0 && (r = add(w->dbl[i].img.mod, ml.dual(i, 1), 6 * h))) return r;
    }
    for (int i = 0; i < cfg->n_single; ++i)
      if ((r = add(w->sgl[i].mod, ml.single(i), 3 * h))) return r;
    if ((r = flush())) return r;
    if (g.Lt > 0) {
      GemmProblem gt = base_problem(w->txt_in);
      gt.A = txt_emb; gt.lda = cfg->txt_in_dim; gt.M = B * g.Lt;
      gt.out = x; gt.ldo = h; gt.out_f32 = !rb;
      if ((r = gemm(c, &gt, 1, EPI_STORE))) return r;
    }
    for (int i = 0; i < cfg->n_double; ++i) {
      parts[0].mod = ml.dual(i, 0);
      parts[1].mod = ml.dual(i, 1);
      const mmdit_stream_w* sw[2] = {&w->dbl[i].txt, &w->dbl[i].img};
      if ((r = run_double(c, sw, parts, !rb, table, ws, lay.blk))) return r;
    }
    for (int i = 0; i < cfg->n_single; ++i) {
      float* ms = ml.single(i);
      parts[0].mod = ms;
      parts[1].mod = ms;
      if (g.Lt > 0) {
        if ((r = run_single(c, w->sgl[i], parts, 2, !rb, table, ws, lay.blk))) return r;
      } else {
        if ((r = run_single(c, w->sgl[i], &parts[1], 1, !rb, table, ws, lay.blk))) return r;
      }
    }
    if (dev_cache) HIP_TRY(launch_cache_store(resid, (const float*)ximg, nimg, c.skip, c.s));  // img - img0
    else if (cache) HIP_TRY(launch_axpby(resid, (const float*)ximg, -1.f, 1.f, nimg, c.s));  // resid <- img - img0
    c.skip = nullptr;
  }
  // final layer on the generated image rows, Euler update fused into the epilogue
  Part fin = parts[1];
  fin.len = Lg;
  fin.x_in.rows_per_batch = Lg;  // batch stride stays Li rows
  fin.mod = ml.fin();
  void* xn = ptr(ws, lay.blk.xn);
  if ((r = run_ln(c, &fin, 1, 2 * h, 0, h, !rb, xn))) return r;
  GemmProblem f = base_problem(w->final_lin);
  f.A = xn; f.lda = h; f.M = B * Lg;
  f.res_out = rows_of(x_packed, 0, Lg, cfg->in_ch, 4);
  f.res_in = f.res_out;
  f.dsigma = (float)(sigma_next - sigma);
  f.v_out = (float*)v_out;
  if ((r = gemm(c, &f, 1, EPI_EULER))) return r;
  if (dev_cache) {
    cache->valid = 1;
    cache->ran_blocks = -1;  // on the device until mmdit_step_cache_read
  } else if (cache) {
    cache->valid = 1;
    cache->ran_blocks = run_blocks ? 1 : 0;
    cache->acc = acc;
    cache->rel = rel;
  }
  return MMDIT_OK;
}

extern "C" {

int mmdit_step(const mmdit_config* cfg, const mmdit_model_w* w, void* x_packed, void* v_out,
               const void* txt_emb, const void* y, const int32_t* ids, double sigma,
               double sigma_next, void* ws, size_t ws_bytes, void* hip_stream) {
  return step_impl(cfg, w, x_packed, v_out, txt_emb, y, ids, sigma, sigma_next, nullptr, ws, ws_bytes, hip_stream);
}

int mmdit_step_ex(const mmdit_config* cfg, const mmdit_model_w* w, void* x_packed, void* v_out,
                  const void* txt_emb, const void* y, const int32_t* ids, double sigma, double sigma_next,
                  const mmdit_step_opts* opts, void* ws, size_t ws_bytes, void* hip_stream) {
  return step_impl(cfg, w, x_packed, v_out, txt_emb, y, ids, sigma, sigma_next, opts, ws, ws_bytes, hip_stream);
}

// ------------------------------------------------------------ single ops --
int mmdit_adaln_layernorm(const void* x, int32_t x_f32, void* y, int32_t act_dtype, int32_t rows, int32_t hidden,
                          const float* shift_scale, float eps, void* hip_stream) {
  if (rows < 0) return fail(MMDIT_ERR_SHAPE, "rows %d < 0", rows);
  if (rows == 0) return MMDIT_OK;
  if (!x || !y || !shift_scale) return fail(MMDIT_ERR_NULL, "NULL x, y or shift_scale");
  if (act_dtype != MMDIT_F32 && act_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "act_dtype %d", act_dtype);
  if (hidden < 256 || hidden > 4096 || hidden % 256)
    return fail(MMDIT_ERR_SHAPE, "hidden %d must be a multiple of 256 in [256, 4096]", hidden);
  if (!(eps > 0)) return fail(MMDIT_ERR_SHAPE, "eps must be > 0");
  const bool bf = act_dtype == MMDIT_BF16;
  const bool xf = x_f32 || !bf;
  if ((uintptr_t)x % 16 || (uintptr_t)y % 16 || (uintptr_t)shift_scale % 16)
    return fail(MMDIT_ERR_SHAPE, "x, y and shift_scale must be 16-byte aligned");
  LnArgs a{};
  RowSeg r;
  r.base = const_cast<void*>(x);
  r.batch_stride = (int64_t)rows * hidden;
  r.rows_per_batch = rows;
  r.ld = hidden;
  a.seg[0] = a.seg[1] = r;
  a.seg_rows[0] = rows;
  a.seg_rows[1] = 0;
  a.mod[0] = a.mod[1] = shift_scale;
  a.mod_bstride = 0;
  a.shift_off = 0;
  a.scale_off = hidden;
  a.y = y;
  a.h = hidden;
  a.eps = eps;
  ProfScope ps(PC_LN, (double)rows * hidden * ((xf ? 4 : 2) + (bf ? 2 : 4)), (hipStream_t)hip_stream);
  HIP_TRY(launch_adaln_ln(a, rows, xf, bf, (hipStream_t)hip_stream));
  return MMDIT_OK;
}

// Route of mmdit_linear_fwd for bf16 activations.
static int linear_route(const mmdit_linear& l, int M, int route) {
  if (route != MMDIT_ROUTE_AUTO) return route;
  if (M <= 16 && l.k_in % 128 == 0) return MMDIT_ROUTE_STREAM;
  if (l.fmt != MMDIT_W_DENSE && M >= kExpandMinRows) return MMDIT_ROUTE_DECODE;
  return MMDIT_ROUTE_TILED;
}

static int check_linear_call(const mmdit_linear* l, int32_t act_dtype, int32_t M, int32_t route, Geo& g) {
  if (!l) return fail(MMDIT_ERR_NULL, "linear is NULL");
  if (act_dtype != MMDIT_F32 && act_dtype != MMDIT_BF16) return fail(MMDIT_ERR_DTYPE, "act_dtype %d", act_dtype);
  if (M < 0 || l->n_out < 1 || l->k_in < 1) return fail(MMDIT_ERR_SHAPE, "need M >= 0, n_out >= 1, k_in >= 1");
  if (route < MMDIT_ROUTE_AUTO || route > MMDIT_ROUTE_STREAM) return fail(MMDIT_ERR_SHAPE, "route %d", route);
  g = Geo{};
  g.B = 1;
  g.bf16 = act_dtype == MMDIT_BF16;
  g.esz = g.bf16 ? 2 : 4;
  g.L = M;
  int r;
  if ((r = check_linear(*l, l->n_out, l->k_in, g, "linear"))) return r;
  if (!g.bf16 && route != MMDIT_ROUTE_AUTO && route != MMDIT_ROUTE_TILED)
    return fail(MMDIT_ERR_UNSUPPORTED, "float32 layers run on the tiled route only");
  if (g.bf16) {
    const int rt = linear_route(*l, M, route);
    if (rt == MMDIT_ROUTE_STREAM && (M > 16 || l->k_in % 128))
      return fail(MMDIT_ERR_SHAPE, "the weight-streaming route needs M <= 16 and k_in a multiple of 128");
    if (rt == MMDIT_ROUTE_DECODE && l->fmt == MMDIT_W_DENSE)
      return fail(MMDIT_ERR_SHAPE, "the decoding route needs a quantised layer");
  }
  if ((int64_t)M * l->k_in >= (int64_t(1) << 31) || (int64_t)M * l->n_out >= (int64_t(1) << 31))
    return fail(MMDIT_ERR_SHAPE, "M * width too large for 32-bit indexing");
  return MMDIT_OK;
}

int mmdit_linear_workspace(const mmdit_linear* l, int32_t act_dtype, int32_t M, int32_t route, size_t* bytes) {
  Geo g;
  int r;
  if (!bytes) return fail(MMDIT_ERR_NULL, "bytes is NULL");
  if ((r = check_linear_call(l, act_dtype, M, route, g))) return r;
  *bytes = g.bf16 && linear_route(*l, M, route) == MMDIT_ROUTE_DECODE ? align_up((size_t)l->n_out * l->k_in * 2) : 0;
  return MMDIT_OK;
}

int mmdit_linear_fwd(const mmdit_linear* l, int32_t act_dtype, const void* x, int32_t M, void* y, int32_t y_f32,
                     int32_t route, void* ws, size_t ws_bytes, void* hip_stream) {
  Geo g;
  int r;
  if ((r = check_linear_call(l, act_dtype, M, route, g))) return r;
  if (M == 0) return MMDIT_OK;
  if (!x || !y) return fail(MMDIT_ERR_NULL, "NULL x or y");
  if ((uintptr_t)x % 16 || (uintptr_t)y % 16) return fail(MMDIT_ERR_SHAPE, "x and y must be 16-byte aligned");
  const hipStream_t st = (hipStream_t)hip_stream;
  const bool yf = y_f32 || !g.bf16;
  const int rt = g.bf16 ? linear_route(*l, M, route) : MMDIT_ROUTE_TILED;
  size_t need = 0;
  if ((r = mmdit_linear_workspace(l, act_dtype, M, route, &need))) return r;
  if (need && (!ws || ws_bytes < need)) return fail(MMDIT_ERR_WORKSPACE, "workspace %zu bytes, need %zu", ws_bytes, need);
  if (rt == MMDIT_ROUTE_STREAM) {
    // the kernel reads 16-byte pieces of dense, 4-bit and 8-bit rows (8 and
    // 4 bytes of ternary and 1-bit rows) and 4-byte pairs of 4/8-bit scales
    const int wal = l->fmt == MMDIT_W_Q1G128 ? 4 : l->fmt == MMDIT_W_TQ2G128 ? 8 : 16;
    if ((uintptr_t)l->w % wal || (l->scales && (uintptr_t)l->scales % 4))
      return fail(MMDIT_ERR_SHAPE, "weight-streaming route: weights must be %d-byte and scales 4-byte aligned", wal);
    const double wb = l->fmt == MMDIT_W_DENSE ? 2.0 : l->fmt == MMDIT_W_Q4G64 ? 0.5 + 2.0 / 64
                      : l->fmt == MMDIT_W_Q8G64 ? 1.0 + 2.0 / 64 : l->fmt == MMDIT_W_Q1G128 ? 0.125 + 2.0 / 128
                      : 0.25 + 2.0 / 128;
    ProfScope ps(PC_STREAM, (double)l->n_out * l->k_in * wb, st);
    HIP_TRY(launch_linear_skinny(x, M, l->w, l->scales, l->bias, l->fmt, y, yf, l->n_out, l->k_in, st));
    return MMDIT_OK;
  }
  Ctx c{st, g, 1e-6f, 1e-6f};
  if (rt == MMDIT_ROUTE_DECODE) {
    c.xw = ws;
    c.xw_bytes = ws_bytes;
  }
  GemmProblem p = base_problem(*l);
  p.A = x; p.lda = l->k_in; p.M = M;
  p.out = y; p.ldo = l->n_out; p.out_f32 = yf;
  return gemm(c, &p, 1, EPI_STORE);
}

int mmdit_pack_latents(const void* z, void* x, int32_t B, int32_t C, int32_t H, int32_t W,
                       int32_t elem_bytes, void* hip_stream) {
  if (!z || !x) return fail(MMDIT_ERR_NULL, "NULL buffer");
  if (B < 1 || C < 1 || H < 2 || W < 2 || H % 2 || W % 2) return fail(MMDIT_ERR_SHAPE, "need B, C >= 1 and even H, W >= 2");
  if (elem_bytes != 2 && elem_bytes != 4) return fail(MMDIT_ERR_DTYPE, "elem_bytes must be 2 or 4");
  HIP_TRY(launch_pack(z, x, B, C, H, W, elem_bytes, false, (hipStream_t)hip_stream));
  return MMDIT_OK;
}

int mmdit_unpack_latents(const void* x, void* z, int32_t B, int32_t C, int32_t H, int32_t W,
                         int32_t elem_bytes, void* hip_stream) {
  if (!z || !x) return fail(MMDIT_ERR_NULL, "NULL buffer");
  if (B < 1 || C < 1 || H < 2 || W < 2 || H % 2 || W % 2) return fail(MMDIT_ERR_SHAPE, "need B, C >= 1 and even H, W >= 2");
  if (elem_bytes != 2 && elem_bytes != 4) return fail(MMDIT_ERR_DTYPE, "elem_bytes must be 2 or 4");
  HIP_TRY(launch_pack(x, z, B, C, H, W, elem_bytes, true, (hipStream_t)hip_stream));
  return MMDIT_OK;
}

int mmdit_rope_table(const int32_t* ids, int32_t L, const int32_t* axes_dim, double theta,
                     float* table, void* hip_stream) {
  if (!ids || !axes_dim || !table) return fail(MMDIT_ERR_NULL, "NULL buffer");
  if (L < 0) return fail(MMDIT_ERR_SHAPE, "L < 0");
  for (int a = 0; a < 3; ++a)
    if (axes_dim[a] < 0 || axes_dim[a] % 2) return fail(MMDIT_ERR_SHAPE, "axes must be even");
  if (!(theta > 0)) return fail(MMDIT_ERR_SHAPE, "theta must be > 0");
  HIP_TRY(launch_rope_table(ids, L, axes_dim[0], axes_dim[1], axes_dim[2], theta, table, (hipStream_t)hip_stream));
  return MMDIT_OK;
}

int mmdit_profile_begin(int32_t kernel_class, int32_t max_launches) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (kernel_class < PC_GEMM || kernel_class > PC_STREAM) return fail(MMDIT_ERR_SHAPE, "unknown kernel class %d", kernel_class);
  if (max_launches < 1 || max_launches > 1 << 20) return fail(MMDIT_ERR_SHAPE, "max_launches out of range");
  if (g_prof.active) return fail(MMDIT_ERR_UNSUPPORTED, "profiling already active");
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  for (auto& e : g_prof.ev) HIP_TRY(hipEventCreate(&e));
  g_prof.gen++;
  g_prof.cls = kernel_class;
  g_prof.cap = max_launches;
  g_prof.used = 0;
  g_prof.work = 0;
  g_prof.active = true;
  return MMDIT_OK;
}

int mmdit_profile_end(double* total_ms, int32_t* launches, double* work) {
  std::lock_guard<std::mutex> lk(g_prof.mu);
  if (!g_prof.active) return fail(MMDIT_ERR_UNSUPPORTED, "profiling not active");
  g_prof.active = false;
  double tot = 0;
  for (int i = 0; i < g_prof.used; ++i) {
    HIP_TRY(hipEventSynchronize(g_prof.ev[2 * i + 1]));
    float ms = 0;
    HIP_TRY(hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]));
    tot += ms;
  }
  if (total_ms) *total_ms = tot;
  if (launches) *launches = g_prof.used;
  if (work) *work = g_prof.work;
  for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
  g_prof.ev.clear();
  return MMDIT_OK;
}

const char* mmdit_status_str(int32_t status) {
  switch (status) {
    case MMDIT_OK: return "ok";
    case MMDIT_ERR_NULL: return "null pointer";
    case MMDIT_ERR_SHAPE: return "invalid shape";
    case MMDIT_ERR_DTYPE: return "invalid dtype or weight format";
    case MMDIT_ERR_WORKSPACE: return "workspace too small";
    case MMDIT_ERR_UNSUPPORTED: return "unsupported";
    case MMDIT_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* mmdit_last_error(void) { return g_err.c_str(); }

const char* mmdit_version(void) { return "mmdit 0.1 gfx950"; }

}  // extern "C"
