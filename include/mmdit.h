/*
 * mmdit.h - C ABI of the MI355X (gfx950) FLUX-style MMDiT denoising step.
 *
 * The library computes the denoising step of a multimodal diffusion
 * transformer: dual-stream blocks (separate text and image weights, joint
 * attention), single-stream blocks over the concatenated [text; image]
 * sequence, the conditioning vector and the flow-matching Euler update.
 * Sources: mflux-rs "Native Apple Silicon FLUX.1 in Safe Rust", section
 * "FLUX.1 MMDiT Architecture" (cards Dual-Stream MMDiT, Single-Stream Blocks,
 * 3D RoPE Coordinates, Flow-Matching Euler) and its patch-packing calculator;
 * the mistral.rs FLUX.1-schnell article, section on FluxStepper and its
 * sampling parameters; the stable-diffusion.rs README on quantised weights
 * dequantised inside the matmul.
 *
 * Conventions for every entry point:
 *  - Memory. The caller owns every buffer. Pointers documented as "device"
 *    are HIP device allocations on the current device; "host" pointers are
 *    ordinary CPU memory. The library never allocates or frees device memory
 *    and keeps no device state between calls. Weight structs hold borrowed
 *    device pointers.
 *  - Streams. Device work is enqueued on `hip_stream` (a hipStream_t passed
 *    as void*, NULL = the null stream) and the call returns without waiting.
 *    Faults inside kernels surface at the caller's next synchronisation.
 *  - Errors. Every function returns an mmdit_status. Argument, shape, format
 *    and workspace checks all run before the first launch, so on an error no
 *    kernel has been enqueued and no output has been written.
 *    mmdit_last_error() returns a per-thread text describing the last error.
 *  - Layouts. Matrices are row-major. Activations are [B, tokens, width].
 *    Joint sequences put the text tokens first, then the image tokens.
 *  - Re-entrancy. Calls on distinct streams with distinct workspaces may run
 *    concurrently.
 */
#ifndef MMDIT_H
#define MMDIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MMDIT_OK = 0,
  MMDIT_ERR_NULL = 1,        /* a required pointer is NULL */
  MMDIT_ERR_SHAPE = 2,       /* sizes inconsistent or out of the supported range */
  MMDIT_ERR_DTYPE = 3,       /* dtype / weight format not valid for this call */
  MMDIT_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required */
  MMDIT_ERR_UNSUPPORTED = 5, /* valid request the library does not implement */
  MMDIT_ERR_HIP = 6          /* a HIP runtime call failed (detail in mmdit_last_error) */
} mmdit_status;

typedef enum { MMDIT_F32 = 0, MMDIT_BF16 = 1 } mmdit_dtype;

/* Storage of the residual stream (the block inputs and outputs that the gated
 * residual updates add into). DEFAULT: the block calls keep it in the
 * activation dtype, mmdit_step in float32 (pictor README: FP32 accumulate;
 * reading: a bf16 residual random walk over 76 additions would spend a large
 * part of the bf16 error budget). F32: float32 everywhere (block inputs and
 * outputs are float32 arrays). BF16: bf16 everywhere (needs bf16
 * activations; mmdit_step then holds its residual in bf16). */
typedef enum { MMDIT_RESID_DEFAULT = 0, MMDIT_RESID_F32 = 1, MMDIT_RESID_BF16 = 2 } mmdit_resid;

/* Weight storage of one linear layer y = x W^T + b.
 * DENSE: W [n_out, k_in] in the activation dtype.
 * Q4G64: symmetric 4-bit codes in -7..7, two's complement nibbles, two per
 *        byte with the even k in the low nibble: uint8 [n_out, k_in/2];
 *        scales bf16 [n_out, k_in/64], one per group of 64 consecutive k.
 * Q8G64: symmetric 8-bit codes in -127..127: int8 [n_out, k_in]; scales as Q4G64.
 * The dequantised weight is code * scale. Quantised formats need bf16
 * activations and k_in % 64 == 0. (stable-diffusion.rs README: weights held
 * quantised at rest and dequantised inside the matmul a tile at a time.) */
/* Sub-byte formats with groups of 128 along k (pictor-tokenizer page: 1-bit
 * Q1_0_g128 and ternary TQ2_0_g128 weights; reading for the layout and the
 * scale, which the page does not give): per row and group, one bf16 scale
 * s >= 0 in scales bf16 [n_out, k_in/128];
 * Q1G128: one bit per weight, uint8 [n_out, k_in/8], weight k at bit k%8 of
 *   byte k/8; bit 1 -> +s, bit 0 -> -s.
 * TQ2G128: two bits per weight, uint8 [n_out, k_in/4], weight k at bits
 *   2(k%4), 2(k%4)+1 of byte k/4; code 0 -> -s, 2 -> +s, 1 and 3 -> 0.
 * They need bf16 activations and k_in % 128 == 0. */
typedef enum { MMDIT_W_DENSE = 0, MMDIT_W_Q4G64 = 1, MMDIT_W_Q8G64 = 2, MMDIT_W_Q1G128 = 3,
               MMDIT_W_TQ2G128 = 4 } mmdit_wfmt;

typedef struct {
  int32_t batch;       /* B >= 1 */
  int32_t hidden;      /* h = heads * head_dim, a multiple of 256 */
  int32_t heads;       /* H >= 1 */
  int32_t head_dim;    /* d; must be 128 */
  int32_t mlp_hidden;  /* m, a multiple of 64 */
  int32_t txt_len;     /* Lt >= 0 text tokens */
  int32_t img_len;     /* Li >= 1 image tokens */
  int32_t axes_dim[3]; /* RoPE axes (frame, row, col), each even, summing to head_dim */
  double theta;        /* RoPE base (10000) */
  float ln_eps;        /* LayerNorm epsilon (1e-6) */
  float rms_eps;       /* QK RMSNorm epsilon (1e-6) */
  int32_t act_dtype;   /* mmdit_dtype of activations, dense weights, biases, norm scales */
  int32_t resid;       /* mmdit_resid: storage of the residual stream (0 = default) */
} mmdit_dims;

typedef struct {
  const void* w;       /* device; layout per mmdit_wfmt */
  const void* scales;  /* device bf16 [n_out, k_in/64] (Q4G64/Q8G64) or [n_out, k_in/128] (Q1G128/TQ2G128), else NULL */
  const void* bias;    /* device [n_out] in the activation dtype, or NULL for no bias */
  int32_t fmt;         /* mmdit_wfmt */
  int32_t n_out;
  int32_t k_in;
} mmdit_linear;

/* One stream (text or image) of a dual-stream block.
 * mod: h -> 6h, output split (shift1, scale1, gate1, shift2, scale2, gate2).
 * qkv: h -> 3h, output columns [q | k | v], each head-major (head, dim).
 * proj: h -> h.  fc1: h -> m (GELU-tanh).  fc2: m -> h.
 * q_norm, k_norm: device RMSNorm scales [head_dim], shared by all heads. */
typedef struct {
  mmdit_linear mod, qkv, proj, fc1, fc2;
  const void* q_norm;
  const void* k_norm;
} mmdit_stream_w;

typedef struct {
  mmdit_stream_w img, txt;
} mmdit_double_w;

/* Single-stream block. mod: h -> 3h split (shift, scale, gate).
 * lin1: h -> 3h + m with columns [q | k | v | mlp].
 * lin2: h + m -> h, input columns [attention | GELU(mlp)]. */
typedef struct {
  mmdit_linear mod, lin1, lin2;
  const void* q_norm;
  const void* k_norm;
} mmdit_single_w;

typedef struct {
  mmdit_dims dims;
  int32_t n_double;    /* dual-stream blocks (19 for FLUX.1) */
  int32_t n_single;    /* single-stream blocks (38 for FLUX.1) */
  int32_t in_ch;       /* packed latent channels (64 = 16 channels x 2x2), a multiple of 64 */
  int32_t txt_in_dim;  /* text embedding width (4096 for T5), a multiple of 64 */
  int32_t vec_in_dim;  /* pooled text vector width (768) */
  int32_t temb_dim;    /* sinusoidal timestep embedding width (256), even */
} mmdit_config;

/* Whole-model weights. img_in: in_ch -> h. txt_in: txt_in_dim -> h.
 * time_in0: temb_dim -> h, time_in1: h -> h. vec_in0: vec_in_dim -> h,
 * vec_in1: h -> h. final_mod: h -> 2h split (shift, scale). final_lin: h -> in_ch.
 * dbl / sgl: HOST arrays of n_double / n_single block weight structs.
 * guidance_in0: temb_dim -> h, guidance_in1: h -> h: the guidance embedder of
 * guidance-distilled models (FLUX.1-dev: mflux-rs card, generation with a
 * guidance scale; mistral.rs article, FluxStepper guidance_scale). All-zero
 * (guidance_in0.w == NULL) for models without one (schnell). */
typedef struct {
  mmdit_linear img_in, txt_in, time_in0, time_in1, vec_in0, vec_in1, final_mod, final_lin;
  const mmdit_double_w* dbl;
  const mmdit_single_w* sgl;
  mmdit_linear guidance_in0, guidance_in1;
} mmdit_model_w;

/* Workspace sizes in bytes (host-only; no device work). With bf16
 * activations and at least 1024 rows (batch * (txt_len + img_len), context
 * tokens included) a call with a quantised layer decodes each such layer
 * once per launch into room in the workspace (2 bytes per weight of the
 * largest launch: both streams' fc1 or fc2, or linear1; 151 MB at h 3072)
 * and multiplies the bf16 copy with the dense kernels (profile class 8);
 * below 1024 rows the GEMM kernels dequantise weight tiles as they stage
 * them. Both give the same bf16 weights. These three queries do not see the
 * weights and always include that room; the calls themselves need it only
 * when they decode a layer, so a dense model needs the smaller size that
 * mmdit_step_workspace_ex reports for the step (the block calls check
 * against the size for their own weights the same way). */
int mmdit_double_block_workspace(const mmdit_dims* dims, size_t* bytes);
int mmdit_single_block_workspace(const mmdit_dims* dims, size_t* bytes);
int mmdit_step_workspace(const mmdit_config* cfg, size_t* bytes);

/* Dual-stream block forward (mflux-rs, card "Dual-Stream MMDiT").
 * img_in [B, Li, h], txt_in [B, Lt, h]: device, activation dtype.
 * img_out, txt_out: same shapes; each may alias its input.
 * vec [B, h]: device, activation dtype; modulation = W_mod SiLU(vec) + b.
 * ids [Lt + Li, 3]: device int32 position ids (frame, row, col), text first,
 *   shared by the batch; RoPE angles are ids[:, a] * theta^(-2j/axes_dim[a]).
 * ws: device workspace of at least mmdit_double_block_workspace() bytes.
 * img_in/txt_in/img_out/txt_out are the residual stream: in the activation
 * dtype, or float32 when dims->resid is MMDIT_RESID_F32. */
int mmdit_double_block_fwd(const mmdit_dims* dims, const mmdit_double_w* w,
                           const void* img_in, const void* txt_in, void* img_out, void* txt_out,
                           const void* vec, const int32_t* ids,
                           void* ws, size_t ws_bytes, void* hip_stream);

/* Single-stream block forward (mflux-rs, card "Single-Stream Blocks").
 * x_in, x_out [B, Lt + Li, h]: device, activation dtype (float32 when
 * dims->resid is MMDIT_RESID_F32), text rows first; x_out may alias x_in.
 * vec, ids and ws as for the dual block. */
int mmdit_single_block_fwd(const mmdit_dims* dims, const mmdit_single_w* w,
                           const void* x_in, void* x_out, const void* vec, const int32_t* ids,
                           void* ws, size_t ws_bytes, void* hip_stream);

/* One denoising step (mflux-rs architecture cards and "Flow-Matching Euler").
 * x_packed [B, Li, in_ch]: device float32 packed latent, updated in place to
 *   x + (sigma_next - sigma) * v.
 * v_out [B, Li, in_ch]: device float32 velocity, or NULL.
 * txt_emb [B, Lt, txt_in_dim], y [B, vec_in_dim]: device, activation dtype.
 * ids as for the blocks. sigma, sigma_next: the schedule pair of this step;
 * the timestep embedding uses 1000 * sigma.
 * Inside the step the residual stream is float32 whatever the activation
 * dtype, or bf16 when cfg->dims.resid is MMDIT_RESID_BF16. */
int mmdit_step(const mmdit_config* cfg, const mmdit_model_w* w,
               void* x_packed, void* v_out, const void* txt_emb, const void* y,
               const int32_t* ids, double sigma, double sigma_next,
               void* ws, size_t ws_bytes, void* hip_stream);

/* Options of mmdit_step_ex; a zeroed struct (or opts == NULL) is mmdit_step.
 *
 * Reference-image tokens (FLUX.1-Kontext instruction editing:
 * stable-diffusion.rs README, the Kontext example with a reference picture;
 * the frame axis of the ids: mflux-rs card, 3D RoPE visualiser, axis 0
 * temporal). Reading where the pages are silent: per batch, the image stream
 * is the Lg = img_len - ctx_len generated tokens followed by the ctx_len
 * context tokens; the context latent goes through the same input projection;
 * ids carry frame 1 for the context tokens (the caller builds them); the
 * velocity and the update cover the generated tokens only.
 *   ctx_packed [B, ctx_len, in_ch]: device float32 packed context latent, read
 *   only; NULL when ctx_len is 0. 0 <= ctx_len < cfg->dims.img_len.
 *
 * Guidance (FLUX.1-dev: mflux-rs card, generation with guidance 3.5;
 * mistral.rs article: guidance models run 50 shifted steps with
 * guidance_scale 4.0). Reading: like the timestep, the guidance value g is
 * embedded as temb(1000 g) and mapped by guidance_in0 / SiLU / guidance_in1;
 * the result is added to the conditioning vector.
 *   has_guidance: 1 to pass `guidance`; required (and only used) when the
 *   model has a guidance embedder.
 *
 * Step caching (stable-diffusion.rs README: step caching behind a cache
 * threshold, for deterministic samplers only, credited to TeaCache). Reading
 * where the pages are silent: each step computes a = (1 + scale1) LN(img0) +
 * shift1 with the first dual block's image-stream modulation, img0 the image
 * tokens after the input projection (context tokens included), and its
 * relative L1 change rel = sum|a - a_prev| / sum|a_prev| against the previous
 * step; rel is added to a running sum. While the sum stays below the
 * threshold the step skips every block and adds the image-stream residual
 * (image tokens after the last block minus img0) of the last step that ran
 * the blocks to img0; otherwise it runs the blocks, stores their residual and
 * resets the sum to 0. A first step (valid == 0) always runs the blocks.
 *   cache: the generation's state (below), NULL for no caching.
 *   cache_threshold: >= 0; 0 runs the blocks on every step.
 *   cache_on_device: 0 = the host decides: the step waits for its stream
 *   once to read rel back, and fills ran_blocks, acc and rel before it
 *   returns (not capturable into a HIP graph). 1 = a kernel decides: the
 *   decision state (acc, rel, ran_blocks) stays in cache->buf, every launch
 *   of the blocks is enqueued and does nothing when the step reuses the
 *   residual, and the call never waits, so the step can be captured into a
 *   HIP graph; read the state with mmdit_step_cache_read. A graph captured
 *   with valid == 1 continues the generation on each replay; start a
 *   generation with an ordinary call (valid == 0). The results are bit for
 *   bit those of cache_on_device = 0.
 * Needs n_double >= 1. */
typedef struct {
  void* buf;          /* device memory of mmdit_step_cache_bytes(cfg) bytes, caller-owned;
                         the library keeps a_prev and the residual there (float32) */
  size_t bytes;       /* size of buf */
  int32_t valid;      /* in/out: 0 starts a generation; set to 1 by a successful step.
                         After an error return, set it to 0 before the next step. */
  int32_t ran_blocks; /* out: 1 if the step ran the blocks, 0 if it reused the residual;
                         -1 after a cache_on_device step (see mmdit_step_cache_read) */
  double acc;         /* in/out: summed rel since the last step that ran the blocks */
  double rel;         /* out: the step's rel (0 when it started a generation) */
} mmdit_step_cache;

/* Host. Bytes of mmdit_step_cache.buf for cfg (2 B img_len hidden floats for
 * a_prev and the residual, per-row partial sums and 32 bytes of decision
 * state). */
int mmdit_step_cache_bytes(const mmdit_config* cfg, size_t* bytes);

/* Host, waits for hip_stream. After steps with cache_on_device = 1: copies
 * the decision of the last step enqueued on hip_stream from cache->buf into
 * cache->ran_blocks, acc and rel. Errors: MMDIT_ERR_NULL (cache or buf),
 * MMDIT_ERR_WORKSPACE (cache->bytes too small), MMDIT_ERR_SHAPE (valid == 0:
 * no step has run), MMDIT_ERR_HIP. */
int mmdit_step_cache_read(const mmdit_config* cfg, mmdit_step_cache* cache, void* hip_stream);

/* dequant (quantised layers only): 0 = automatic (decoded once per launch
 * into bf16 scratch from 1024 rows on, see the workspace functions), 1 =
 * always dequantised inside the GEMM while staging weight tiles. */
typedef struct {
  const void* ctx_packed;
  int32_t ctx_len;
  int32_t has_guidance;
  double guidance;
  mmdit_step_cache* cache;
  double cache_threshold;
  int32_t dequant;
  int32_t cache_on_device; /* 0 or 1, see step caching above */
  /* Modulation vectors computed beforehand by mmdit_step_modulations (device,
   * 16-byte aligned), or NULL to compute them in the step. mods_count: the
   * n_sigma of that call; mods_index: which of its timesteps this step is
   * (its sigma must be the one the step is called with; the library cannot
   * check that). With mods set the step neither reads y nor needs a
   * guidance value. */
  const void* mods;
  int32_t mods_count;
  int32_t mods_index;
} mmdit_step_opts;

/* One denoising step with options (context tokens, guidance). Arguments as
 * for mmdit_step, except: cfg->dims.img_len counts generated plus context
 * tokens; x_packed, v_out are [B, Lg, in_ch]; ids [txt_len + img_len, 3] are
 * text, generated, then context rows. The workspace is
 * mmdit_step_workspace(cfg). Errors as for mmdit_step; MMDIT_ERR_SHAPE for
 * ctx_len out of range, a non-finite guidance, a negative or NaN
 * cache_threshold, caching without a dual block, dequant or
 * cache_on_device not 0 or 1, mods_index outside [0, mods_count) or mods
 * misaligned;
 * MMDIT_ERR_NULL for a NULL
 * ctx_packed with ctx_len > 0, a NULL cache->buf, or a guidance model called
 * without a guidance value (mmdit_step on such a model fails the same way);
 * MMDIT_ERR_WORKSPACE for cache->bytes below mmdit_step_cache_bytes(cfg). */
int mmdit_step_ex(const mmdit_config* cfg, const mmdit_model_w* w,
                  void* x_packed, void* v_out, const void* txt_emb, const void* y,
                  const int32_t* ids, double sigma, double sigma_next, const mmdit_step_opts* opts,
                  void* ws, size_t ws_bytes, void* hip_stream);

/* Host. Bytes of the buffer mmdit_step_modulations fills for n_sigma
 * timesteps: n_sigma * batch * hidden * (12 n_double + 3 n_single + 2)
 * floats of modulation vectors plus scratch for the conditioning vectors.
 * Errors: MMDIT_ERR_NULL, config errors, MMDIT_ERR_SHAPE when n_sigma is
 * below 1 or n_sigma * batch exceeds 4. */
int mmdit_step_modulations_bytes(const mmdit_config* cfg, int32_t n_sigma, size_t* bytes);

/* Device, async. The conditioning vectors and every modulation vector of the
 * step (each block's adaLN shift / scale / gate chunks and the final layer's)
 * for the n_sigma timesteps sigmas[0 .. n_sigma) (host array) at once: each
 * modulation weight matrix is read once for all of them instead of once per
 * step (these weights are 6.5 GB at h 3072, the step's largest HBM stream;
 * they depend on the step only through the conditioning vector, mflux-rs
 * page, Dual-Stream MMDiT and Single-Stream Blocks cards). y [B, vec_in_dim]
 * as for mmdit_step; opts: only has_guidance / guidance are read (required
 * when the model has a guidance embedder). mods: device buffer of
 * mmdit_step_modulations_bytes(cfg, n_sigma) bytes, 16-byte aligned, passed
 * to the steps as opts->mods with mods_count = n_sigma and mods_index = j for
 * the step at sigmas[j]. The results are bit for bit those a step computes
 * for itself. Errors: MMDIT_ERR_NULL, MMDIT_ERR_SHAPE (n_sigma, alignment,
 * non-finite sigma or guidance), MMDIT_ERR_WORKSPACE (mods_bytes too small),
 * MMDIT_ERR_DTYPE, MMDIT_ERR_HIP; nothing is launched on an argument error. */
int mmdit_step_modulations(const mmdit_config* cfg, const mmdit_model_w* w, const void* y, const double* sigmas,
                           int32_t n_sigma, const mmdit_step_opts* opts, void* mods, size_t mods_bytes,
                           void* hip_stream);

/* Host. The workspace mmdit_step_ex needs for these weights and options
 * (opts may be NULL): without room for decoded weights when no layer is
 * decoded (dense weights, fewer than 1024 rows, or opts->dequant == 1).
 * w->dbl / w->sgl are read; device pointers are not touched. Errors:
 * MMDIT_ERR_NULL, and those of mmdit_step_workspace. */
int mmdit_step_workspace_ex(const mmdit_config* cfg, const mmdit_model_w* w, const mmdit_step_opts* opts,
                            size_t* bytes);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops that must not call hipMalloc): mmdit_step_ex
 * without a workspace argument. The workspace is a scratch array the library
 * holds in device memory, 256 MiB (268435456 bytes) on each GPU the library
 * is loaded on, for the life of the process. Configurations whose
 * mmdit_step_workspace() exceeds that size are refused with
 * MMDIT_ERR_WORKSPACE before any launch (the 512x512 step at h 3072 fits; the
 * 1024x1024 step does not). Every call on one GPU uses that GPU's one array:
 * calls that overlap on a GPU (other streams or threads) race and give
 * undefined results; calls on one stream are ordered. The step initialises
 * every scratch byte it reads, so nothing is carried between calls. The
 * first call on a device resolves the array's device address (no
 * allocation). Arguments and errors as for mmdit_step_ex; opts may be NULL. */
int mmdit_step_noalloc(const mmdit_config* cfg, const mmdit_model_w* w,
                       void* x_packed, void* v_out, const void* txt_emb, const void* y,
                       const int32_t* ids, double sigma, double sigma_next, const mmdit_step_opts* opts,
                       void* hip_stream);

/* ---- helpers ---------------------------------------------------------- */

/* Host. sigmas[0..n_steps] of the shifted flow-matching schedule: t_i = 1 - i/n,
 * mu = base + (max - base) * (img_len - 256) / (4096 - 256) when shift != 0 else 0,
 * sigma_i = e^mu / (e^mu + 1/t_i - 1), sigma_n = 0. With sigma_terminal > 0 and
 * n_steps >= 2 the non-zero sigmas are stretched so the last equals
 * sigma_terminal. (mistral.rs article, FluxStepper shift 0.5 / 1.15; mflux-rs
 * card "Flow-Matching Euler", sigma_terminal 0.02.) */
int mmdit_schedule(int32_t n_steps, int32_t img_len, double base_shift, double max_shift,
                   double sigma_terminal, int32_t shift, double* sigmas);

/* Host. ids [txt_len + grid_h*grid_w, 3] int32: text rows (0,0,0); image
 * token r*grid_w + c gets (frame, r, c). (mflux-rs RoPE visualiser: axis 0
 * frame, axis 1 row, axis 2 column.) */
int mmdit_make_ids(int32_t grid_h, int32_t grid_w, int32_t txt_len, int32_t frame, int32_t* ids);

/* Device, async. Bit-exact 2x2 patch packing of z [B, C, H, W] into
 * x [B, (H/2)(W/2), 4C] with x[b, hp*(W/2)+wp, c*4+ph*2+pw] = z[b, c, 2hp+ph, 2wp+pw],
 * and its inverse. elem_bytes is 2 or 4; values are moved as raw bits.
 * (mflux-rs patch packing calculator; telemetry: bit-exact bijection.) */
int mmdit_pack_latents(const void* z, void* x, int32_t B, int32_t C, int32_t H, int32_t W,
                       int32_t elem_bytes, void* hip_stream);
int mmdit_unpack_latents(const void* x, void* z, int32_t B, int32_t C, int32_t H, int32_t W,
                         int32_t elem_bytes, void* hip_stream);

/* Device, async. RoPE table [L, sum(axes)/2, 2] float32 (cos, sin) for ids
 * [L, 3] (mflux-rs, card "3D RoPE Coordinates" and its RoPE visualiser: the
 * head dimension split over the (frame, row, column) axes, here axes_dim).
 * Pair j of axis a turns by ids[:, a] * theta^(-2j / axes_dim[a]); the pairs
 * run axis 0, then 1, then 2. Angles are evaluated in float64 and stored as
 * float32; the blocks build the same table. ids and table are device
 * arrays, axes_dim a host array of 3. Errors: MMDIT_ERR_NULL,
 * MMDIT_ERR_SHAPE (L < 0, odd or negative axes, theta <= 0), MMDIT_ERR_HIP. */
int mmdit_rope_table(const int32_t* ids, int32_t L, const int32_t* axes_dim, double theta,
                     float* table, void* hip_stream);

/* Host. Symmetric group quantiser for w [n_out, k_in] float32 (host).
 * bits 4 or 8 (k_in % 64 == 0): per row and group of 64 k,
 * s = smallest bf16 >= max|w| / qmax (qmax 7 or 127), q = round-half-even(w / s),
 * all-zero group -> s = 0, q = 0. packed: host, n_out*k_in/2 bytes (4-bit,
 * even k in the low nibble) or n_out*k_in bytes (8-bit); scales_bf16: host
 * [n_out, k_in/64].
 * bits 1 (Q1G128) or 2 (TQ2G128), k_in % 128 == 0: per row and group of 128
 * k, m = sum of |w| in k order in float64, divided by 128, rounded to float32
 * then to bf16 (both to nearest even): s. 1-bit: bit = (w >= 0). 2-bit:
 * q = round-half-even(w / s) in float64 clamped to [-1, 1] (q = 0 when
 * s = 0), code q + 1. (The absmean scale; for sign codes it is the
 * least-squares scale.) packed: n_out*k_in/8 or n_out*k_in/4 bytes;
 * scales_bf16: [n_out, k_in/128]. */
int mmdit_quantise(const float* w, int32_t n_out, int32_t k_in, int32_t bits,
                   void* packed, uint16_t* scales_bf16);

/* Device. Decodes a quantised weight matrix into dense bf16 out [n_out, k_in]
 * (stable-diffusion.rs README: weights held quantised and dequantised for
 * the matmul; pictor page: Q1_0_g128 / TQ2_0_g128), giving the weights the
 * GEMMs multiply: code * scale rounded to bf16 (nearest even) for
 * MMDIT_W_Q4G64 / MMDIT_W_Q8G64, exactly +s, -s or 0 for MMDIT_W_Q1G128 /
 * MMDIT_W_TQ2G128. w (packed codes) and scales (bf16) are device arrays in
 * the layouts of mmdit_wfmt; out is device memory the caller owns. w must be
 * 16-byte aligned (8 for ternary, 4 for 1-bit), scales 2-byte and out
 * 16-byte aligned. Enqueued on hip_stream (NULL: the null stream).
 * Errors: MMDIT_ERR_NULL; MMDIT_ERR_DTYPE for fmt not one of the four
 * quantised formats; MMDIT_ERR_SHAPE for n_out < 0, k_in not a positive
 * multiple of the format's group, or misaligned pointers; MMDIT_ERR_HIP. */
int mmdit_dequantise(const void* w, const void* scales, int32_t fmt, int32_t n_out, int32_t k_in,
                     void* out, void* hip_stream);

/* ---- single operations ------------------------------------------------ */

/* Device, async. adaLN-modulated LayerNorm of `rows` rows (mflux-rs cards
 * "Dual-Stream MMDiT" / "Single-Stream Blocks": LayerNorm modulated by shift
 * and scale from the conditioning vector; stable-diffusion.rs README: fused
 * layer_norm): y[r, :] = (1 + scale) * LN(x[r, :]) + shift, LN without
 * affine, biased variance, statistics in float32. x [rows, hidden]: float32
 * when x_f32 (or act_dtype is F32), else bf16; y [rows, hidden] in act_dtype;
 * shift_scale: device float32 [2, hidden], shift then scale, shared by all
 * rows. hidden a multiple of 256 in [256, 4096]; pointers 16-byte aligned.
 * The same kernel as the blocks' modulated LayerNorm. Errors:
 * MMDIT_ERR_NULL, MMDIT_ERR_DTYPE, MMDIT_ERR_SHAPE, MMDIT_ERR_HIP. */
int mmdit_adaln_layernorm(const void* x, int32_t x_f32, void* y, int32_t act_dtype, int32_t rows, int32_t hidden,
                          const float* shift_scale, float eps, void* hip_stream);

/* Routes of mmdit_linear_fwd (bf16 activations). AUTO: STREAM for M <= 16
 * (k_in a multiple of 128), else DECODE for quantised weights from 1024
 * rows, else TILED. TILED: the tiled MFMA GEMMs, quantised weight tiles
 * dequantised as they are staged (stable-diffusion.rs README: dequantised
 * inside the matmul a tile at a time). DECODE: the quantised layer decoded
 * once into the workspace as bf16 (the values mmdit_dequantise gives), then
 * the dense tiled GEMM. STREAM: the weight-streaming kernel for M <= 16:
 * every weight read once, codes decoded in registers (HBM-bound). */
typedef enum { MMDIT_ROUTE_AUTO = 0, MMDIT_ROUTE_TILED = 1, MMDIT_ROUTE_DECODE = 2, MMDIT_ROUTE_STREAM = 3 } mmdit_route;

/* Host. Workspace bytes of mmdit_linear_fwd: 2 * n_out * k_in (rounded up)
 * when the route decodes, else 0. */
int mmdit_linear_workspace(const mmdit_linear* l, int32_t act_dtype, int32_t M, int32_t route, size_t* bytes);

/* Device, async. One linear layer y = x W^T + b of the step (any projection,
 * weights in any mmdit_wfmt): x [M, k_in] in act_dtype (row stride k_in),
 * y [M, n_out] float32 when y_f32 (or act_dtype is F32), else bf16; both
 * device, 16-byte aligned. route: mmdit_route (float32 activations: AUTO or
 * TILED only). ws: device workspace of mmdit_linear_workspace() bytes (may
 * be NULL when that is 0). Results are the bf16-operand, float32-accumulated
 * products the blocks compute; the weight-streaming route multiplies each
 * 4-bit group's float32 sum of q x by its scale instead of rounding s q to
 * bf16 first. The weight-streaming route needs l->w 16-byte aligned (8 for
 * ternary, 4 for 1-bit) and l->scales 4-byte aligned. Errors:
 * MMDIT_ERR_NULL, MMDIT_ERR_DTYPE (format / dtype), MMDIT_ERR_SHAPE (sizes,
 * a route the shape does not allow, alignment), MMDIT_ERR_WORKSPACE,
 * MMDIT_ERR_UNSUPPORTED, MMDIT_ERR_HIP. */
int mmdit_linear_fwd(const mmdit_linear* l, int32_t act_dtype, const void* x, int32_t M, void* y, int32_t y_f32,
                     int32_t route, void* ws, size_t ws_bytes, void* hip_stream);

/* Kernel timing for benchmarks. While enabled, each launch of the selected
 * kernel class is bracketed by HIP events recorded on the launch stream.
 * classes: 1 = GEMMs (all projections), 2 = joint attention,
 * 3 = adaLN LayerNorm, 4 = QK RMSNorm + RoPE, 5 = modulation / conditioning
 * GEMV, 6 = single-block linear1 GEMM (split GELU epilogue), 7 = GEMMs with
 * the gated-residual epilogue (out-projection, fc2, linear2), 8 = decoding of
 * quantised weights to bf16 ahead of a launch, 9 = dual-block QKV GEMM (QK
 * RMSNorm + RoPE epilogue), 10 = dual-block fc1 GEMM (GELU epilogue),
 * 11 = weight-streaming linear (mmdit_linear_fwd, STREAM route; work = weight
 * bytes).
 * mmdit_profile_begin creates up to max_launches event pairs (host call, no
 * device allocation). mmdit_profile_end waits for the recorded events and
 * returns the summed kernel time, the launch count and the summed algorithmic
 * FLOPs (classes 1, 2, 6, 7, 9, 10) or bytes (classes 3-5, 8, 11) of those
 * launches.
 * Thread-safe; a launch whose call is still in progress when
 * mmdit_profile_end runs on another thread is not counted. */
int mmdit_profile_begin(int32_t kernel_class, int32_t max_launches);
int mmdit_profile_end(double* total_ms, int32_t* launches, double* work);

const char* mmdit_status_str(int32_t status);
const char* mmdit_last_error(void);
/* Library version string, e.g. "mmdit 0.1 gfx950". */
const char* mmdit_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MMDIT_H */
