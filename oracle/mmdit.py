"""Plain NumPy definitions of the MMDiT denoising step (test infrastructure;
only tests, the smoke check and the benchmark's CPU baseline may use it).

Arrays are computed in the dtype of the inputs (float32 by default;
float64 for small checks). Contractions use np.matmul; everything else is
the formula written out. There is no blocking, fusion or reordering.

Notation: h hidden width, H heads, d head dim (128), m MLP width,
Lt text tokens, Li image tokens, L = Lt + Li, B batch.
"""
from __future__ import annotations

import math
from typing import Dict, Sequence, Tuple

import numpy as np

LN_EPS = 1e-6
RMS_EPS = 1e-6


# ------------------------------------------------------------- packing -----
def pack_latents(z: np.ndarray) -> np.ndarray:
    """Packed image tokens from a latent z [B, C, H, W].

    mflux-rs, "Patch Packing & Memory Calculator": a 128x128 latent becomes
    a 64x64 patch grid of 4096 tokens, and the "Dual-Stream MMDiT" card
    speaks of 64-channel patches (16 channels x 2x2). The telemetry table
    requires the packing to be a bit-exact bijection.
    Reading: token index hp*Wp + wp, channel index c*4 + ph*2 + pw, i.e.
        X[b, hp*Wp + wp, c*4 + ph*2 + pw] = z[b, c, 2*hp + ph, 2*wp + pw].
    """
    B, C, H, W = z.shape
    if H % 2 or W % 2:
        raise ValueError("latent height and width must be even")
    Hp, Wp = H // 2, W // 2
    X = np.empty((B, Hp * Wp, 4 * C), dtype=z.dtype)
    for c in range(C):
        for ph in range(2):
            for pw in range(2):
                X[:, :, c * 4 + ph * 2 + pw] = z[:, c, ph::2, pw::2].reshape(B, Hp * Wp)
    return X


def unpack_latents(X: np.ndarray, C: int, H: int, W: int) -> np.ndarray:
    """Inverse of pack_latents: z[b, c, 2hp+ph, 2wp+pw] = X[b, hp*Wp+wp, c*4+ph*2+pw]."""
    B = X.shape[0]
    Hp, Wp = H // 2, W // 2
    if X.shape != (B, Hp * Wp, 4 * C):
        raise ValueError("packed shape does not match the latent size")
    z = np.empty((B, C, H, W), dtype=X.dtype)
    for c in range(C):
        for ph in range(2):
            for pw in range(2):
                z[:, c, ph::2, pw::2] = X[:, :, c * 4 + ph * 2 + pw].reshape(B, Hp, Wp)
    return z


# ---------------------------------------------------------- position ids ---
def make_ids(grid_h: int, grid_w: int, txt_len: int, frame: int = 0) -> np.ndarray:
    """Position ids [Lt + gh*gw, 3] int32, text first.

    mflux-rs, "3D Rotary Position Embedding (RoPE) Visualizer": axis 0 is
    the temporal/frame coordinate, axis 1 the row, axis 2 the column.
    Reading: text tokens get (0, 0, 0); image token k = r*gw + c gets
    (frame, r, c) with frame 0 for a plain text-to-image step.
    """
    ids = np.zeros((txt_len + grid_h * grid_w, 3), dtype=np.int32)
    for r in range(grid_h):
        for c in range(grid_w):
            k = txt_len + r * grid_w + c
            ids[k, 0] = frame
            ids[k, 1] = r
            ids[k, 2] = c
    return ids


# ------------------------------------------------------------------ RoPE ---
def rope_frequencies(axes_dim: Sequence[int] = (16, 56, 56), theta: float = 10000.0):
    """Per-axis rotation frequencies omega_{a,j} = theta^(-2j/d_a), j < d_a/2
    (float64), for the axes [16, 56, 56] of the "3D RoPE Coordinates" card."""
    return [theta ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d) for d in axes_dim]


def rope_table(ids: np.ndarray, axes_dim=(16, 56, 56), theta: float = 10000.0):
    """cos, sin tables [L, sum(axes)/2] float32.

    mflux-rs, "3D RoPE Coordinates" and the RoPE visualiser: the head dim
    128 is split over axes [16, 56, 56]. Reading: the 64 rotation pairs are
    laid out axis 0 (8 pairs), then axis 1 (28), then axis 2 (28); pair j of
    axis a turns by angle ids[:, a] * omega_{a,j}. Angles and their cos/sin
    are evaluated in float64 and stored as float32.
    """
    freqs = rope_frequencies(axes_dim, theta)
    ang = np.concatenate(
        [ids[:, a:a + 1].astype(np.float64) * freqs[a][None, :] for a in range(len(axes_dim))],
        axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate adjacent pairs (2k, 2k+1) of the last axis of x [..., L, d]:
        y_2k   = cos_k x_2k - sin_k x_2k+1
        y_2k+1 = sin_k x_2k + cos_k x_2k+1
    (reading: interleaved pairs, the FLUX convention)."""
    c = cos.astype(x.dtype)
    s = sin.astype(x.dtype)
    x0 = x[..., 0::2]
    x1 = x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = c * x0 - s * x1
    y[..., 1::2] = s * x0 + c * x1
    return y


# ----------------------------------------------------------------- norms ---
def layer_norm(x: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """LayerNorm over the last axis without affine parameters (stable-
    diffusion.rs credits the fused layer_norm kernel; reading: biased
    variance, eps 1e-6, the affine part comes from adaLN)."""
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + x.dtype.type(eps))


def modulate(x: np.ndarray, shift: np.ndarray, scale: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """adaLN modulation (1 + scale) * LN(x) + shift; shift/scale [B, 1, h]
    broadcast over tokens (reading: the adaLN-Zero "1 + scale" form)."""
    return (1 + scale) * layer_norm(x, eps) + shift


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) * g, g of size d
    shared across heads (stable-diffusion.rs credits the fused rms_norm
    kernel; reading: eps 1e-6, applied to q and k per head)."""
    ms = (x * x).mean(axis=-1, keepdims=True)
    return x / np.sqrt(ms + x.dtype.type(eps)) * g.astype(x.dtype)


# ----------------------------------------------------------- pointwise -----
def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))."""
    k = x.dtype.type(math.sqrt(2.0 / math.pi))
    return x.dtype.type(0.5) * x * (1 + np.tanh(k * (x + x.dtype.type(0.044715) * x * x * x)))


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU u / (1 + exp(-u))."""
    return x / (1 + np.exp(-x))


def linear(x: np.ndarray, w: np.ndarray, b) -> np.ndarray:
    """y = x W^T + b with W [N, K] (reading: every linear carries a bias)."""
    y = np.matmul(x, w.astype(x.dtype).T)
    if b is not None:
        y = y + b.astype(x.dtype)
    return y


# ------------------------------------------------------------ attention ----
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Softmax attention per (batch, head) on [B, H, L, d], no mask, scale
    1/sqrt(d): every text and image token attends to every token (mflux-rs
    "Dual-Stream MMDiT": bidirectional attention between text and image;
    "Single-Stream Blocks": one self-attention sequence)."""
    B, H, L, d = q.shape
    out = np.empty_like(q)
    scale = q.dtype.type(1.0 / math.sqrt(d))
    for b in range(B):
        for hh in range(H):
            s = np.matmul(q[b, hh], k[b, hh].T) * scale
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=-1, keepdims=True)
            out[b, hh] = np.matmul(p, v[b, hh])
    return out


def _heads(x: np.ndarray, H: int, d: int) -> np.ndarray:
    """[B, L, H*d] -> [B, H, L, d] (head-major columns)."""
    B, L, _ = x.shape
    return x.reshape(B, L, H, d).transpose(0, 2, 1, 3)


def _merge(x: np.ndarray) -> np.ndarray:
    """[B, H, L, d] -> [B, L, H*d]."""
    B, H, L, d = x.shape
    return x.transpose(0, 2, 1, 3).reshape(B, L, H * d)


def _chunks(m: np.ndarray, n: int):
    """Split a modulation vector [B, n*h] into n pieces [B, 1, h]."""
    B, nh = m.shape
    h = nh // n
    return [m[:, None, i * h:(i + 1) * h] for i in range(n)]


# ---------------------------------------------------------------- blocks ---
def double_block(w: Dict[str, Dict[str, np.ndarray]], x_img: np.ndarray, x_txt: np.ndarray,
                 vec: np.ndarray, ids: np.ndarray, heads: int, axes_dim=(16, 56, 56),
                 theta: float = 10000.0) -> Tuple[np.ndarray, np.ndarray]:
    """Dual-stream block (mflux-rs "Dual-Stream MMDiT": separate text and
    image weights, joint attention over both token sets).

    Per stream s with its own weights:
      mod_s = W_mod SiLU(vec) + b -> (shift1, scale1, gate1, shift2, scale2, gate2)
      [q|k|v] = modulate(x_s; shift1, scale1) W_qkv^T + b   (columns q, k, v, head-major)
      q, k <- RMSNorm per head (stream's own q/k scales)
    Joint: Q = [q_txt; q_img] (text first), K, V likewise; RoPE(ids) on Q, K;
      O = softmax(QK^T/sqrt d) V, split back into text and image rows.
    Per stream: x_s += gate1 * (O_s W_proj^T + b)
                x_s += gate2 * (GELU(modulate(x_s; shift2, scale2) W_fc1^T + b) W_fc2^T + b)
    Returns (x_img, x_txt).
    """
    dt = x_img.dtype
    d = x_img.shape[-1] // heads
    Lt = x_txt.shape[1]
    xs = {"txt": x_txt.astype(dt), "img": x_img.astype(dt)}
    mods, qs, ks, vs = {}, {}, {}, {}
    for s in ("txt", "img"):
        ws = w[s]
        mods[s] = _chunks(linear(silu(vec.astype(dt)), ws["mod_w"], ws["mod_b"]), 6)
        sh1, sc1 = mods[s][0], mods[s][1]
        qkv = linear(modulate(xs[s], sh1, sc1), ws["qkv_w"], ws["qkv_b"])
        hd = heads * d
        qs[s] = rms_norm(_heads(qkv[..., 0:hd], heads, d), ws["q_norm"])
        ks[s] = rms_norm(_heads(qkv[..., hd:2 * hd], heads, d), ws["k_norm"])
        vs[s] = _heads(qkv[..., 2 * hd:3 * hd], heads, d)
    cos, sin = rope_table(ids, axes_dim, theta)
    Q = apply_rope(np.concatenate([qs["txt"], qs["img"]], axis=2), cos, sin)
    K = apply_rope(np.concatenate([ks["txt"], ks["img"]], axis=2), cos, sin)
    V = np.concatenate([vs["txt"], vs["img"]], axis=2)
    O = _merge(attention(Q, K, V))
    Os = {"txt": O[:, :Lt], "img": O[:, Lt:]}
    for s in ("txt", "img"):
        ws = w[s]
        _, _, g1, sh2, sc2, g2 = mods[s]
        x = xs[s] + g1 * linear(Os[s], ws["proj_w"], ws["proj_b"])
        hmid = gelu_tanh(linear(modulate(x, sh2, sc2), ws["fc1_w"], ws["fc1_b"]))
        xs[s] = x + g2 * linear(hmid, ws["fc2_w"], ws["fc2_b"])
    return xs["img"], xs["txt"]


def single_block(w: Dict[str, np.ndarray], x: np.ndarray, vec: np.ndarray, ids: np.ndarray,
                 heads: int, axes_dim=(16, 56, 56), theta: float = 10000.0) -> np.ndarray:
    """Single-stream block on x = [txt; img] (mflux-rs "Single-Stream Blocks":
    text and image tokens as one self-attention sequence).

      (shift, scale, gate) = W_mod SiLU(vec) + b
      [q|k|v|r] = modulate(x; shift, scale) W_1^T + b       widths h, h, h, m
      q, k <- RoPE(RMSNorm(q)), RoPE(RMSNorm(k));  O = softmax(QK^T/sqrt d) V
      x += gate * ([O | GELU(r)] W_2^T + b)       (attention columns first)
    """
    dt = x.dtype
    hd = x.shape[-1]
    d = hd // heads
    sh, sc, g = _chunks(linear(silu(vec.astype(dt)), w["mod_w"], w["mod_b"]), 3)
    y = linear(modulate(x, sh, sc), w["lin1_w"], w["lin1_b"])
    q = rms_norm(_heads(y[..., 0:hd], heads, d), w["q_norm"])
    k = rms_norm(_heads(y[..., hd:2 * hd], heads, d), w["k_norm"])
    v = _heads(y[..., 2 * hd:3 * hd], heads, d)
    cos, sin = rope_table(ids, axes_dim, theta)
    O = _merge(attention(apply_rope(q, cos, sin), apply_rope(k, cos, sin), v))
    r = gelu_tanh(y[..., 3 * hd:])
    return x + g * linear(np.concatenate([O, r], axis=-1), w["lin2_w"], w["lin2_b"])


# ---------------------------------------------------------- conditioning ---
def timestep_embedding(sigma: float, dim: int = 256, max_period: float = 10000.0,
                       dtype=np.float32) -> np.ndarray:
    """Sinusoidal embedding of tau = 1000 * sigma (mflux-rs ODE solver table
    lists a timestep beside each sigma). Reading: f_i = exp(-ln(max_period)
    * i / (dim/2)), output [cos(tau f) | sin(tau f)], evaluated in float64."""
    half = dim // 2
    tau = 1000.0 * float(sigma)
    f = np.exp(-math.log(max_period) * np.arange(half, dtype=np.float64) / half)
    a = tau * f
    return np.concatenate([np.cos(a), np.sin(a)]).astype(dtype)


def conditioning_vec(g: Dict[str, np.ndarray], sigma, y: np.ndarray, temb_dim: int = 256,
                     guidance=None) -> np.ndarray:
    """vec [B, h] = L1(SiLU(L0(temb(sigma)))) + V1(SiLU(V0(y))) with y the
    pooled text vector (mistral.rs article: FluxStepper encodes with T5 and
    CLIP). Without guidance weights (schnell) that is all.

    Guidance-distilled models (FLUX.1-dev: mflux-rs card, generation with a
    guidance scale; mistral.rs article, guidance models with guidance_scale
    4.0) also add G1(SiLU(G0(temb(guidance)))): reading, the guidance value
    is embedded exactly like the timestep (1000 g, the same sinusoid) by its
    own two-layer map. `guidance` is required when g holds guidance_in0_w."""
    dt = y.dtype
    B = y.shape[0]
    t = np.broadcast_to(timestep_embedding(sigma, temb_dim, dtype=dt), (B, temb_dim))
    vt = linear(silu(linear(t, g["time_in0_w"], g["time_in0_b"])), g["time_in1_w"], g["time_in1_b"])
    vy = linear(silu(linear(y, g["vec_in0_w"], g["vec_in0_b"])), g["vec_in1_w"], g["vec_in1_b"])
    if g.get("guidance_in0_w") is None:
        return vt + vy
    if guidance is None:
        raise ValueError("guidance-distilled weights need a guidance value")
    e = np.broadcast_to(timestep_embedding(guidance, temb_dim, dtype=dt), (B, temb_dim))
    vg = linear(silu(linear(e, g["guidance_in0_w"], g["guidance_in0_b"])), g["guidance_in1_w"], g["guidance_in1_b"])
    return vt + vg + vy


def final_layer(g: Dict[str, np.ndarray], img: np.ndarray, vec: np.ndarray) -> np.ndarray:
    """Velocity v = modulate(img; shift, scale) W_out^T + b with
    (shift, scale) = W_fm SiLU(vec) + b (reading: shift first)."""
    sh, sc = _chunks(linear(silu(vec), g["final_mod_w"], g["final_mod_b"]), 2)
    return linear(modulate(img, sh, sc), g["final_w"], g["final_b"])


# ------------------------------------------------------------------ step ---
def step(g: Dict[str, np.ndarray], dbl: Sequence, sgl: Sequence, X: np.ndarray, T: np.ndarray,
         y: np.ndarray, ids: np.ndarray, sigma: float, sigma_next: float, heads: int,
         axes_dim=(16, 56, 56), theta: float = 10000.0, Xc: np.ndarray = None, guidance=None):
    """One denoising step (mflux-rs architecture cards and "Flow-Matching
    Euler"): project packed latents [B, Li, 64] and text embeddings
    [B, Lt, 4096] to width h, run the dual-stream blocks, concatenate
    [txt; img], run the single-stream blocks, take the image rows, apply the
    final layer to get v, and return (X + (sigma_next - sigma) v, v).

    Xc [B, Lc, 64]: optional packed reference-image latent (FLUX.1-Kontext
    editing, stable-diffusion.rs README; frame axis of the ids, mflux-rs 3D
    RoPE visualiser). Reading: its tokens follow the generated ones in the
    image stream, through the same input projection, with ids carrying frame
    1 (ids covers [txt; generated; context]); v and the update are taken for
    the generated rows only. guidance: passed to conditioning_vec."""
    dt = X.dtype
    Lg = X.shape[1]
    img = linear(X if Xc is None else np.concatenate([X, Xc.astype(dt)], axis=1), g["img_in_w"], g["img_in_b"])
    txt = linear(T.astype(dt), g["txt_in_w"], g["txt_in_b"])
    vec = conditioning_vec(g, sigma, y.astype(dt), temb_dim=g["time_in0_w"].shape[1], guidance=guidance)
    for i in range(len(dbl)):
        img, txt = double_block(dbl[i], img, txt, vec, ids, heads, axes_dim, theta)
    x = np.concatenate([txt, img], axis=1)
    for i in range(len(sgl)):
        x = single_block(sgl[i], x, vec, ids, heads, axes_dim, theta)
    v = final_layer(g, x[:, T.shape[1]:T.shape[1] + Lg], vec)
    return euler_update(X, v, sigma, sigma_next), v


# ---------------------------------------------------------- step caching ---
# stable-diffusion.rs README: step caching behind a cache threshold, only
# with a deterministic sampler, credited to TeaCache. The pages give no
# formula; reading: the change of the first dual block's modulated image
# input between consecutive steps, measured as a relative L1 distance and
# summed since the last step that ran the blocks, decides whether the blocks
# run again (sum >= threshold) or their image-stream residual from that step
# is added to this step's image tokens instead.
def rel_l1(a: np.ndarray, p: np.ndarray) -> float:
    """sum |a - p| / sum |p| over every element, in float64 (0 when both sums
    are 0, inf when only the second is)."""
    num = float(np.abs(a.astype(np.float64) - p.astype(np.float64)).sum())
    den = float(np.abs(p.astype(np.float64)).sum())
    if den == 0.0:
        return 0.0 if num == 0.0 else math.inf
    return num / den


def cache_decide(valid: bool, acc: float, rel: float, threshold: float):
    """(run_blocks, new_acc): a first step always runs the blocks; later
    steps add rel to the running sum and reuse the residual while the sum
    stays below the threshold; running the blocks resets the sum to 0."""
    if not valid:
        return True, 0.0
    acc = acc + rel
    if acc < threshold:
        return False, acc
    return True, 0.0


def new_cache_state() -> dict:
    """Cache state of one generation: prev (last modulated input), resid
    (image-stream residual of the last step that ran the blocks), acc, valid."""
    return {"prev": None, "resid": None, "acc": 0.0, "valid": False}


def step_cached(g: Dict[str, np.ndarray], dbl: Sequence, sgl: Sequence, X: np.ndarray, T: np.ndarray,
                y: np.ndarray, ids: np.ndarray, sigma: float, sigma_next: float, heads: int, state: dict,
                threshold: float, axes_dim=(16, 56, 56), theta: float = 10000.0, Xc: np.ndarray = None,
                guidance=None):
    """One denoising step with step caching (reading above). Needs a dual
    block. The indicator is a = modulate(img0; shift1, scale1) of the first
    dual block's image stream, img0 the image tokens after the input
    projection (context tokens included). state (new_cache_state()) is
    updated in place. Returns (X_next, v, ran_blocks, rel)."""
    if len(dbl) == 0:
        raise ValueError("step caching needs a dual-stream block")
    dt = X.dtype
    Lg = X.shape[1]
    img0 = linear(X if Xc is None else np.concatenate([X, Xc.astype(dt)], axis=1), g["img_in_w"], g["img_in_b"])
    vec = conditioning_vec(g, sigma, y.astype(dt), temb_dim=g["time_in0_w"].shape[1], guidance=guidance)
    sh1, sc1 = _chunks(linear(silu(vec.astype(dt)), dbl[0]["img"]["mod_w"], dbl[0]["img"]["mod_b"]), 6)[:2]
    a = modulate(img0, sh1, sc1)
    rel = rel_l1(a, state["prev"]) if state["valid"] else 0.0
    run, acc = cache_decide(state["valid"], state["acc"], rel, threshold)
    if run:
        img = img0
        txt = linear(T.astype(dt), g["txt_in_w"], g["txt_in_b"])
        for i in range(len(dbl)):
            img, txt = double_block(dbl[i], img, txt, vec, ids, heads, axes_dim, theta)
        x = np.concatenate([txt, img], axis=1)
        for i in range(len(sgl)):
            x = single_block(sgl[i], x, vec, ids, heads, axes_dim, theta)
        img = x[:, T.shape[1]:]
        state["resid"] = img - img0
    else:
        img = img0 + state["resid"]
    state["prev"] = a
    state["acc"] = acc
    state["valid"] = True
    v = final_layer(g, img[:, :Lg], vec)
    return euler_update(X, v, sigma, sigma_next), v, run, rel


# -------------------------------------------------------------- schedule ---
def mu_for_tokens(img_len: int, base_shift: float = 0.5, max_shift: float = 1.15,
                  lo: int = 256, hi: int = 4096) -> float:
    """Shift mu interpolated linearly in the image token count between
    (256, base_shift) and (4096, max_shift) (mistral.rs article: base_shift
    0.5, max_shift 1.15; reading: the FLUX endpoints 256 and 4096)."""
    return base_shift + (max_shift - base_shift) * (img_len - lo) / (hi - lo)


def time_shift(mu: float, t):
    """Exponential time shift sigma(t) = e^mu / (e^mu + (1/t - 1)) for
    0 < t <= 1 (mflux-rs "Flow-Matching Euler": shift factor mu; the
    telemetry table checks the t -> 1 limit and strict monotonicity)."""
    t = np.asarray(t, dtype=np.float64)
    em = math.exp(mu)
    return em / (em + (1.0 / t - 1.0))


def schedule(n_steps: int, img_len: int, base_shift: float = 0.5, max_shift: float = 1.15,
             sigma_terminal: float = 0.0, shift: bool = True) -> np.ndarray:
    """sigmas [n_steps + 1] float64 for t_i = 1 - i/N, shifted by mu, with
    sigma_N = 0 (the t = 0 limit). Optional terminal stretch (mflux-rs names
    sigma_terminal = 0.02 without a formula; reading, off by default): with
    off_i = 1 - sigma_i over the non-zero sigmas, sigma_i <- 1 - off_i *
    (1 - sigma_terminal) / off_last, so the last non-zero sigma becomes
    sigma_terminal."""
    if n_steps < 1:
        raise ValueError("n_steps must be >= 1")
    t = 1.0 - np.arange(n_steps + 1, dtype=np.float64) / n_steps
    sig = np.zeros(n_steps + 1, dtype=np.float64)
    mu = mu_for_tokens(img_len, base_shift, max_shift) if shift else 0.0
    sig[:-1] = time_shift(mu, t[:-1])
    if sigma_terminal > 0.0 and n_steps >= 2:
        off = 1.0 - sig[:-1]
        sig[:-1] = 1.0 - off * ((1.0 - sigma_terminal) / off[-1])
    return sig


def euler_update(X: np.ndarray, v: np.ndarray, sigma: float, sigma_next: float) -> np.ndarray:
    """Flow-matching Euler step X + (sigma_next - sigma) v (mflux-rs ODE
    solver table, column dt; dt < 0 as sigma falls)."""
    return X + X.dtype.type(sigma_next - sigma) * v


# ------------------------------------------------------------- quantiser ---
def bf16_round_up(a: np.ndarray) -> np.ndarray:
    """Smallest bf16 value >= a (a >= 0, float32), returned as float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    up = (u & np.uint32(0xFFFF)) != 0
    r = (u >> np.uint32(16)) + up.astype(np.uint32)
    return (r << np.uint32(16)).view(np.float32)


def quantise(w: np.ndarray, bits: int, group: int = 64):
    """Symmetric group quantisation along K (stable-diffusion.rs: weights
    held as packed bits, dequantised a tile at a time; 4-bit and 8-bit).

    Per output row n and group g of `group` consecutive k, in float32:
      s = smallest bf16 >= max|w| / qmax  (qmax 7 for 4-bit, 127 for 8-bit)
      q = round_half_even(w / s), so |q| <= qmax; an all-zero group has s = q = 0.
    Returns q [N, K] int8 and s [N, K/group] float32 (bf16-valued).
    """
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    qmax = np.float32(7 if bits == 4 else 127)
    wg = w.astype(np.float32).reshape(N, K // group, group)
    amax = np.abs(wg).max(axis=-1)
    s = bf16_round_up(amax / qmax)
    safe = np.where(s > 0, s, np.float32(1.0))
    q = np.rint(wg / safe[..., None])
    q = np.where(s[..., None] > 0, q, 0)
    q = np.clip(q, -qmax, qmax).astype(np.int8)
    return q.reshape(N, K), s


def dequantise(q: np.ndarray, s: np.ndarray, group: int = 64) -> np.ndarray:
    """w_hat = q * s per group (exact in float32)."""
    N, K = q.shape
    return (q.reshape(N, K // group, group).astype(np.float32) * s[..., None]).reshape(N, K)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, two per byte, the even k in the low nibble."""
    u = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    lo = (p & 0xF).astype(np.int16)
    hi = (p >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((p.shape[0], 2 * p.shape[1]), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


# ------------------------------------------- sub-byte weights (group 128) ---
def bf16_rne(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return (r << np.uint32(16)).view(np.float32)


def quantise_g128(w: np.ndarray, bits: int):
    """1-bit (Q1_0_g128) and ternary (TQ2_0_g128) weights with groups of 128
    along K (pictor-tokenizer page: 1-bit and ternary {-1, 0, +1} formats
    with group 128; the page gives neither layout nor scale, so this is a
    reading). Per output row n and group of 128 consecutive k:
      m = (sum of |w| over the group, in k order, float64) / 128,
      s = m rounded to float32, then to bf16 (both to nearest even);
      1-bit: code 1 where w >= 0 (value +s), else 0 (value -s);
      2-bit: q = round_half_even(w / s) in float64 clamped to [-1, 1], q = 0
             when s = 0; code q + 1.
    For sign codes, s = mean |w| is the least-squares scale. Returns codes
    [N, K] uint8 and s [N, K/128] float32 (bf16-valued)."""
    if bits not in (1, 2):
        raise ValueError("bits must be 1 or 2")
    N, K = w.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    g = np.asarray(w, dtype=np.float32).reshape(N, K // 128, 128).astype(np.float64)
    m = np.cumsum(np.abs(g), axis=-1)[..., -1] / 128.0
    s = bf16_rne(m.astype(np.float32))
    if bits == 1:
        return (g >= 0).astype(np.uint8).reshape(N, K), s
    sd = s.astype(np.float64)[..., None]
    q = np.clip(np.rint(g / np.where(sd > 0, sd, 1.0)), -1.0, 1.0)
    q = np.where(sd > 0, q, 0.0)
    return (q + 1).astype(np.uint8).reshape(N, K), s


def dequantise_g128(codes: np.ndarray, s: np.ndarray, bits: int) -> np.ndarray:
    """w_hat [N, K] float32: 1-bit code 1 -> +s, 0 -> -s; 2-bit code
    0 -> -s, 2 -> +s, 1 and 3 -> 0 (exact in float32)."""
    N, K = codes.shape
    if bits == 1:
        v = np.where(codes == 1, 1.0, -1.0)
    else:
        v = np.select([codes == 0, codes == 2], [-1.0, 1.0], 0.0)
    return (v.reshape(N, K // 128, 128) * s[..., None].astype(np.float64)).astype(np.float32).reshape(N, K)


def pack_g128(codes: np.ndarray, bits: int) -> np.ndarray:
    """Codes [N, K] -> bytes [N, K*bits/8]: weight k at bit (k % (8/bits)) *
    bits of byte k // (8/bits), low bits first."""
    per = 8 // bits
    N, K = codes.shape
    c = codes.astype(np.uint32).reshape(N, K // per, per)
    shifts = (np.arange(per, dtype=np.uint32) * bits)[None, None, :]
    return np.bitwise_or.reduce(c << shifts, axis=-1).astype(np.uint8)


def unpack_g128(p: np.ndarray, bits: int) -> np.ndarray:
    per = 8 // bits
    N, B = p.shape
    shifts = (np.arange(per, dtype=np.uint32) * bits)[None, None, :]
    return ((p.astype(np.uint32)[..., None] >> shifts) & np.uint32((1 << bits) - 1)).astype(np.uint8).reshape(N, B * per)

