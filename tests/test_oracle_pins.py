"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks one oracle function against something other than its own
formula: the pages' printed constants, closed forms, invariants, brute
force on tiny inputs, or torch library routines in float64 (tests/torch_ref).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from diffusion_transformer_mmdit_amd import inputs as I
from tests import torch_ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")
PAGES = json.load(open(os.path.join(GOLD, "pages_constants.json")))


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def tiny_shape(**kw):
    base = dict(hidden=256, heads=2, head_dim=128, mlp_hidden=512, txt_len=5, grid_h=3,
                grid_w=4, dtype="f32", cfg_id=77, txt_in_dim=96, vec_in_dim=48, temb_dim=256,
                in_ch=64)
    base.update(kw)
    return I.Shape(**base)


# ------------------------------------------------------------- packing -----
def test_pack_bijection_bit_exact_on_raw_bits():
    # random 32-bit patterns, NaN payloads included, travel as uint32
    rng = np.random.default_rng(1)
    z = rng.integers(0, 2**32, size=(2, 16, 128, 128), dtype=np.uint64).astype(np.uint32)
    z[0, 0, 0, :8] = np.array([0x7FC00001, 0xFFC12345, 0x7F800000, 0xFF800000, 0, 0x80000000, 1, 0x7FFFFFFF],
                              dtype=np.uint32)
    X = oracle.pack_latents(z)
    assert X.shape == (2, 4096, 64)
    back = oracle.unpack_latents(X, 16, 128, 128)
    assert back.dtype == np.uint32 and np.array_equal(back, z)
    # every input element lands exactly once: a permutation
    assert np.array_equal(np.sort(X.ravel()), np.sort(z.ravel()))


def test_pack_explicit_index_formula_brute_force():
    rng = np.random.default_rng(2)
    B, C, H, W = 1, 3, 6, 4
    z = rng.standard_normal((B, C, H, W)).astype(np.float32)
    X = oracle.pack_latents(z)
    Wp = W // 2
    for c in range(C):
        for yy in range(H):
            for xx in range(W):
                tok = (yy // 2) * Wp + (xx // 2)
                ch = c * 4 + (yy % 2) * 2 + (xx % 2)
                assert X[0, tok, ch] == z[0, c, yy, xx]


def test_pack_sizes_match_page_calculator():
    r = PAGES["resolution_1024"]
    lat = r["latent_hw"]
    z = np.zeros((1, 16, lat, lat), np.float32)
    X = oracle.pack_latents(z)
    assert r["width"] // 8 == lat and r["width"] // 16 == r["grid_hw"]
    assert X.shape == (1, r["image_tokens"], PAGES["patch_channels"]["value"])


# ------------------------------------------------------------------ ids ----
def test_ids_closed_form():
    ids = oracle.make_ids(3, 5, 4)
    assert ids.dtype == np.int32 and ids.shape == (4 + 15, 3)
    assert np.all(ids[:4] == 0)
    for k in range(15):
        assert tuple(ids[4 + k]) == (0, k // 5, k % 5)
    ids2 = oracle.make_ids(2, 2, 0, frame=3)
    assert np.array_equal(ids2, np.array([[3, 0, 0], [3, 0, 1], [3, 1, 0], [3, 1, 1]], np.int32))


# ----------------------------------------------------------------- RoPE ----
def test_rope_axes_sum_to_head_dim():
    a = PAGES["rope_axes"]
    assert sum(a["axes"]) == a["head_dim"]
    cos, sin = oracle.rope_table(oracle.make_ids(4, 4, 2))
    assert cos.shape == (18, a["head_dim"] // 2)


def test_rope_closed_form_angles():
    ids = oracle.make_ids(64, 64, 0)
    cos, sin = oracle.rope_table(ids)
    rows = ids[:, 1].astype(np.float64)
    cols = ids[:, 2].astype(np.float64)
    # axis-1 pair 0 (table column 8) has omega = 1, so its angle is the row
    assert np.allclose(cos[:, 8], np.cos(rows), atol=1e-7)
    assert np.allclose(sin[:, 8], np.sin(rows), atol=1e-7)
    # axis-2 pair 5 (column 8 + 28 + 5) has omega = 10000^(-10/56)
    om = 10000.0 ** (-10.0 / 56.0)
    assert np.allclose(sin[:, 41], np.sin(cols * om), atol=1e-7)
    # axis 0 uses the frame coordinate: all zero here
    assert np.all(cos[:, :8] == 1.0) and np.all(sin[:, :8] == 0.0)


def test_rope_norm_preservation():
    rng = np.random.default_rng(3)
    ids = oracle.make_ids(8, 8, 3, frame=2)
    cos, sin = oracle.rope_table(ids)
    x = rng.standard_normal((2, 67, 128))
    y = oracle.apply_rope(x, cos, sin)
    pair_x = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    pair_y = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    assert np.max(np.abs(pair_y - pair_x) / np.maximum(pair_x, 1e-12)) < 1e-6
    nx = np.linalg.norm(x, axis=-1)
    ny = np.linalg.norm(y, axis=-1)
    assert np.max(np.abs(ny - nx) / nx) < 1e-6


def test_rope_identity_at_zero_ids_bit_exact():
    x = np.random.default_rng(4).standard_normal((3, 10, 128)).astype(np.float32)
    cos, sin = oracle.rope_table(np.zeros((10, 3), np.int32))
    y = oracle.apply_rope(x, cos, sin)
    assert np.array_equal(y, x)


def test_rope_relative_position_property():
    rng = np.random.default_rng(5)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    p = np.array([[1, 7, 40], [0, 3, 11]], np.int32)
    cos, sin = oracle.rope_table(p)
    rq = oracle.apply_rope(q[None], cos[0:1].astype(np.float64), sin[0:1].astype(np.float64))[0]
    rk = oracle.apply_rope(k[None], cos[1:2].astype(np.float64), sin[1:2].astype(np.float64))[0]
    diff = (p[0] - p[1])[None]
    c2, s2 = oracle.rope_table(diff)
    rd = oracle.apply_rope(q[None], c2.astype(np.float64), s2.astype(np.float64))[0]
    assert abs(np.dot(rq, rk) - np.dot(rd, k)) < 1e-5


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(6)
    ids = oracle.make_ids(5, 7, 2, frame=1)
    x = rng.standard_normal((2, 3, ids.shape[0], 128))
    cos, sin = oracle.rope_table(ids)
    ours = oracle.apply_rope(x, cos.astype(np.float64), sin.astype(np.float64))
    ref = torch_ref.rope_complex(torch.from_numpy(x), ids).numpy()
    # tables are float32 in the oracle: ~6e-8 relative per element
    assert np.max(np.abs(ours - ref)) < 1e-6


# ---------------------------------------------------------------- norms ----
def test_layer_norm_moments_and_library():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((4, 3072)) * 3.0 + 1.5)
    y = oracle.layer_norm(x)
    var = x.var(axis=-1)
    assert np.max(np.abs(y.mean(-1))) < 1e-12
    assert np.allclose(y.var(-1), var / (var + 1e-6), rtol=1e-10)
    ref = F.layer_norm(torch.from_numpy(x), (3072,), eps=1e-6).numpy()
    assert np.max(np.abs(y - ref)) < 1e-12


def test_modulate_special_cases():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, 6, 64))
    z = np.zeros((1, 1, 64))
    assert np.array_equal(oracle.modulate(x, z, z), oracle.layer_norm(x))
    shift = rng.standard_normal((1, 1, 64))
    out = oracle.modulate(x, shift, -np.ones((1, 1, 64)))
    assert np.array_equal(out, np.broadcast_to(shift, out.shape))


def test_rms_norm_unit_scale_and_library():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 128)) * 4.0
    y = oracle.rms_norm(x, np.ones(128))
    assert np.max(np.abs(np.sqrt((y * y).mean(-1)) - 1.0)) < 1e-5
    g = 1.0 + 0.1 * rng.standard_normal(128)
    ref = F.rms_norm(torch.from_numpy(x), (128,), torch.from_numpy(g), eps=1e-6).numpy()
    assert np.max(np.abs(oracle.rms_norm(x, g) - ref)) < 1e-12


# ------------------------------------------------------------ pointwise ----
def test_gelu_tanh():
    x = np.linspace(-8, 8, 2001)
    y = oracle.gelu_tanh(x)
    ref = F.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    assert np.max(np.abs(y - ref)) < 1e-14
    assert oracle.gelu_tanh(np.zeros(1))[0] == 0.0
    assert np.max(np.abs(y - oracle.gelu_tanh(-x) - x)) < 1e-12
    # float64 evaluation of the written-out definition at a few points
    for v in (-2.5, -0.3, 0.7, 3.1):
        e = 0.5 * v * (1 + math.tanh(math.sqrt(2 / math.pi) * (v + 0.044715 * v ** 3)))
        assert abs(oracle.gelu_tanh(np.array([v]))[0] - e) < 1e-14


def test_silu_and_linear():
    x = np.linspace(-6, 6, 101)
    assert np.max(np.abs(oracle.silu(x) - F.silu(torch.from_numpy(x)).numpy())) < 1e-14
    rng = np.random.default_rng(10)
    a, w, b = rng.standard_normal((3, 7)), rng.standard_normal((5, 7)), rng.standard_normal(5)
    ref = F.linear(torch.from_numpy(a), torch.from_numpy(w), torch.from_numpy(b)).numpy()
    assert np.max(np.abs(oracle.linear(a, w, b) - ref)) < 1e-12


# ------------------------------------------------------------ attention ----
def _brute_attention(q, k, v):
    B, H, L, d = q.shape
    out = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            for i in range(L):
                s = [sum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) / math.sqrt(d) for j in range(L)]
                mx = max(s)
                e = [math.exp(x - mx) for x in s]
                tot = sum(e)
                for c in range(d):
                    out[b, h, i, c] = sum(e[j] * v[b, h, j, c] for j in range(L)) / tot
    return out


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((1, 2, 9, 128)) * 1.5 for _ in range(3))
    ref = _brute_attention(q, k, v)
    got = oracle.attention(q.astype(np.float32), k.astype(np.float32), v.astype(np.float32))
    assert rel_l2(got, ref) < 1e-6


def test_attention_identical_keys_gives_mean_v():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 3, 20, 128)).astype(np.float32)
    k = np.broadcast_to(rng.standard_normal((1, 3, 1, 128)), (1, 3, 20, 128)).astype(np.float32)
    v = rng.standard_normal((1, 3, 20, 128)).astype(np.float32)
    o = oracle.attention(q, k, v)
    assert np.max(np.abs(o - v.mean(axis=2, keepdims=True))) < 1e-6


def test_attention_single_token_and_library():
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((2, 2, 1, 128)) for _ in range(3))
    assert np.array_equal(oracle.attention(q, k, v), v)
    q, k, v = (rng.standard_normal((2, 3, 33, 128)) for _ in range(3))
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(a) for a in (q, k, v))).numpy()
    assert rel_l2(oracle.attention(q, k, v), ref) < 1e-12


# --------------------------------------------------------------- blocks ----
def _tiny_block_case(s, seed=0):
    w = I.double_block_weights(s, seed)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len, frame=1)
    ids[: s.txt_len, 1] = np.arange(s.txt_len)    # distinct text ids exercise RoPE on text rows too
    return w, x, ids


def _f64(d):
    if isinstance(d, dict):
        return {k: _f64(v) for k, v in d.items()}
    return np.asarray(d, np.float64)


def test_double_block_matches_torch_composition():
    s = tiny_shape()
    w, x, ids = _tiny_block_case(s)
    img, txt = oracle.double_block(_f64(w), _f64(x["x_img"]), _f64(x["x_txt"]), _f64(x["vec"]), ids, s.heads)
    rimg, rtxt = torch_ref.double_block(w, x["x_img"], x["x_txt"], x["vec"], ids, s.heads)
    # the oracle's RoPE table is float32 (about 6e-8 relative per entry)
    assert rel_l2(img, rimg) < 1e-6 and rel_l2(txt, rtxt) < 1e-6


def test_single_block_matches_torch_composition():
    s = tiny_shape()
    w = I.single_block_weights(s, 0)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len, frame=1)
    got = oracle.single_block(_f64(w), _f64(x["x"]), _f64(x["vec"]), ids, s.heads)
    ref = torch_ref.single_block(w, x["x"], x["vec"], ids, s.heads)
    assert rel_l2(got, ref) < 1e-6


def test_double_block_gate_zero_identity_bit_exact():
    s = tiny_shape()
    w, x, ids = _tiny_block_case(s)
    w0 = I.zero_modulation(w)
    img, txt = oracle.double_block(w0, x["x_img"], x["x_txt"], x["vec"], ids, s.heads)
    assert np.array_equal(img, x["x_img"]) and np.array_equal(txt, x["x_txt"])
    w1 = I.zero_modulation(I.single_block_weights(s, 0))
    assert np.array_equal(oracle.single_block(w1, x["x"], x["vec"], ids, s.heads), x["x"])


def test_blocks_uniform_id_shift_invariance():
    s = tiny_shape()
    w, x, ids = _tiny_block_case(s)
    img, txt = oracle.double_block(_f64(w), _f64(x["x_img"]), _f64(x["x_txt"]), _f64(x["vec"]), ids, s.heads)
    img2, txt2 = oracle.double_block(_f64(w), _f64(x["x_img"]), _f64(x["x_txt"]), _f64(x["vec"]),
                                     ids + np.array([3, 5, 9], np.int32), s.heads)
    assert rel_l2(img2, img) < 1e-5 and rel_l2(txt2, txt) < 1e-5
    # a non-uniform change (swap row/col) must change the output
    img3, _ = oracle.double_block(_f64(w), _f64(x["x_img"]), _f64(x["x_txt"]), _f64(x["vec"]),
                                  ids[:, [0, 2, 1]].copy(), s.heads)
    assert rel_l2(img3, img) > 1e-4


def test_blocks_permutation_equivariance():
    s = tiny_shape()
    w, x, _ = _tiny_block_case(s)
    ids = np.zeros((s.seq_len, 3), np.int32)
    perm = np.random.default_rng(14).permutation(s.img_len)
    img, txt = oracle.double_block(_f64(w), _f64(x["x_img"]), _f64(x["x_txt"]), _f64(x["vec"]), ids, s.heads)
    img_p, txt_p = oracle.double_block(_f64(w), _f64(x["x_img"][:, perm]), _f64(x["x_txt"]),
                                       _f64(x["vec"]), ids, s.heads)
    assert rel_l2(img_p, img[:, perm]) < 1e-12 and rel_l2(txt_p, txt) < 1e-12
    ws = I.single_block_weights(s, 0)
    perm2 = np.random.default_rng(15).permutation(s.seq_len)
    y = oracle.single_block(_f64(ws), _f64(x["x"]), _f64(x["vec"]), ids, s.heads)
    y_p = oracle.single_block(_f64(ws), _f64(x["x"][:, perm2]), _f64(x["vec"]), ids, s.heads)
    assert rel_l2(y_p, y[:, perm2]) < 1e-12


def test_double_block_image_only_reduces_to_prenorm_block():
    # Lt = 0 and ids = 0: a pre-LN adaLN transformer block on the image
    # tokens, composed directly from torch routines.
    s = tiny_shape(txt_len=0)
    w, x, _ = _tiny_block_case(s)
    ids = np.zeros((s.img_len, 3), np.int32)
    img, txt = oracle.double_block(_f64(w), _f64(x["x_img"]), _f64(x["x_txt"]), _f64(x["vec"]), ids, s.heads)
    assert txt.shape == (1, 0, s.hidden)
    T = torch_ref.t
    wi = {n: T(a) for n, a in w["img"].items()}
    xi = T(x["x_img"])
    m = F.linear(F.silu(T(x["vec"])), wi["mod_w"], wi["mod_b"])[:, None].chunk(6, -1)
    hN = F.layer_norm(xi, (s.hidden,), eps=1e-6) * (1 + m[1]) + m[0]
    q, k, v = F.linear(hN, wi["qkv_w"], wi["qkv_b"]).chunk(3, -1)
    H = s.heads

    def hd(a):
        return a.reshape(1, -1, H, 128).transpose(1, 2)
    q = F.rms_norm(hd(q), (128,), wi["q_norm"], eps=1e-6)
    k = F.rms_norm(hd(k), (128,), wi["k_norm"], eps=1e-6)
    o = F.scaled_dot_product_attention(q, k, hd(v)).transpose(1, 2).reshape(1, -1, s.hidden)
    xi = xi + m[2] * F.linear(o, wi["proj_w"], wi["proj_b"])
    h2 = F.layer_norm(xi, (s.hidden,), eps=1e-6) * (1 + m[4]) + m[3]
    xi = xi + m[5] * F.linear(F.gelu(F.linear(h2, wi["fc1_w"], wi["fc1_b"]), approximate="tanh"),
                              wi["fc2_w"], wi["fc2_b"])
    assert rel_l2(img, xi.numpy()) < 1e-12


def test_dual_block_with_shared_weights_is_joint_sequence_block():
    # Same weights in both streams and ids = 0: the dual block acts on the
    # concatenated [txt; img] sequence as one stream would.
    s = tiny_shape()
    w, x, _ = _tiny_block_case(s)
    shared = {"txt": w["img"], "img": w["img"]}
    ids = np.zeros((s.seq_len, 3), np.int32)
    img, txt = oracle.double_block(_f64(shared), _f64(x["x_img"]), _f64(x["x_txt"]), _f64(x["vec"]), ids, s.heads)
    s0 = tiny_shape(txt_len=0, grid_h=1, grid_w=s.seq_len)
    joint = np.concatenate([x["x_txt"], x["x_img"]], axis=1)
    ji, _ = oracle.double_block(_f64(shared), _f64(joint), np.zeros((1, 0, s.hidden)), _f64(x["vec"]),
                                np.zeros((s0.seq_len, 3), np.int32), s.heads)
    assert rel_l2(np.concatenate([txt, img], 1), ji) < 1e-12


# ---------------------------------------------------- conditioning, step ---
def test_timestep_embedding_closed_forms():
    e = oracle.timestep_embedding(0.0, 256)
    assert np.array_equal(e[:128], np.ones(128, np.float32)) and np.array_equal(e[128:], np.zeros(128, np.float32))
    e = oracle.timestep_embedding(0.37, 256, dtype=np.float64)
    assert abs(e[0] - math.cos(370.0)) < 1e-12 and abs(e[128] - math.sin(370.0)) < 1e-12
    assert abs(e[127] - math.cos(370.0 * math.exp(-math.log(1e4) * 127 / 128))) < 1e-12
    assert np.max(np.abs(e - torch_ref.temb(0.37).numpy())) < 1e-12


def test_step_matches_torch_composition():
    s = tiny_shape(txt_len=3, grid_h=2, grid_w=3)
    g = I.global_weights(s)
    dbl = [I.double_block_weights(s, i) for i in range(2)]
    sgl = [I.single_block_weights(s, i) for i in range(2)]
    inp = I.step_inputs(s)
    X = oracle.pack_latents(inp["z"])
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    sig = oracle.schedule(4, s.img_len)
    Xn, v = oracle.step(_f64(g), [_f64(w) for w in dbl], [_f64(w) for w in sgl], _f64(X), _f64(inp["T"]),
                        _f64(inp["y"]), ids, sig[1], sig[2], s.heads)
    rX, rv = torch_ref.step(g, dbl, sgl, X, inp["T"], inp["y"], ids, sig[1], sig[2], s.heads)
    assert rel_l2(v, rv) < 1e-6 and rel_l2(Xn, rX) < 1e-6


def test_step_gate_zero_reduces_to_final_layer():
    s = tiny_shape(txt_len=3, grid_h=2, grid_w=3)
    g = I.global_weights(s)
    dbl = [I.zero_modulation(I.double_block_weights(s, i)) for i in range(2)]
    sgl = [I.zero_modulation(I.single_block_weights(s, i)) for i in range(2)]
    inp = I.step_inputs(s)
    X = oracle.pack_latents(inp["z"])
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    _, v = oracle.step(g, dbl, sgl, X, inp["T"], inp["y"], ids, 1.0, 0.9, s.heads)
    img = oracle.linear(X, g["img_in_w"], g["img_in_b"])
    vec = oracle.conditioning_vec(g, 1.0, inp["y"])
    assert np.array_equal(v, oracle.final_layer(g, img, vec))


def _ctx_case():
    s = tiny_shape(txt_len=3, grid_h=2, grid_w=3)
    g = I.global_weights(s)
    dbl = [I.double_block_weights(s, i) for i in range(2)]
    sgl = [I.single_block_weights(s, i) for i in range(2)]
    inp = I.step_inputs(s)
    X = oracle.pack_latents(inp["z"])
    Xc = np.random.default_rng(21).standard_normal((1, 5, X.shape[2])).astype(np.float32)
    ids = np.concatenate([oracle.make_ids(s.grid_h, s.grid_w, s.txt_len),
                          np.array([[1, r, c] for r, c in [(0, 0), (0, 1), (1, 0), (1, 1), (2, 0)]], np.int32)])
    return s, g, dbl, sgl, inp, X, Xc, ids


def test_step_context_tokens_are_a_set():
    # Reference-image tokens reach the generated rows only through joint
    # attention, which sees them as a set: permuting them together with their
    # ids leaves v unchanged; dropping them changes v.
    s, g, dbl, sgl, inp, X, Xc, ids = _ctx_case()
    args = (_f64(g), [_f64(w) for w in dbl], [_f64(w) for w in sgl], _f64(X), _f64(inp["T"]), _f64(inp["y"]))
    Xn, v = oracle.step(*args, ids, 0.8, 0.6, s.heads, Xc=_f64(Xc))
    assert v.shape == X.shape and Xn.shape == X.shape
    perm = np.random.default_rng(22).permutation(Xc.shape[1])
    Lf = s.txt_len + s.img_len
    ids_p = np.concatenate([ids[:Lf], ids[Lf:][perm]])
    _, vp = oracle.step(*args, ids_p, 0.8, 0.6, s.heads, Xc=_f64(Xc[:, perm]))
    assert rel_l2(vp, v) < 1e-12
    _, v0 = oracle.step(*args, ids[:Lf], 0.8, 0.6, s.heads)
    assert rel_l2(v0, v) > 1e-3


def test_step_context_gate_zero_takes_generated_rows():
    # With every modulation zero the blocks are the identity, so v is the
    # final layer of the generated tokens' input projection whatever the
    # context tokens hold: the update uses exactly the first Lg image rows.
    s, g, dbl, sgl, inp, X, Xc, ids = _ctx_case()
    dbl = [I.zero_modulation(w) for w in dbl]
    sgl = [I.zero_modulation(w) for w in sgl]
    _, v = oracle.step(g, dbl, sgl, X, inp["T"], inp["y"], ids, 1.0, 0.9, s.heads, Xc=Xc)
    vec = oracle.conditioning_vec(g, 1.0, inp["y"])
    assert np.array_equal(v, oracle.final_layer(g, oracle.linear(X, g["img_in_w"], g["img_in_b"]), vec))


def test_guidance_embedding_is_a_second_timestep_map():
    # With the guidance map's weights equal to the timestep map's and
    # guidance == sigma, the guidance term equals the timestep term: vec gains
    # exactly the timestep part (the guidance value is embedded like sigma).
    s = tiny_shape(txt_len=3, grid_h=2, grid_w=3)
    g = _f64(I.global_weights(s))
    y = _f64(I.step_inputs(s)["y"])
    vec = oracle.conditioning_vec(g, 0.7, y)
    gg = dict(g, guidance_in0_w=g["time_in0_w"], guidance_in0_b=g["time_in0_b"],
              guidance_in1_w=g["time_in1_w"], guidance_in1_b=g["time_in1_b"])
    vt = oracle.conditioning_vec(dict(g, vec_in1_w=0 * g["vec_in1_w"], vec_in1_b=0 * g["vec_in1_b"]), 0.7, y)
    assert rel_l2(oracle.conditioning_vec(gg, 0.7, y, guidance=0.7) - vec, vt) < 1e-12
    # a zero output layer adds nothing; a different value changes vec
    gw = dict(g, **{k: _f64(v) for k, v in I.guidance_weights(s).items()})
    z = dict(gw, guidance_in1_w=0 * gw["guidance_in1_w"], guidance_in1_b=0 * gw["guidance_in1_b"])
    assert np.array_equal(oracle.conditioning_vec(z, 0.7, y, guidance=4.0), vec)
    assert rel_l2(oracle.conditioning_vec(gw, 0.7, y, guidance=4.0),
                  oracle.conditioning_vec(gw, 0.7, y, guidance=3.5)) > 1e-4
    with pytest.raises(ValueError):
        oracle.conditioning_vec(gw, 0.7, y)


# --------------------------------------------------------- step caching ---
def test_rel_l1_hand_worked():
    # |1-2| + |2-2| + |-3+1| = 3 over |2| + |2| + |-1| = 5
    assert oracle.rel_l1(np.array([1.0, 2.0, -3.0]), np.array([2.0, 2.0, -1.0])) == 0.6
    assert oracle.rel_l1(np.zeros(3), np.zeros(3)) == 0.0
    assert oracle.rel_l1(np.ones(3), np.zeros(3)) == np.inf


def test_cache_decide_hand_traced():
    # threshold 0.5, every later step changes by 0.25: run, reuse (0.25),
    # run (0.5 reaches the threshold, sum reset), reuse (0.25), run (0.5)
    valid, acc, got = False, 0.0, []
    for _ in range(5):
        run, acc = oracle.cache_decide(valid, acc, 0.25, 0.5)
        valid = True
        got.append((run, acc))
    assert got == [(True, 0.0), (False, 0.25), (True, 0.0), (False, 0.25), (True, 0.0)]
    # threshold 0: every step runs the blocks
    assert all(oracle.cache_decide(True, a, r, 0.0)[0] for a in (0.0, 3.0) for r in (0.0, 1.0))


def _cache_case(**kw):
    s = tiny_shape(txt_len=3, grid_h=2, grid_w=3, **kw)
    g = _f64(I.global_weights(s))
    dbl = [_f64(I.double_block_weights(s, i)) for i in range(2)]
    sgl = [_f64(I.single_block_weights(s, i)) for i in range(2)]
    inp = _f64(I.step_inputs(s))
    X = oracle.pack_latents(inp["z"])
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    return s, g, dbl, sgl, inp, X, ids


def test_step_cached_threshold_zero_is_the_plain_step():
    s, g, dbl, sgl, inp, X, ids = _cache_case()
    sig = oracle.schedule(3, s.img_len)
    st = oracle.new_cache_state()
    for i in range(3):
        Xn, v, run, rel = oracle.step_cached(g, dbl, sgl, X, inp["T"], inp["y"], ids, sig[i], sig[i + 1],
                                             s.heads, st, 0.0)
        Xr, vr = oracle.step(g, dbl, sgl, X, inp["T"], inp["y"], ids, sig[i], sig[i + 1], s.heads)
        assert run and np.array_equal(v, vr) and np.array_equal(Xn, Xr)
        assert (rel == 0.0) if i == 0 else (rel > 0.0)
        X = Xn


def test_step_cached_repeat_reuses_the_residual():
    # The same latent and sigma twice: the indicator does not move (rel 0),
    # the second step reuses the residual, and img0 + (img - img0) gives the
    # first step's v up to rounding. Context tokens ride in the residual.
    s, g, dbl, sgl, inp, X, Xc, ids = _ctx_case()
    g, dbl, sgl, X, Xc = _f64(g), [_f64(w) for w in dbl], [_f64(w) for w in sgl], _f64(X), _f64(Xc)
    st = oracle.new_cache_state()
    out = [oracle.step_cached(g, dbl, sgl, X, inp["T"], inp["y"], ids, 1.0, 0.9, s.heads, st, 1e-9, Xc=Xc)
           for _ in range(2)]
    assert out[0][2] and not out[1][2] and out[1][3] == 0.0
    assert rel_l2(out[1][1], out[0][1]) < 1e-13
    _, vr = oracle.step(g, dbl, sgl, X, inp["T"], inp["y"], ids, 1.0, 0.9, s.heads, Xc=Xc)
    assert np.array_equal(out[0][1], vr)


def test_step_cached_identity_blocks_skip_equals_compute():
    # With every modulation zero the blocks add nothing: the residual is
    # exactly zero, so a reused step is exactly the plain step at the new
    # latent and sigma (the residual is added to this step's tokens).
    s, g, dbl, sgl, inp, X, ids = _cache_case()
    dbl = [I.zero_modulation(w) for w in dbl]
    sgl = [I.zero_modulation(w) for w in sgl]
    st = oracle.new_cache_state()
    X1, _, run1, _ = oracle.step_cached(g, dbl, sgl, X, inp["T"], inp["y"], ids, 1.0, 0.6, s.heads, st, np.inf)
    X2, v2, run2, rel = oracle.step_cached(g, dbl, sgl, X1, inp["T"], inp["y"], ids, 0.6, 0.2, s.heads, st, np.inf)
    assert run1 and not run2 and rel > 0.0
    Xr, vr = oracle.step(g, dbl, sgl, X1, inp["T"], inp["y"], ids, 0.6, 0.2, s.heads)
    assert np.array_equal(v2, vr) and np.array_equal(X2, Xr)


def test_step_cached_indicator_reads_the_first_dual_block_image_input():
    # rel depends on the latent, sigma and the first dual block's image
    # modulation only: new text or a different second block leave it as is.
    s, g, dbl, sgl, inp, X, ids = _cache_case()
    def rels(T, blocks):
        st = oracle.new_cache_state()
        out = []
        for Xi, a, b in ((X, 1.0, 0.7), (1.1 * X, 0.7, 0.3)):
            out.append(oracle.step_cached(g, blocks, sgl, Xi, T, inp["y"], ids, a, b, s.heads, st, 0.0)[3])
        return out
    base = rels(inp["T"], dbl)
    assert base[0] == 0.0 and base[1] > 0.0
    assert rels(2.0 * inp["T"] + 1.0, dbl) == base
    assert rels(inp["T"], [dbl[0], dbl[0]]) == base
    d0 = {"txt": dbl[0]["txt"], "img": dict(dbl[0]["img"], mod_b=dbl[0]["img"]["mod_b"] + 0.5)}
    assert rels(inp["T"], [d0, dbl[1]])[1] != base[1]
    with pytest.raises(ValueError):
        oracle.step_cached(g, [], sgl, X, inp["T"], inp["y"], ids, 1.0, 0.7, s.heads, oracle.new_cache_state(), 0.0)


# ------------------------------------------------------- schedule, Euler ---
def test_schedule_page_invariants():
    sh = PAGES["shift"]
    for n in (1, 2, 4, 7, 50):
        for li in (256, 1024, 4096):
            sig = oracle.schedule(n, li, sh["base_shift"], sh["max_shift"])
            assert sig[0] == 1.0 and sig[-1] == 0.0
            assert np.all(np.diff(sig) < 0), "strictly decreasing, 0 inversions"
    mu = oracle.mu_for_tokens(4096)
    lim = PAGES["time_shift_limit"]
    assert abs(float(oracle.time_shift(mu, 1.0 - 1e-12)) - lim["value"]) < lim["tol"]
    assert float(oracle.time_shift(mu, 1.0)) == 1.0


def test_schedule_closed_forms():
    assert oracle.mu_for_tokens(4096) == pytest.approx(1.15, abs=1e-15)
    assert oracle.mu_for_tokens(256) == pytest.approx(0.5, abs=1e-15)
    # t = 1/2 gives sigma = e^mu / (e^mu + 1) = logistic(mu)
    sig = oracle.schedule(4, 4096)
    assert abs(sig[2] - 1.0 / (1.0 + math.exp(-1.15))) < 1e-15
    # mu = 0 (no shift) gives sigma_i = t_i
    assert np.allclose(oracle.schedule(8, 4096, shift=False), np.linspace(1, 0, 9), atol=1e-15)
    anchor = json.load(open(os.path.join(GOLD, "schedule_anchor.json")))
    assert np.allclose(oracle.schedule(4, 4096), anchor["n4_li4096"], rtol=0, atol=1e-15)
    term = oracle.schedule(4, 4096, sigma_terminal=PAGES["sigma_terminal"]["value"])
    assert abs(term[-2] - 0.02) < 1e-15 and term[0] == 1.0 and np.all(np.diff(term) < 0)


def test_euler_recovers_endpoint_for_constant_velocity():
    rng = np.random.default_rng(16)
    x0 = rng.standard_normal((1, 40, 64))
    eps = rng.standard_normal((1, 40, 64))
    for sig in (oracle.schedule(4, 4096), oracle.schedule(9, 700), oracle.schedule(5, 4096, sigma_terminal=0.02)):
        X = eps.copy()
        for i in range(len(sig) - 1):
            X = oracle.euler_update(X, eps - x0, sig[i], sig[i + 1])
        assert np.max(np.abs(X - x0)) < 1e-12


# ------------------------------------------------------------- quantiser ---
@pytest.mark.parametrize("bits", [4, 8])
def test_quantiser_error_bound_and_grid(bits):
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((33, 256)) * 0.02).astype(np.float32)
    w[3, 64:128] = 0.0
    q, s = oracle.quantise(w, bits)
    qmax = 7 if bits == 4 else 127
    assert q.dtype == np.int8 and np.all(np.abs(q) <= qmax)
    assert s.shape == (33, 4) and s[3, 1] == 0.0 and np.all(q[3, 64:128] == 0)
    # s is a bf16 value
    assert np.all((s.view(np.uint32) & 0xFFFF) == 0)
    wh = oracle.dequantise(q, s)
    bound = np.repeat(s, 64, axis=1) / 2
    assert np.all(np.abs(wh - w) <= bound * (1 + 1e-6))
    # a weight already on a grid (bf16 scale, codes reaching qmax in every
    # group) round-trips exactly
    qg = rng.integers(-qmax, qmax + 1, size=(9, 128)).astype(np.int8)
    qg[:, 5] = qmax
    qg[:, 64 + 9] = -qmax
    sg = I.round_bf16(np.abs(rng.standard_normal((9, 2))).astype(np.float32) * 1e-3)
    q2, s2 = oracle.quantise(oracle.dequantise(qg, sg), bits)
    assert np.array_equal(q2, qg) and np.array_equal(s2, sg)
    # the largest magnitude of a non-zero group reaches qmax or qmax-1
    assert np.all(np.abs(q).reshape(33, 4, 64).max(-1)[s > 0] >= qmax - 1)


def test_int4_packing_round_trip():
    q = np.random.default_rng(18).integers(-7, 8, size=(5, 128)).astype(np.int8)
    p = oracle.pack_int4(q)
    assert p.shape == (5, 64) and p.dtype == np.uint8
    assert np.array_equal(oracle.unpack_int4(p), q)
    assert p[0, 0] & 0xF == (int(q[0, 0]) & 0xF)      # low nibble holds the even k


def test_quantised_gemm_equals_dense_on_dequantised():
    rng = np.random.default_rng(19)
    w = (rng.standard_normal((48, 192)) * 0.02).astype(np.float32)
    x = rng.standard_normal((7, 192)).astype(np.float32)
    q, s = oracle.quantise(w, 4)
    wh = oracle.dequantise(q, s)
    y = oracle.linear(x.astype(np.float64), wh.astype(np.float64), None)
    ref = x.astype(np.float64) @ (q.astype(np.float64) * np.repeat(s, 64, axis=1)).T
    assert np.max(np.abs(y - ref)) < 1e-12


def test_g128_hand_worked_row():
    # one group: w = [0.5, -0.25, 0, 1, 0 ...]; sum |w| = 1.75, m = 7/512
    # (exact in bf16). 1-bit: signs with w >= 0 -> 1: byte 0 = 0b11111101.
    # 2-bit: w/s = 36.6, -18.3, 0, 73.1 -> q = 1, -1, 0, 1 -> codes 2, 0, 1, 2
    # -> byte 0 = 2 | 0 << 2 | 1 << 4 | 2 << 6 = 0x92; zeros -> code 1 -> 0x55.
    w = np.zeros((1, 128), np.float32)
    w[0, :4] = [0.5, -0.25, 0.0, 1.0]
    for bits, b0, rest in ((1, 0xFD, 0xFF), (2, 0x92, 0x55)):
        c, sc = oracle.quantise_g128(w, bits)
        assert sc[0, 0] == 7.0 / 512.0
        p = oracle.pack_g128(c, bits)
        assert p.shape == (1, 128 * bits // 8) and p[0, 0] == b0 and np.all(p[0, 1:] == rest)
    wh = oracle.dequantise_g128(oracle.quantise_g128(w, 2)[0], np.array([[7.0 / 512.0]], np.float32), 2)
    assert wh[0, :4].tolist() == [7.0 / 512.0, -7.0 / 512.0, 0.0, 7.0 / 512.0]


def test_g128_scale_is_least_squares_for_sign_codes():
    from scipy.optimize import minimize_scalar
    rng = np.random.default_rng(23)
    w = (rng.standard_normal((6, 256)) * 0.02).astype(np.float32)
    c, sc = oracle.quantise_g128(w, 1)
    for n in range(6):
        for gi in range(2):
            g = w[n, 128 * gi:128 * (gi + 1)].astype(np.float64)
            sg = np.where(g >= 0, 1.0, -1.0)
            best = minimize_scalar(lambda t: float(np.sum((g - t * sg) ** 2)), bounds=(0.0, 1.0), method="bounded",
                                   options={"xatol": 1e-12}).x
            assert abs(sc[n, gi] - best) <= 2.0 ** -8 * best   # bf16 rounding of the minimiser
    assert np.array_equal(c, (w >= 0).astype(np.uint8))


def test_g128_ternary_codes_are_nearest_levels():
    rng = np.random.default_rng(24)
    w = (rng.standard_normal((5, 384)) * 0.02).astype(np.float32)
    w[2, 128:256] = 0.0
    c, sc = oracle.quantise_g128(w, 2)
    assert set(np.unique(c)) <= {0, 1, 2} and sc[2, 1] == 0.0 and np.all(c[2, 128:256] == 1)
    s_full = np.repeat(sc, 128, axis=1).astype(np.float64)
    levels = np.array([-1.0, 0.0, 1.0])
    for n in range(5):
        for k in range(384):
            if s_full[n, k] == 0:
                continue
            d = np.abs(w[n, k] / s_full[n, k] - levels)
            want = 1 if abs(abs(w[n, k] / s_full[n, k]) - 0.5) < 1e-12 else int(np.argmin(d))
            assert c[n, k] == want
    # absmean: the scale is within bf16 rounding of the mean |w| of the group
    m = np.abs(w.astype(np.float64)).reshape(5, 3, 128).mean(-1)
    assert np.all(np.abs(sc - m) <= 2.0 ** -8 * m + 1e-30)


def test_g128_packing_round_trip():
    rng = np.random.default_rng(25)
    for bits in (1, 2):
        codes = rng.integers(0, 1 << bits, size=(4, 256)).astype(np.uint8)
        p = oracle.pack_g128(codes, bits)
        assert p.dtype == np.uint8 and p.shape == (4, 256 * bits // 8)
        assert np.array_equal(oracle.unpack_g128(p, bits), codes)
    # code 3 decodes to 0 like code 1
    assert oracle.dequantise_g128(np.array([[3] * 128], np.uint8), np.array([[0.5]], np.float32), 2).max() == 0.0


# ------------------------------------------------------------- inputs ------
def test_box_muller_moments_page_bounds():
    bm = PAGES["box_muller"]
    z = I.box_muller(16 * 128 * 128)
    assert abs(float(z.mean())) < bm["abs_mean_lt"]
    assert abs(float(z.var()) - 1.0) < bm["abs_var_minus_one_lt"]
    # tighter than the page's bound at this size (about 2e-3 expected)
    assert abs(float(z.mean())) < 0.01 and abs(float(z.var()) - 1.0) < 0.01
    assert np.array_equal(z, I.box_muller(16 * 128 * 128)), "seeded and repeatable"


def test_bf16_rounding_is_round_to_nearest_even():
    vals = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -2.5, 3.0e-3], np.float32)
    r = I.round_bf16(vals)
    t = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(r, t)


def test_oracle_bf16_rne_equals_an_exact_cast():
    # oracle.bf16_rne against torch's float32 -> bfloat16 conversion (round to
    # nearest, ties to even): ties in both directions, the largest finite
    # values, subnormals, signed zeros and random bit patterns
    rng = np.random.default_rng(26)
    special = np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-9, -(1.0 + 2**-8), 3.0e-3, 0.0, -0.0,
                        1e-40, -1e-40, 3.3895e38, -3.3895e38, 2**-126, 65504.0], np.float32)
    bits = rng.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    rand = bits.view(np.float32)
    rand = rand[np.isfinite(rand) & (np.abs(rand) < 3.38e38)]
    for vals in (special, rand):
        got = oracle.bf16_rne(vals)
        want = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
