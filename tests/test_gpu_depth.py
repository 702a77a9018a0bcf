"""The step at the model's full depth (19 dual + 38 single blocks, h 3072,
24 x 128 heads, MLP 12288) compared element by element with the oracle.

The weights are the seeded random-init model the benchmark times, drawn on
the GPU by the input generator (random_init); the oracle receives a float32
copy of every block as it reaches it, so it never holds more than one block
on the host. Quantised layers reach the oracle as their codes and bf16
scales and are decoded there (oracle.unpack_int4 / oracle.dequantise).

Cases:
  * 1024^2 (4096 image + 512 text tokens, bf16): the benchmarked step, and
    the same step with its residual stream held in bf16 (dims.resid);
  * the same with group-quantised weights (4-bit inner projections, 8-bit
    residual-writing layers), both the route that dequantises inside the GEMM
    tile loop and the automatic route (decoded once per launch);
  * 256 image + 64 text tokens: the same depth at a size the oracle finishes
    in seconds, dense and quantised (in-GEMM route, below 1024 rows).

Bar: rel-L2 <= 2e-2 and cosine >= 0.999 on v and on the updated latent
(pictor README, "Parity is the product": cosine >= 0.999 per stage).
"""
import dataclasses

import numpy as np
import pytest

import oracle
from diffusion_transformer_mmdit_amd import binding as bd
from diffusion_transformer_mmdit_amd import inputs as I
from tests.gpu_util import assert_parity, sync, torch

pytestmark = pytest.mark.gpu

S = I.CFG4
SMALL = dataclasses.replace(I.CFG4, txt_len=64, grid_h=16, grid_w=16)


# ------------------------------------------------- weights for the oracle ---
def lin_np(L: bd.Linear):
    """(w, b) float32 of one device Linear; quantised codes decoded by the oracle."""
    b = None if L.bias is None else L.bias.float().cpu().numpy()
    if L.fmt == bd.W_DENSE:
        return L.w.float().cpu().numpy(), b
    s = L.scales.float().cpu().numpy()
    raw = L.w.cpu().numpy()
    if L.fmt == bd.W_Q4G64:
        return oracle.dequantise(oracle.unpack_int4(raw.view(np.uint8)), s), b
    if L.fmt == bd.W_Q8G64:
        return oracle.dequantise(raw.view(np.int8), s), b
    bits = 1 if L.fmt == bd.W_Q1G128 else 2
    return oracle.dequantise_g128(oracle.unpack_g128(raw.view(np.uint8), bits), s, bits), b


def stream_np(sw: bd.StreamW):
    d = {}
    for n in ("mod", "qkv", "proj", "fc1", "fc2"):
        d[n + "_w"], d[n + "_b"] = lin_np(getattr(sw, n))
    d["q_norm"] = sw.q_norm.float().cpu().numpy()
    d["k_norm"] = sw.k_norm.float().cpu().numpy()
    return d


def double_np(w: bd.DoubleW):
    return {"img": stream_np(w.img), "txt": stream_np(w.txt)}


def single_np(w: bd.SingleW):
    d = {}
    for n in ("mod", "lin1", "lin2"):
        d[n + "_w"], d[n + "_b"] = lin_np(getattr(w, n))
    d["q_norm"] = w.q_norm.float().cpu().numpy()
    d["k_norm"] = w.k_norm.float().cpu().numpy()
    return d


def global_np(M: bd.ModelW):
    g = {}
    for n in bd.GLOBAL_LINEARS:
        key = "final" if n == "final_lin" else n
        g[key + "_w"], g[key + "_b"] = lin_np(getattr(M, n))
    return g


class Lazy:
    """Sequence view of device block weights that converts block i for the
    oracle when the oracle asks for it (one block on the host at a time)."""

    def __init__(self, blocks, conv, tag):
        self.blocks, self.conv, self.tag = blocks, conv, tag

    def __len__(self):
        return len(self.blocks)

    def __getitem__(self, i):
        if i % 8 == 0:
            print(f"  oracle {self.tag} block {i}", flush=True)
        return self.conv(self.blocks[i])


# ------------------------------------------------------------ fixtures ------
def _model(quant):
    t = torch()
    from diffusion_transformer_mmdit_amd import random_init as RI
    print(f"building the {S.n_double}+{S.n_single}-block model, quant {quant}", flush=True)
    return RI.model(S, seed=42, device=t.device("cuda:0"), quant=quant)


@pytest.fixture(scope="module")
def dense():
    M = _model(None)
    yield M
    del M


@pytest.fixture(scope="module")
def quant():
    M = _model(bd.QUANT_POLICY)
    yield M
    del M


def _inputs(s: I.Shape):
    """Latent noise (Box-Muller), text embeddings and pooled vector of shape s
    (bf16-valued), ids and the 4-step schedule, on the host."""
    z = I.box_muller(s.batch * 16 * 4 * s.grid_h * s.grid_w).reshape(s.batch, 16, 2 * s.grid_h, 2 * s.grid_w)
    X = oracle.pack_latents(z).astype(np.float32)
    rng = np.random.default_rng(4242)
    T = I.round_bf16(rng.standard_normal((s.batch, s.txt_len, s.txt_in_dim)).astype(np.float32))
    y = I.round_bf16(rng.standard_normal((s.batch, s.vec_in_dim)).astype(np.float32))
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    sig = oracle.schedule(4, s.img_len)
    return X, T, y, ids, sig


def gpu_step(s: I.Shape, M: bd.ModelW, X, T, y, ids, sigma, sigma_next, dequant_in_gemm=False,
             resid=bd.RESID_DEFAULT):
    t = torch()
    cfg = bd.make_config(s, resid=resid)
    mc = M.c()
    d = t.device("cuda:0")
    Xd = t.from_numpy(X).to(d)
    v = t.empty_like(Xd)
    Td = t.from_numpy(T).to(d).to(t.bfloat16)
    yd = t.from_numpy(y).to(d).to(t.bfloat16)
    idd = t.from_numpy(ids).to(d)
    ws = t.empty(bd.mmdit_step_workspace(cfg), dtype=t.uint8, device=d)
    print(f"GPU step {s.n_double}+{s.n_single} blocks, L {s.seq_len}, sigma {sigma:.4f} -> {sigma_next:.4f}, "
          f"dequant_in_gemm {dequant_in_gemm}, resid {resid}", flush=True)
    if dequant_in_gemm:
        bd.mmdit_step_ex(cfg, mc, Xd, v, Td, yd, idd, sigma, sigma_next, ws, dequant_in_gemm=True)
    else:
        bd.mmdit_step(cfg, mc, Xd, v, Td, yd, idd, sigma, sigma_next, ws)
    sync()
    out = Xd.cpu().numpy(), v.cpu().numpy()
    del ws
    return out


def oracle_step(s: I.Shape, M: bd.ModelW, X, T, y, ids, sigma, sigma_next):
    print(f"oracle step {len(M.dbl)}+{len(M.sgl)} blocks, L {s.seq_len}", flush=True)
    return oracle.step(global_np(M), Lazy(M.dbl, double_np, "dual"), Lazy(M.sgl, single_np, "single"), X, T, y,
                       ids, sigma, sigma_next, s.heads, s.axes_dim, s.theta)


# --------------------------------------------------------------- tests ------
@pytest.mark.timeout(600)
def test_full_depth_step_1024_matches_oracle(dense):
    # the benchmarked step: 19 + 38 blocks at 4096 image + 512 text tokens
    X, T, y, ids, sig = _inputs(S)
    Xg, vg = gpu_step(S, dense, X, T, y, ids, sig[1], sig[2])
    # the same step with the residual stream held in bf16 (76 rounded
    # residual additions instead of float32 ones)
    Xb, vb = gpu_step(S, dense, X, T, y, ids, sig[1], sig[2], resid=bd.RESID_BF16)
    Xr, vr = oracle_step(S, dense, X, T, y, ids, sig[1], sig[2])
    assert_parity(vg, vr, "bf16", "19+38 step at 1024^2: v")
    assert_parity(Xg, Xr, "bf16", "19+38 step at 1024^2: x_next")
    assert_parity(vb, vr, "bf16", "19+38 step at 1024^2, bf16 residual: v")
    assert_parity(Xb, Xr, "bf16", "19+38 step at 1024^2, bf16 residual: x_next")


@pytest.mark.timeout(600)
def test_full_depth_quantised_step_1024_matches_oracle(quant):
    # config 5 as written (dequantised inside the GEMM tile loop) and the
    # automatic route (each quantised layer decoded once per launch)
    X, T, y, ids, sig = _inputs(S)
    Xq, vq = gpu_step(S, quant, X, T, y, ids, sig[1], sig[2], dequant_in_gemm=True)
    Xa, va = gpu_step(S, quant, X, T, y, ids, sig[1], sig[2])
    Xr, vr = oracle_step(S, quant, X, T, y, ids, sig[1], sig[2])
    assert_parity(vq, vr, "bf16", "quantised 19+38 step, in-GEMM dequantisation: v")
    assert_parity(Xq, Xr, "bf16", "quantised 19+38 step, in-GEMM dequantisation: x_next")
    assert_parity(va, vr, "bf16", "quantised 19+38 step, decoded once: v")
    assert_parity(Xa, Xr, "bf16", "quantised 19+38 step, decoded once: x_next")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("sig_i", [0, 3])
def test_full_depth_step_320_tokens_matches_oracle(dense, sig_i):
    X, T, y, ids, sig = _inputs(SMALL)
    Xg, vg = gpu_step(SMALL, dense, X, T, y, ids, sig[sig_i], sig[sig_i + 1])
    Xb, vb = gpu_step(SMALL, dense, X, T, y, ids, sig[sig_i], sig[sig_i + 1], resid=bd.RESID_BF16)
    Xr, vr = oracle_step(SMALL, dense, X, T, y, ids, sig[sig_i], sig[sig_i + 1])
    assert_parity(vg, vr, "bf16", f"19+38 step at 320 tokens, sigma {sig[sig_i]:.3f}: v")
    assert_parity(Xg, Xr, "bf16", f"19+38 step at 320 tokens, sigma {sig[sig_i]:.3f}: x_next")
    assert_parity(vb, vr, "bf16", f"19+38 step at 320 tokens, sigma {sig[sig_i]:.3f}, bf16 residual: v")
    assert_parity(Xb, Xr, "bf16", f"19+38 step at 320 tokens, sigma {sig[sig_i]:.3f}, bf16 residual: x_next")


@pytest.mark.timeout(300)
def test_full_depth_quantised_step_320_tokens_matches_oracle(quant):
    X, T, y, ids, sig = _inputs(SMALL)
    Xg, vg = gpu_step(SMALL, quant, X, T, y, ids, sig[0], sig[1])
    Xr, vr = oracle_step(SMALL, quant, X, T, y, ids, sig[0], sig[1])
    assert_parity(vg, vr, "bf16", "quantised 19+38 step at 320 tokens: v")
    assert_parity(Xg, Xr, "bf16", "quantised 19+38 step at 320 tokens: x_next")
