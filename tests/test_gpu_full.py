"""The step at its full size (1024^2: 19 dual + 38 single blocks, h 3072,
4096 image + 512 text tokens, bf16), on the benchmark's seeded random-init
weights. The oracle cannot run 57 blocks over 4608 tokens within a test's
time, so these check properties that hold at any size, each against
something the oracle does compute:
  * with every block's modulation zero the blocks are the identity
    (adaLN gates are zero), so v is the oracle's final layer applied to the
    oracle's input projection of the latent;
  * the step is bit-deterministic and its update is x + (sigma' - sigma) v;
  * a cached step repeated on the same latent and sigma reuses the block
    residual (relative change exactly 0) and returns the same v.
"""
import numpy as np
import pytest

import oracle
from diffusion_transformer_mmdit_amd import binding as bd
from diffusion_transformer_mmdit_amd import inputs as I
from tests.gpu_util import assert_parity, rel_l2, sync, torch

pytestmark = pytest.mark.gpu

S = I.CFG4


@pytest.fixture(scope="module")
def full():
    t = torch()
    from diffusion_transformer_mmdit_amd import random_init as RI
    dev = t.device("cuda:0")
    print(f"building the full model: {S.n_double}+{S.n_single} blocks, h {S.hidden}", flush=True)
    M = RI.model(S, seed=42, device=dev)
    cfg = bd.make_config(S)
    z = I.box_muller(S.batch * 16 * 4 * S.grid_h * S.grid_w).reshape(S.batch, 16, 2 * S.grid_h, 2 * S.grid_w)
    X = t.empty((S.batch, S.img_len, S.in_ch), dtype=t.float32, device=dev)
    bd.mmdit_pack_latents(t.from_numpy(z).to(dev), X)
    g = t.Generator(device=dev)
    g.manual_seed(7)
    T = t.randn((S.batch, S.txt_len, S.txt_in_dim), generator=g, device=dev).to(t.bfloat16)
    y = t.randn((S.batch, S.vec_in_dim), generator=g, device=dev).to(t.bfloat16)
    ids = t.from_numpy(bd.mmdit_make_ids(S.grid_h, S.grid_w, S.txt_len)).to(dev)
    ws = t.empty(bd.mmdit_step_workspace(cfg), dtype=t.uint8, device=dev)
    sync()
    yield dict(M=M, cfg=cfg, X=X, T=T, y=y, ids=ids, ws=ws, sig=bd.mmdit_schedule(4, S.img_len))
    del M, ws


def _step(f, mc, sig_i=1, X=None):
    t = torch()
    Xr = (f["X"] if X is None else X).clone()
    v = t.empty_like(Xr)
    print(f"full step sigma {f['sig'][sig_i]:.4f} -> {f['sig'][sig_i + 1]:.4f}", flush=True)
    bd.mmdit_step(f["cfg"], mc, Xr, v, f["T"], f["y"], f["ids"], f["sig"][sig_i], f["sig"][sig_i + 1], f["ws"])
    sync()
    return Xr, v


def test_full_step_is_deterministic_and_an_euler_update(full):
    mc = full["M"].c()
    X1, v1 = _step(full, mc)
    X2, v2 = _step(full, mc)
    assert bool(torch().equal(X1, X2)) and bool(torch().equal(v1, v2)), "reruns differ"
    x0 = full["X"].cpu().numpy().astype(np.float64)
    x1 = X1.cpu().numpy()
    v = v1.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(x1)) and np.all(np.isfinite(v))
    d = full["sig"][2] - full["sig"][1]
    dv = np.float64(np.float32(d)) * v
    want = x0 + dv
    # one rounding of the sum, plus the product's own if it is rounded first
    tol = np.spacing(np.abs(x1)).astype(np.float64) + 0.5 * np.spacing(np.abs(dv).astype(np.float32)).astype(np.float64)
    err = np.abs(x1.astype(np.float64) - want)
    print(f"Euler update: max error / tolerance {np.max(err / tol):.3f}", flush=True)
    assert np.all(err <= tol)


def _f32(lin):
    return lin.w.float().cpu().numpy(), lin.bias.float().cpu().numpy()


def test_full_step_with_zero_modulation_is_the_final_layer_of_the_input(full):
    t = torch()
    M = full["M"]
    h = S.hidden
    zw = t.zeros((6 * h, h), dtype=t.bfloat16, device="cuda")
    zb = t.zeros((6 * h,), dtype=t.bfloat16, device="cuda")

    def zero_mod(n):
        return bd.Linear(zw[:n], zb[:n])

    dbl = [bd.DoubleW(None, img=bd.StreamW(zero_mod(6 * h), d.img.qkv, d.img.proj, d.img.fc1, d.img.fc2,
                                           d.img.q_norm, d.img.k_norm),
                      txt=bd.StreamW(zero_mod(6 * h), d.txt.qkv, d.txt.proj, d.txt.fc1, d.txt.fc2,
                                     d.txt.q_norm, d.txt.k_norm)) for d in M.dbl]
    sgl = [bd.SingleW(None, mod=zero_mod(3 * h), lin1=w.lin1, lin2=w.lin2, q_norm=w.q_norm, k_norm=w.k_norm)
           for w in M.sgl]
    Mz = bd.ModelW(None, dbl, sgl, linears={n: getattr(M, n) for n in bd.GLOBAL_LINEARS})
    _, v = _step(full, Mz.c())
    # oracle: conditioning, input projection of the (bf16-staged) latent, final layer
    g = {}
    for n in ("img_in", "time_in0", "time_in1", "vec_in0", "vec_in1", "final_mod"):
        g[n + "_w"], g[n + "_b"] = _f32(getattr(M, n))
    g["final_w"], g["final_b"] = _f32(M.final_lin)
    X = full["X"].to(t.bfloat16).float().cpu().numpy()
    yv = full["y"].float().cpu().numpy()
    vec = oracle.conditioning_vec(g, full["sig"][1], yv, temb_dim=S.temb_dim)
    img = oracle.linear(X, g["img_in_w"], g["img_in_b"])
    vr = oracle.final_layer(g, img, vec)
    assert_parity(v.cpu().numpy(), vr, "bf16", "full step, zero modulation: v")


def test_full_step_cache_repeat_reuses_the_residual(full):
    t = torch()
    mc = full["M"].c()
    cache = bd.StepCache(full["cfg"])
    vs = []
    for k in range(2):
        Xr = full["X"].clone()
        v = t.empty_like(Xr)
        print(f"full cached step {k}", flush=True)
        bd.mmdit_step_ex(full["cfg"], mc, Xr, v, full["T"], full["y"], full["ids"], full["sig"][1], full["sig"][2],
                         full["ws"], cache=cache, cache_threshold=1e-9)
        sync()
        vs.append(v.cpu().numpy())
        assert cache.ran_blocks == (k == 0)
    assert cache.rel == 0.0
    r = rel_l2(vs[1], vs[0])
    print(f"reused step v rel_l2 {r:.2e}", flush=True)
    assert r < 1e-5
