"""mmdit_step_noalloc (the step on the library's own device scratch) against
mmdit_step with a caller workspace, through the C ABI: two calls in a row
on one GPU, the second with a smaller input (the scratch keeps the first
call's contents)."""
import dataclasses

import numpy as np
import pytest

from diffusion_transformer_mmdit_amd import binding as bd
from diffusion_transformer_mmdit_amd import inputs as I
from tests.gpu_util import assert_parity, sync, torch

pytestmark = pytest.mark.gpu

BIG = dataclasses.replace(I.CFG4, txt_len=256, grid_h=32, grid_w=32, n_double=2, n_single=2, cfg_id=71)
SMALL = dataclasses.replace(BIG, txt_len=40, grid_h=12, grid_w=14)


def _inputs(s, dev):
    t = torch()
    g = t.Generator(device=dev)
    g.manual_seed(71 + s.seq_len)
    X = t.randn((s.batch, s.img_len, s.in_ch), generator=g, device=dev)
    T = t.randn((s.batch, s.txt_len, s.txt_in_dim), generator=g, device=dev).to(t.bfloat16)
    y = t.randn((s.batch, s.vec_in_dim), generator=g, device=dev).to(t.bfloat16)
    ids = t.from_numpy(bd.mmdit_make_ids(s.grid_h, s.grid_w, s.txt_len)).to(dev)
    return X, T, y, ids


def test_noalloc_step_matches_workspace_step_twice():
    t = torch()
    from diffusion_transformer_mmdit_amd import random_init as RI
    dev = t.device("cuda:0")
    M = RI.model(BIG, seed=71, device=dev)
    mc = M.c()
    for s in (BIG, SMALL):
        cfg = bd.make_config(s)
        # dense weights: the exact size leaves out room for decoded layers
        need = bd.mmdit_step_workspace_ex(cfg, mc)
        assert need <= bd.NOALLOC_SCRATCH_BYTES
        X, T, y, ids = _inputs(s, dev)
        sig = bd.mmdit_schedule(4, s.img_len)
        Xa, Xb = X.clone(), X.clone()
        va, vb = t.empty_like(X), t.empty_like(X)
        ws = t.empty(need, dtype=t.uint8, device=dev)
        print(f"noalloc step: L {s.seq_len}, workspace {need / 2**20:.1f} MiB", flush=True)
        bd.mmdit_step(cfg, mc, Xa, va, T, y, ids, sig[1], sig[2], ws)
        bd.mmdit_step_noalloc(cfg, mc, Xb, vb, T, y, ids, sig[1], sig[2])
        sync()
        got_v, ref_v = vb.cpu().numpy(), va.cpu().numpy()
        got_x, ref_x = Xb.cpu().numpy(), Xa.cpu().numpy()
        print(f"  bit-identical: v {np.array_equal(got_v, ref_v)}, x {np.array_equal(got_x, ref_x)}", flush=True)
        assert_parity(got_v, ref_v, "bf16", f"noalloc vs workspace step, L {s.seq_len}: v")
        assert_parity(got_x, ref_x, "bf16", f"noalloc vs workspace step, L {s.seq_len}: x_next")
        del ws
