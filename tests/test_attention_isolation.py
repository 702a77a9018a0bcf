"""CPU check of the attention-isolating construction the GPU tests use
(inputs.attention_only with the block input scaled by 2^-6): a relative
error planted in the oracle's attention output shows up at about its full
size in the block's output-minus-input, so the 2e-2 parity bar on that
difference catches an attention error of a few percent."""
import dataclasses

import numpy as np
import pytest

import oracle
import oracle.mmdit as om
from diffusion_transformer_mmdit_amd import inputs as I

S = dataclasses.replace(I.CFG2, hidden=1024, heads=8, mlp_hidden=4096, txt_len=64, grid_h=16, grid_w=16,
                        dtype="f32", cfg_id=61)


def _small(x):
    return {k: (v * np.float32(2.0 ** -6) if k != "vec" else v) for k, v in x.items()}


def _noisy_attention(eps, seed=0):
    rng = np.random.default_rng(seed)
    clean = om.attention

    def f(q, k, v):
        o = clean(q, k, v)
        return o * (1 + eps * rng.standard_normal(o.shape)).astype(o.dtype)
    return f


def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("eps", [0.05, 0.02])
def test_planted_attention_error_shows_at_full_size(monkeypatch, eps):
    x = _small(I.block_inputs(S))
    ids = oracle.make_ids(S.grid_h, S.grid_w, S.txt_len)
    wd = I.attention_only(I.double_block_weights(S, 0))
    ws = I.attention_only(I.single_block_weights(S, 0))
    ri, rt = oracle.double_block(wd, x["x_img"], x["x_txt"], x["vec"], ids, S.heads)
    rs = oracle.single_block(ws, x["x"], x["vec"], ids, S.heads)
    monkeypatch.setattr(om, "attention", _noisy_attention(eps))
    ni, nt = oracle.double_block(wd, x["x_img"], x["x_txt"], x["vec"], ids, S.heads)
    ns = oracle.single_block(ws, x["x"], x["vec"], ids, S.heads)
    for got, ref, x0, what in ((ni, ri, x["x_img"], "dual img"), (nt, rt, x["x_txt"], "dual txt"),
                               (ns, rs, x["x"], "single")):
        r = _rel(got - x0, ref - x0)
        print(f"{what}: planted {eps:.2f} -> difference moves by {r:.4f}")
        assert 0.8 * eps <= r <= 1.2 * eps, (what, r)


def test_isolated_difference_is_the_attention_branch():
    # with the construction, out - in equals gate1 * O W_proj^T computed from
    # the oracle's own pieces (dual image stream)
    x = _small(I.block_inputs(S))
    ids = oracle.make_ids(S.grid_h, S.grid_w, S.txt_len)
    w = I.attention_only(I.double_block_weights(S, 0))
    seen = {}
    clean = om.attention

    def keep(q, k, v):
        seen["o"] = clean(q, k, v)
        return seen["o"]
    om_attention = om.attention
    try:
        om.attention = keep
        ri, _ = oracle.double_block(w, x["x_img"], x["x_txt"], x["vec"], ids, S.heads)
    finally:
        om.attention = om_attention
    O = om._merge(seen["o"])[:, S.txt_len:]
    g1 = om._chunks(oracle.linear(oracle.silu(x["vec"]), w["img"]["mod_w"], w["img"]["mod_b"]), 6)[2]
    want = g1 * oracle.linear(O, w["img"]["proj_w"], None)
    assert _rel(ri - x["x_img"], want) < 1e-5
