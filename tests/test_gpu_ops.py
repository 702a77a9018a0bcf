"""GPU parity of the single-operation entry points against the oracle:
mmdit_linear_fwd on every route and weight format, and
mmdit_adaln_layernorm."""
import numpy as np
import pytest

import oracle
from diffusion_transformer_mmdit_amd import binding as bd
from diffusion_transformer_mmdit_amd import inputs as I
from tests.gpu_util import assert_parity, down, sync, torch, up

pytestmark = pytest.mark.gpu

N, K = 328, 384  # 20.5 column blocks of 16; 3 blocks of 128 along k
BITS = {"dense": 0, "q4": 4, "q8": 8, "q1": 1, "tq2": 2}


def _layer(fmt: str, seed: int = 0):
    """Device Linear in the format and the float32 weights the oracle multiplies."""
    w = I.round_bf16(I.normal((N, K), (80, seed, 0), std=0.02))
    b = I.round_bf16(I.normal((N,), (80, seed, 1), std=0.02))
    bits = BITS[fmt]
    lin = bd.Linear.from_numpy(w, b, bd.BF16, "cuda", bits)
    if bits in (4, 8):
        q, s = oracle.quantise(w, bits)
        wo = oracle.dequantise(q, s)
    elif bits in (1, 2):
        c, s = oracle.quantise_g128(w, bits)
        wo = oracle.dequantise_g128(c, s, bits)
    else:
        wo = w
    return lin, wo, b


def _x(M, seed=3):
    return I.round_bf16(I.normal((M, K), (81, seed, M)))


@pytest.mark.parametrize("fmt", list(BITS))
@pytest.mark.parametrize("M", [1, 5, 16])
def test_linear_weight_streaming_route(fmt, M):
    t = torch()
    lin, wo, b = _layer(fmt)
    x = _x(M)
    for y_f32 in (True, False):
        y = t.empty((M, N), dtype=t.float32 if y_f32 else t.bfloat16, device="cuda")
        print(f"linear stream {fmt} M={M} y_f32={y_f32}", flush=True)
        bd.mmdit_linear_fwd(lin, up(x, "bf16"), y, route=bd.ROUTE_STREAM)
        sync()
        assert_parity(down(y), oracle.linear(x, wo, b), "bf16", f"stream {fmt} M={M}")


@pytest.mark.parametrize("fmt", list(BITS))
def test_linear_tiled_and_decode_routes(fmt):
    t = torch()
    lin, wo, b = _layer(fmt, seed=1)
    for M in (17, 300):
        x = _x(M, seed=4)
        ref = oracle.linear(x, wo, b)
        routes = [bd.ROUTE_TILED, bd.ROUTE_AUTO] + ([bd.ROUTE_DECODE] if fmt != "dense" else [])
        for route in routes:
            need = bd.mmdit_linear_workspace(lin, bd.BF16, M, route)
            ws = t.empty(max(need, 16), dtype=t.uint8, device="cuda")
            y = t.empty((M, N), dtype=t.float32, device="cuda")
            print(f"linear {fmt} M={M} route {route}", flush=True)
            bd.mmdit_linear_fwd(lin, up(x, "bf16"), y, route=route, ws=ws)
            sync()
            assert_parity(down(y), ref, "bf16", f"{fmt} M={M} route {route}")


def test_linear_routes_agree_at_stream_size():
    # M = 16, 4-bit weights: the tiled GEMM and the decode route multiply the
    # same bf16 weights bf16(s q), so they agree to accumulation order; the
    # weight-streaming kernel applies the group scale to each group's float32
    # sum of q x, so it differs from them by at most the bf16 rounding of
    # s q (2^-9 relative per weight) summed over k
    t = torch()
    lin, wo, b = _layer("q4", seed=2)
    xh = _x(16, seed=5)
    x = up(xh, "bf16")
    outs = []
    for route in (bd.ROUTE_STREAM, bd.ROUTE_TILED, bd.ROUTE_DECODE):
        need = bd.mmdit_linear_workspace(lin, bd.BF16, 16, route)
        ws = t.empty(max(need, 16), dtype=t.uint8, device="cuda")
        y = t.empty((16, N), dtype=t.float32, device="cuda")
        bd.mmdit_linear_fwd(lin, x, y, route=route, ws=ws)
        sync()
        outs.append(down(y))
    scale = np.max(np.abs(outs[1]))
    assert np.max(np.abs(outs[2] - outs[1])) <= 1e-4 * scale
    bound = 2.0 ** -9 * (np.abs(xh) @ np.abs(wo).T) + 1e-5 * scale
    assert np.all(np.abs(outs[0] - outs[1]) <= bound)
    assert np.max(np.abs(outs[0] - outs[1])) > 0  # the two really differ in rounding


def test_linear_float32():
    t = torch()
    w = I.normal((N, K), (82, 0, 0), std=0.02)
    b = I.normal((N,), (82, 0, 1), std=0.02)
    lin = bd.Linear.from_numpy(w, b, bd.F32, "cuda")
    x = I.normal((37, K), (82, 0, 2))
    y = t.empty((37, N), dtype=t.float32, device="cuda")
    bd.mmdit_linear_fwd(lin, up(x, "f32"), y)
    sync()
    assert_parity(down(y), oracle.linear(x, w, b), "f32", "float32 linear")


@pytest.mark.parametrize("h,x_f32", [(3072, True), (3072, False), (1280, True)])
def test_adaln_layernorm(h, x_f32):
    t = torch()
    rows = 999
    x = I.normal((rows, h), (83, h, 0)) * np.float32(3.0) + np.float32(0.5)
    if not x_f32:
        x = I.round_bf16(x)
    mod = I.normal((2, h), (83, h, 1), std=0.3)
    y = t.empty((rows, h), dtype=t.bfloat16, device="cuda")
    bd.mmdit_adaln_layernorm(up(x, "f32" if x_f32 else "bf16"), y, up(mod, "f32"))
    sync()
    ref = oracle.modulate(x, mod[0][None, :], mod[1][None, :])
    assert_parity(down(y), ref, "bf16", f"adaLN LayerNorm h {h} x_f32 {x_f32}")


@pytest.mark.parametrize("fmt", list(BITS))
@pytest.mark.parametrize("shape", [(3072, 15360), (21504, 3072)], ids=["linear2", "linear1"])
def test_linear_weight_streaming_model_shapes(fmt, shape):
    # the weight-streaming route at the model's own layer shapes (N, K):
    # single-block linear2 (3072 x 15360, 15 k blocks per wavefront) and
    # linear1 (21504 x 3072, 3 per wavefront), one row and 16 rows
    t = torch()
    n, k = shape
    w = I.round_bf16(I.normal((n, k), (84, n, k), std=0.02))
    b = I.round_bf16(I.normal((n,), (84, n, 1), std=0.02))
    bits = BITS[fmt]
    lin = bd.Linear.from_numpy(w, b, bd.BF16, "cuda", bits)
    if bits in (4, 8):
        q, sc = oracle.quantise(w, bits)
        wo = oracle.dequantise(q, sc)
    elif bits in (1, 2):
        c, sc = oracle.quantise_g128(w, bits)
        wo = oracle.dequantise_g128(c, sc, bits)
    else:
        wo = w
    for M in (1, 16):
        x = I.round_bf16(I.normal((M, k), (85, n, M)))
        y = t.empty((M, n), dtype=t.float32, device="cuda")
        print(f"linear stream {fmt} {n}x{k} M={M}", flush=True)
        bd.mmdit_linear_fwd(lin, up(x, "bf16"), y, route=bd.ROUTE_STREAM)
        sync()
        assert_parity(down(y), oracle.linear(x, wo, b), "bf16", f"stream {fmt} {n}x{k} M={M}")
