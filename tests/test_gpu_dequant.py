"""GPU decoding of quantised weights (mmdit_dequantise) against the oracle,
bit for bit on the bf16 encodings.

Codes and scales are drawn directly (not through the quantiser), so every
code the layouts can hold appears: int4 nibbles -8..7, int8 -128..127,
ternary codes 0..3 (1 and 3 both mean 0), and zero scales (signed zeros for
the sub-byte formats, whose -s is -0.0). Shapes include row counts whose
32-weight runs do not fill the last wavefront (66 runs for 33 x 64)."""
import numpy as np
import pytest

import oracle
from diffusion_transformer_mmdit_amd import binding as bd
from diffusion_transformer_mmdit_amd import inputs as I
from tests.gpu_util import sync, torch

pytestmark = pytest.mark.gpu


def _scales(rng, shape):
    s = np.exp2(rng.uniform(-20, 4, size=shape)).astype(np.float32)
    s[rng.random(shape) < 0.1] = 0.0
    return I.round_bf16(s)


def _decode(packed, scales, fmt, n, k):
    t = torch()
    dev = t.device("cuda:0")
    w = t.from_numpy(np.ascontiguousarray(packed).view(np.uint8)).to(dev)
    sc = t.from_numpy(I.bf16_bits(scales).view(np.int16)).to(dev)
    out = t.full((n, k), float("nan"), dtype=t.bfloat16, device=dev)
    print(f"dequantise fmt {fmt} [{n}, {k}]", flush=True)
    bd.mmdit_dequantise(w, sc, fmt, n, k, out)
    sync()
    return out.view(t.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,k", [(33, 64), (300, 320), (2, 3072)])
@pytest.mark.parametrize("bits", [4, 8])
def test_dequantise_int_codes_bit_exact(n, k, bits):
    rng = np.random.default_rng(1000 * bits + n)
    lo, hi = (-8, 8) if bits == 4 else (-128, 128)
    q = rng.integers(lo, hi, size=(n, k)).astype(np.int8)
    s = _scales(rng, (n, k // 64))
    packed = oracle.pack_int4(q) if bits == 4 else q
    got = _decode(packed, s, bd.W_Q4G64 if bits == 4 else bd.W_Q8G64, n, k)
    # q * s is exact in float32 (at most 8 + 8 significant bits); one rounding to bf16
    want = I.bf16_bits(oracle.dequantise(q, s))
    assert np.array_equal(got, want), f"{np.sum(got != want)} of {got.size} weights differ"


@pytest.mark.parametrize("n,k", [(33, 128), (257, 384), (2, 3072)])
@pytest.mark.parametrize("bits", [1, 2])
def test_dequantise_sub_byte_codes_bit_exact(n, k, bits):
    rng = np.random.default_rng(100 * bits + n)
    codes = rng.integers(0, 2 if bits == 1 else 4, size=(n, k)).astype(np.uint8)
    s = _scales(rng, (n, k // 128))
    got = _decode(oracle.pack_g128(codes, bits), s, bd.W_Q1G128 if bits == 1 else bd.W_TQ2G128, n, k)
    want = I.bf16_bits(oracle.dequantise_g128(codes, s, bits))
    assert np.array_equal(got, want), f"{np.sum(got != want)} of {got.size} weights differ"
