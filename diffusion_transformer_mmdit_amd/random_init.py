"""Random-init MMDiT weights generated directly on the GPU with torch's seeded
generator (fast enough for the 11.9 B-parameter 1024^2 model). Same recipe as
the NumPy generator in inputs.py: linear weights and biases N(0, 0.02^2),
RMSNorm scales 1 + N(0, 0.02^2). Quantised layers get codes drawn uniformly
from the symmetric range and bf16 scales near 0.02 * 3 / qmax, which is the
shape quantising N(0, 0.02^2) weights produces.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import binding as bd
from .inputs import Shape

STD = 0.02


class _Gen:
    def __init__(self, seed: int, device):
        self.g = torch.Generator(device=device)
        self.g.manual_seed(seed)
        self.device = device

    def normal(self, *shape, mean=0.0, dtype=torch.bfloat16):
        t = torch.randn(*shape, generator=self.g, device=self.device, dtype=torch.float32)
        t.mul_(STD)
        if mean:
            t.add_(mean)
        return t.to(dtype)

    def randint(self, lo, hi, *shape):
        return torch.randint(lo, hi, shape, generator=self.g, device=self.device, dtype=torch.int8)

    def uniform(self, lo, hi, *shape):
        return (torch.rand(*shape, generator=self.g, device=self.device) * (hi - lo) + lo)


def _linear(G: _Gen, n: int, k: int, dtype, bits: int = 0) -> bd.Linear:
    b = G.normal(n, dtype=dtype)
    if bits == 0:
        return bd.Linear(G.normal(n, k, dtype=dtype), b)
    if bits in (1, 2):  # sign / ternary codes, groups of 128, absmean-sized scales
        codes = G.randint(0, 2 if bits == 1 else 3, n, k).to(torch.int32)
        per = 8 // bits
        c = codes.reshape(n, k // per, per)
        packed = torch.zeros(n, k // per, dtype=torch.int32, device=codes.device)
        for j in range(per):
            packed |= c[:, :, j] << (bits * j)
        scales = G.uniform(0.5 * STD, 1.0 * STD, n, k // 128).to(torch.bfloat16)
        fmt = bd.W_Q1G128 if bits == 1 else bd.W_TQ2G128
        return bd.Linear(packed.to(torch.uint8).contiguous(), b, scales, fmt, n, k)
    qmax = 7 if bits == 4 else 127
    q = G.randint(-qmax, qmax + 1, n, k)
    scales = G.uniform(2.0 * STD / qmax, 4.0 * STD / qmax, n, k // 64).to(torch.bfloat16)
    if bits == 4:
        u = q.to(torch.int16) & 0xF
        packed = (u[:, 0::2] | (u[:, 1::2] << 4)).to(torch.uint8)
        return bd.Linear(packed.contiguous(), b, scales, bd.W_Q4G64, n, k)
    return bd.Linear(q.contiguous(), b, scales, bd.W_Q8G64, n, k)


def _stream(G, s: Shape, dtype, quant) -> bd.StreamW:
    h, m, d = s.hidden, s.mlp_hidden, s.head_dim
    q = quant or {}
    return bd.StreamW(_linear(G, 6 * h, h, dtype), _linear(G, 3 * h, h, dtype, q.get("qkv", 0)),
                      _linear(G, h, h, dtype, q.get("proj", 0)), _linear(G, m, h, dtype, q.get("fc1", 0)),
                      _linear(G, h, m, dtype, q.get("fc2", 0)), G.normal(d, mean=1.0, dtype=dtype),
                      G.normal(d, mean=1.0, dtype=dtype))


def double_block(s: Shape, seed: int, device="cuda", quant: Optional[dict] = None) -> bd.DoubleW:
    G = _Gen(seed, device)
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    return bd.DoubleW(None, img=_stream(G, s, dt, quant), txt=_stream(G, s, dt, quant))


def single_block(s: Shape, seed: int, device="cuda", quant: Optional[dict] = None) -> bd.SingleW:
    G = _Gen(seed, device)
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    h, m, d = s.hidden, s.mlp_hidden, s.head_dim
    q = quant or {}
    return bd.SingleW(None, mod=_linear(G, 3 * h, h, dt), lin1=_linear(G, 3 * h + m, h, dt, q.get("lin1", 0)),
                      lin2=_linear(G, h, h + m, dt, q.get("lin2", 0)), q_norm=G.normal(d, mean=1.0, dtype=dt),
                      k_norm=G.normal(d, mean=1.0, dtype=dt))


def model(s: Shape, seed: int, device="cuda", quant: Optional[dict] = None, guidance: bool = False) -> bd.ModelW:
    G = _Gen(seed, device)
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    h = s.hidden
    lin = {"img_in": _linear(G, h, s.in_ch, dt), "txt_in": _linear(G, h, s.txt_in_dim, dt),
           "time_in0": _linear(G, h, s.temb_dim, dt), "time_in1": _linear(G, h, h, dt),
           "vec_in0": _linear(G, h, s.vec_in_dim, dt), "vec_in1": _linear(G, h, h, dt),
           "final_mod": _linear(G, 2 * h, h, dt), "final_lin": _linear(G, s.in_ch, h, dt)}
    if guidance:  # guidance embedder of a guidance-distilled model
        lin["guidance_in0"] = _linear(G, h, s.temb_dim, dt)
        lin["guidance_in1"] = _linear(G, h, h, dt)
    dbl = [double_block(s, seed * 1000 + 1 + i, device, quant) for i in range(s.n_double)]
    sgl = [single_block(s, seed * 1000 + 500 + i, device, quant) for i in range(s.n_single)]
    return bd.ModelW(None, dbl, sgl, linears=lin)
