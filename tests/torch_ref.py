"""Second, independent CPU statement of the MMDiT blocks built from torch's
library routines in float64 (F.layer_norm, F.rms_norm, F.linear,
F.scaled_dot_product_attention, F.gelu(approximate="tanh"), F.silu and
complex-number rotation for RoPE). Test-only: it pins the NumPy oracle with
primitives the oracle does not use. It is never used against the GPU.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

D = torch.float64


def t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def rope_complex(x, ids, axes_dim=(16, 56, 56), theta=10000.0):
    """Rotate pairs (2k, 2k+1) as complex numbers x_2k + i x_2k+1 times
    exp(i * angle); angles per axis block, in axis order."""
    ids = torch.as_tensor(np.asarray(ids), dtype=D)
    angs = []
    for a, da in enumerate(axes_dim):
        j = torch.arange(da // 2, dtype=D)
        angs.append(ids[:, a:a + 1] * torch.pow(torch.tensor(theta, dtype=D), -2.0 * j / da)[None])
    ang = torch.cat(angs, dim=1)                       # [L, d/2]
    rot = torch.polar(torch.ones_like(ang), ang)       # e^{i ang}
    xc = torch.view_as_complex(x.reshape(*x.shape[:-1], -1, 2).contiguous())
    return torch.view_as_real(xc * rot).reshape(x.shape)


def modulate(x, shift, scale, eps=1e-6):
    return (1 + scale) * F.layer_norm(x, (x.shape[-1],), eps=eps) + shift


def heads(x, H):
    B, L, hd = x.shape
    return x.reshape(B, L, H, hd // H).transpose(1, 2)


def merge(x):
    B, H, L, d = x.shape
    return x.transpose(1, 2).reshape(B, L, H * d)


def double_block(w, x_img, x_txt, vec, ids, H):
    xs = {"txt": t(x_txt), "img": t(x_img)}
    vec = t(vec)
    mods, q, k, v = {}, {}, {}, {}
    for s in ("txt", "img"):
        ws = {n: t(a) for n, a in w[s].items()}
        mods[s] = F.linear(F.silu(vec), ws["mod_w"], ws["mod_b"])[:, None, :].chunk(6, dim=-1)
        qkv = F.linear(modulate(xs[s], mods[s][0], mods[s][1]), ws["qkv_w"], ws["qkv_b"])
        qq, kk, vv = qkv.chunk(3, dim=-1)
        d = qq.shape[-1] // H
        q[s] = F.rms_norm(heads(qq, H), (d,), ws["q_norm"], eps=1e-6)
        k[s] = F.rms_norm(heads(kk, H), (d,), ws["k_norm"], eps=1e-6)
        v[s] = heads(vv, H)
    Q = rope_complex(torch.cat([q["txt"], q["img"]], 2), ids)
    K = rope_complex(torch.cat([k["txt"], k["img"]], 2), ids)
    V = torch.cat([v["txt"], v["img"]], 2)
    O = merge(F.scaled_dot_product_attention(Q, K, V))
    Lt = xs["txt"].shape[1]
    parts = {"txt": O[:, :Lt], "img": O[:, Lt:]}
    out = {}
    for s in ("txt", "img"):
        ws = {n: t(a) for n, a in w[s].items()}
        _, _, g1, sh2, sc2, g2 = mods[s]
        x = xs[s] + g1 * F.linear(parts[s], ws["proj_w"], ws["proj_b"])
        hid = F.gelu(F.linear(modulate(x, sh2, sc2), ws["fc1_w"], ws["fc1_b"]), approximate="tanh")
        out[s] = x + g2 * F.linear(hid, ws["fc2_w"], ws["fc2_b"])
    return out["img"].numpy(), out["txt"].numpy()


def single_block(w, x, vec, ids, H):
    ws = {n: t(a) for n, a in w.items()}
    x = t(x)
    sh, sc, g = F.linear(F.silu(t(vec)), ws["mod_w"], ws["mod_b"])[:, None, :].chunk(3, dim=-1)
    hd = x.shape[-1]
    y = F.linear(modulate(x, sh, sc), ws["lin1_w"], ws["lin1_b"])
    qq, kk, vv, r = torch.split(y, [hd, hd, hd, y.shape[-1] - 3 * hd], dim=-1)
    d = hd // H
    Q = rope_complex(F.rms_norm(heads(qq, H), (d,), ws["q_norm"], eps=1e-6), ids)
    K = rope_complex(F.rms_norm(heads(kk, H), (d,), ws["k_norm"], eps=1e-6), ids)
    O = merge(F.scaled_dot_product_attention(Q, K, heads(vv, H)))
    cat = torch.cat([O, F.gelu(r, approximate="tanh")], dim=-1)
    return (x + g * F.linear(cat, ws["lin2_w"], ws["lin2_b"])).numpy()


def temb(sigma, dim=256):
    half = dim // 2
    freqs = torch.exp(-math.log(10000.0) * torch.arange(half, dtype=D) / half)
    a = 1000.0 * sigma * freqs
    return torch.cat([torch.cos(a), torch.sin(a)])


def step(g, dbl, sgl, X, T, y, ids, sigma, sigma_next, H):
    gw = {n: t(a) for n, a in g.items()}
    img = F.linear(t(X), gw["img_in_w"], gw["img_in_b"])
    txt = F.linear(t(T), gw["txt_in_w"], gw["txt_in_b"])
    B = img.shape[0]
    te = temb(sigma, gw["time_in0_w"].shape[1])[None].expand(B, -1)
    vec = F.linear(F.silu(F.linear(te, gw["time_in0_w"], gw["time_in0_b"])), gw["time_in1_w"], gw["time_in1_b"])
    vec = vec + F.linear(F.silu(F.linear(t(y), gw["vec_in0_w"], gw["vec_in0_b"])), gw["vec_in1_w"], gw["vec_in1_b"])
    img, txt = img.numpy(), txt.numpy()
    vnp = vec.numpy()
    for w in dbl:
        img, txt = double_block(w, img, txt, vnp, ids, H)
    x = np.concatenate([txt, img], axis=1)
    for w in sgl:
        x = single_block(w, x, vnp, ids, H)
    im = t(x[:, T.shape[1]:])
    sh, sc = F.linear(F.silu(vec), gw["final_mod_w"], gw["final_mod_b"])[:, None, :].chunk(2, dim=-1)
    v = F.linear(modulate(im, sh, sc), gw["final_w"], gw["final_b"])
    return (t(X) + (sigma_next - sigma) * v).numpy(), v.numpy()
