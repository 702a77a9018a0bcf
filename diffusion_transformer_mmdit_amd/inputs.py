"""Seeded synthetic inputs and random-init weights for the MMDiT denoising step.

This module draws random numbers and arranges them into the tensors the step
consumes. It computes none of the method's arithmetic, so both the CPU oracle
(through the tests) and the HIP path (through the binding) can take their
inputs from here without sharing any of the computation being checked.

Random-init recipe (no trained weights exist here):
  * every tensor has its own generator, PCG64 seeded by
    SeedSequence([42, cfg_id, block_idx, tensor_idx]);
  * linear weights and biases are N(0, 0.02^2); RMSNorm scales are
    1 + N(0, 0.02^2) so that attention logits keep an O(1) spread;
  * activations (block inputs, the conditioning vector, text embeddings,
    the pooled vector) are N(0, 1);
  * the initial latent noise is Box-Muller over a splitmix64 counter stream.

For bf16 configurations every tensor is rounded to bf16 (round to nearest,
ties to even) here, once, and both sides receive exactly those values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

GLOBAL_SEED = 42
WEIGHT_STD = 0.02


# ---------------------------------------------------------------- shapes ----
@dataclasses.dataclass(frozen=True)
class Shape:
    """Sizes of one MMDiT workload (block or whole step)."""
    hidden: int = 3072
    heads: int = 24
    head_dim: int = 128
    mlp_hidden: int = 12288
    txt_len: int = 512
    grid_h: int = 64
    grid_w: int = 64
    batch: int = 1
    axes_dim: tuple = (16, 56, 56)
    theta: float = 10000.0
    n_double: int = 19
    n_single: int = 38
    in_ch: int = 64
    txt_in_dim: int = 4096
    vec_in_dim: int = 768
    temb_dim: int = 256
    dtype: str = "bf16"          # "bf16" or "f32"
    cfg_id: int = 0              # seeds weights/inputs apart per workload

    @property
    def img_len(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def seq_len(self) -> int:
        return self.txt_len + self.img_len


# The five workloads: a tiny fp32 block, a 512^2 bf16 block, the 1024^2
# bf16 dual+single blocks, the full 1024^2 step, and the same step with
# group-quantised weights.
CFG1 = Shape(hidden=256, heads=2, mlp_hidden=1024, txt_len=16, grid_h=8,
             grid_w=8, dtype="f32", cfg_id=1, n_double=1, n_single=1,
             txt_in_dim=256, vec_in_dim=256)
CFG2 = Shape(txt_len=256, grid_h=32, grid_w=32, cfg_id=2, n_double=1,
             n_single=0)
CFG3 = Shape(txt_len=512, grid_h=64, grid_w=64, cfg_id=3, n_double=1,
             n_single=1)
CFG4 = Shape(cfg_id=4)
CFG5 = Shape(cfg_id=5)


# ------------------------------------------------------------ generators ----
def generator(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [GLOBAL_SEED] + [int(k) for k in key])))


def normal(shape, key, std=1.0, mean=0.0) -> np.ndarray:
    """float32 draw of N(mean, std^2) from its own seeded generator."""
    a = generator(*key).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return a


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """uint16 bf16 encodings of float32 values, round to nearest even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float32 array holding the bf16-rounded values of `a`."""
    return bf16_to_f32(bf16_bits(a))


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(a) if dtype == "bf16" else a


# Fixed manifests: a tensor's index in its list is its tensor_idx.
STREAM_TENSORS = ["mod_w", "mod_b", "qkv_w", "qkv_b", "proj_w", "proj_b",
                  "fc1_w", "fc1_b", "fc2_w", "fc2_b", "q_norm", "k_norm"]
SINGLE_TENSORS = ["mod_w", "mod_b", "lin1_w", "lin1_b", "lin2_w", "lin2_b",
                  "q_norm", "k_norm"]
GLOBAL_TENSORS = ["img_in_w", "img_in_b", "txt_in_w", "txt_in_b",
                  "time_in0_w", "time_in0_b", "time_in1_w", "time_in1_b",
                  "vec_in0_w", "vec_in0_b", "vec_in1_w", "vec_in1_b",
                  "final_mod_w", "final_mod_b", "final_w", "final_b"]
# block_idx values for tensors outside the blocks, kept clear of block ids
GLOBAL_BLOCK = 10_000
INPUT_BLOCK = 20_000


def _stream_shapes(s: Shape) -> Dict[str, tuple]:
    h, m, d = s.hidden, s.mlp_hidden, s.head_dim
    return {"mod_w": (6 * h, h), "mod_b": (6 * h,),
            "qkv_w": (3 * h, h), "qkv_b": (3 * h,),
            "proj_w": (h, h), "proj_b": (h,),
            "fc1_w": (m, h), "fc1_b": (m,),
            "fc2_w": (h, m), "fc2_b": (h,),
            "q_norm": (d,), "k_norm": (d,)}


def _single_shapes(s: Shape) -> Dict[str, tuple]:
    h, m, d = s.hidden, s.mlp_hidden, s.head_dim
    return {"mod_w": (3 * h, h), "mod_b": (3 * h,),
            "lin1_w": (3 * h + m, h), "lin1_b": (3 * h + m,),
            "lin2_w": (h, h + m), "lin2_b": (h,),
            "q_norm": (d,), "k_norm": (d,)}


def _global_shapes(s: Shape) -> Dict[str, tuple]:
    h = s.hidden
    return {"img_in_w": (h, s.in_ch), "img_in_b": (h,),
            "txt_in_w": (h, s.txt_in_dim), "txt_in_b": (h,),
            "time_in0_w": (h, s.temb_dim), "time_in0_b": (h,),
            "time_in1_w": (h, h), "time_in1_b": (h,),
            "vec_in0_w": (h, s.vec_in_dim), "vec_in0_b": (h,),
            "vec_in1_w": (h, h), "vec_in1_b": (h,),
            "final_mod_w": (2 * h, h), "final_mod_b": (2 * h,),
            "final_w": (s.in_ch, h), "final_b": (s.in_ch,)}


def _draw(name, shape, key, dtype):
    if name in ("q_norm", "k_norm"):
        a = normal(shape, key, std=WEIGHT_STD, mean=1.0)
    else:
        a = normal(shape, key, std=WEIGHT_STD)
    return _finish(a, dtype)


def double_block_weights(s: Shape, block_idx: int = 0) -> Dict[str, Dict[str, np.ndarray]]:
    """{'txt': {...}, 'img': {...}} float32 arrays (bf16-valued for bf16)."""
    shapes = _stream_shapes(s)
    out = {}
    for sidx, stream in enumerate(("txt", "img")):
        out[stream] = {n: _draw(n, shapes[n], (s.cfg_id, block_idx, 100 * sidx + i), s.dtype)
                       for i, n in enumerate(STREAM_TENSORS)}
    return out


def single_block_weights(s: Shape, block_idx: int = 0) -> Dict[str, np.ndarray]:
    shapes = _single_shapes(s)
    return {n: _draw(n, shapes[n], (s.cfg_id, 1000 + block_idx, i), s.dtype)
            for i, n in enumerate(SINGLE_TENSORS)}


def global_weights(s: Shape) -> Dict[str, np.ndarray]:
    shapes = _global_shapes(s)
    return {n: _draw(n, shapes[n], (s.cfg_id, GLOBAL_BLOCK, i), s.dtype)
            for i, n in enumerate(GLOBAL_TENSORS)}


GUIDANCE_TENSORS = ["guidance_in0_w", "guidance_in0_b", "guidance_in1_w", "guidance_in1_b"]
GUIDANCE_INDEX0 = 100  # tensor_idx of the first guidance tensor (clear of GLOBAL_TENSORS)


def guidance_weights(s: Shape) -> Dict[str, np.ndarray]:
    """Guidance embedder of a guidance-distilled model: temb_dim -> h -> h."""
    h = s.hidden
    shapes = {"guidance_in0_w": (h, s.temb_dim), "guidance_in0_b": (h,),
              "guidance_in1_w": (h, h), "guidance_in1_b": (h,)}
    return {n: _draw(n, shapes[n], (s.cfg_id, GLOBAL_BLOCK, GUIDANCE_INDEX0 + i), s.dtype)
            for i, n in enumerate(GUIDANCE_TENSORS)}


def zero_modulation(w: Dict) -> Dict:
    """Copy of block weights with the modulation linear set to zero."""
    if "txt" in w:
        return {k: zero_modulation(v) for k, v in w.items()}
    w = dict(w)
    w["mod_w"] = np.zeros_like(w["mod_w"])
    w["mod_b"] = np.zeros_like(w["mod_b"])
    return w


def attention_only(w: Dict) -> Dict:
    """Copy of block weights whose output minus input is the attention
    branch alone, linear in the attention output O:
      dual stream: gate2 rows of the modulation zero (rows 5h..6h of mod_w
        and mod_b), out-projection bias zero, so x_out - x_in = gate1 * O W_proj^T;
      single: the MLP columns of linear2 (h..h+m) and its bias zero, so
        x_out - x_in = gate * O W_2[:, :h]^T."""
    if "txt" in w:
        return {k: attention_only(v) for k, v in w.items()}
    w = dict(w)
    if "proj_w" in w:
        h = w["proj_w"].shape[0]
        for n in ("mod_w", "mod_b"):
            a = w[n].copy()
            a[5 * h:] = 0
            w[n] = a
        w["proj_b"] = np.zeros_like(w["proj_b"])
    else:
        h = w["lin2_w"].shape[0]
        a = w["lin2_w"].copy()
        a[:, h:] = 0
        w["lin2_w"] = a
        w["lin2_b"] = np.zeros_like(w["lin2_b"])
    return w


class LazyBlocks:
    """Sequence of block weights generated on access (one block in memory)."""

    def __init__(self, fn, s: Shape, n: int, transform=None):
        self.fn, self.s, self.n, self.transform = fn, s, n, transform

    def __len__(self):
        return self.n

    def __getitem__(self, i):
        if not 0 <= i < self.n:
            raise IndexError(i)
        w = self.fn(self.s, i)
        return self.transform(w) if self.transform else w


# ---------------------------------------------------------- activations -----
def block_inputs(s: Shape) -> Dict[str, np.ndarray]:
    """x_txt [B,Lt,h], x_img [B,Li,h], x (joint [B,L,h]) and vec [B,h]."""
    B, h = s.batch, s.hidden
    x_txt = _finish(normal((B, s.txt_len, h), (s.cfg_id, INPUT_BLOCK, 0)), s.dtype)
    x_img = _finish(normal((B, s.img_len, h), (s.cfg_id, INPUT_BLOCK, 1)), s.dtype)
    vec = _finish(normal((B, h), (s.cfg_id, INPUT_BLOCK, 2)), s.dtype)
    x = _finish(normal((B, s.seq_len, h), (s.cfg_id, INPUT_BLOCK, 3)), s.dtype)
    return {"x_txt": x_txt, "x_img": x_img, "vec": vec, "x": x}


def step_inputs(s: Shape) -> Dict[str, np.ndarray]:
    """Latent noise z [B,16,2gh,2gw] (Box-Muller), text embeddings
    T [B,Lt,4096] and pooled vector y [B,768], both N(0,1)."""
    B = s.batch
    c = s.in_ch // 4
    n = B * c * (2 * s.grid_h) * (2 * s.grid_w)
    z = box_muller(n, seed=GLOBAL_SEED + s.cfg_id).reshape(B, c, 2 * s.grid_h, 2 * s.grid_w)
    T = _finish(normal((B, s.txt_len, s.txt_in_dim), (s.cfg_id, INPUT_BLOCK, 10)), s.dtype)
    y = _finish(normal((B, s.vec_in_dim), (s.cfg_id, INPUT_BLOCK, 11)), s.dtype)
    return {"z": z, "T": T, "y": y}


# ----------------------------------------------------- Box-Muller noise ----
_M64 = np.uint64(0xFFFFFFFFFFFFFFFF)


def splitmix64(counter: np.ndarray, seed: int) -> np.ndarray:
    """splitmix64 output for each 64-bit counter value (Steele, Lea and
    Flood's SplittableRandom finaliser), stream offset by `seed`."""
    with np.errstate(over="ignore"):
        z = (counter.astype(np.uint64) + np.uint64(1)) * np.uint64(0x9E3779B97F4A7C15)
        z = z + np.uint64(seed) * np.uint64(0xD1B54A32D192ED03)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def box_muller(n: int, seed: int = GLOBAL_SEED) -> np.ndarray:
    """n standard normal float32 values: counter 2i and 2i+1 give two
    uniforms in (0,1] and [0,1) from their top 53 bits, then
    r = sqrt(-2 ln u1), outputs r cos(2 pi u2) and r sin(2 pi u2)."""
    pairs = (n + 1) // 2
    ctr = np.arange(2 * pairs, dtype=np.uint64)
    bits = splitmix64(ctr, seed) >> np.uint64(11)
    u = bits.astype(np.float64) * (1.0 / 9007199254740992.0)
    u1 = 1.0 - u[0::2]            # (0, 1]
    u2 = u[1::2]                  # [0, 1)
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * pairs, dtype=np.float64)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    return out[:n].astype(np.float32)
