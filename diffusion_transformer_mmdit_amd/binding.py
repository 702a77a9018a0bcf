"""Thin ctypes binding of libmmdit.so (C ABI in include/mmdit.h).

Functions carry the C names and only marshal arguments: torch tensors become
device pointers, the current torch stream becomes the hipStream_t, non-zero
statuses become MMDiTError. Every computation happens in the library's HIP
kernels. There is no fallback: if libmmdit.so has not been built, lib() raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Dict, List, Optional, Sequence

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmmdit.so")
_lib = None

F32, BF16 = 0, 1
RESID_DEFAULT, RESID_F32, RESID_BF16 = 0, 1, 2
W_DENSE, W_Q4G64, W_Q8G64, W_Q1G128, W_TQ2G128 = 0, 1, 2, 3, 4
PC_GEMM, PC_ATTN, PC_LN, PC_QKNORM, PC_GEMV, PC_GEMM_LIN1, PC_GEMM_RES, PC_DEQUANT = 1, 2, 3, 4, 5, 6, 7, 8
PC_GEMM_QKV, PC_GEMM_FC1, PC_STREAM = 9, 10, 11
ROUTE_AUTO, ROUTE_TILED, ROUTE_DECODE, ROUTE_STREAM = 0, 1, 2, 3


class MMDiTError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().mmdit_last_error().decode(errors="replace")
        st = lib().mmdit_status_str(status).decode()
        super().__init__(f"{where}: status {status} ({st}): {msg}")


# ------------------------------------------------------------------ structs --
class mmdit_dims(C.Structure):
    _fields_ = [("batch", C.c_int32), ("hidden", C.c_int32), ("heads", C.c_int32),
                ("head_dim", C.c_int32), ("mlp_hidden", C.c_int32), ("txt_len", C.c_int32),
                ("img_len", C.c_int32), ("axes_dim", C.c_int32 * 3), ("theta", C.c_double),
                ("ln_eps", C.c_float), ("rms_eps", C.c_float), ("act_dtype", C.c_int32), ("resid", C.c_int32)]


class mmdit_linear(C.Structure):
    _fields_ = [("w", C.c_void_p), ("scales", C.c_void_p), ("bias", C.c_void_p),
                ("fmt", C.c_int32), ("n_out", C.c_int32), ("k_in", C.c_int32)]


class mmdit_stream_w(C.Structure):
    _fields_ = [("mod", mmdit_linear), ("qkv", mmdit_linear), ("proj", mmdit_linear),
                ("fc1", mmdit_linear), ("fc2", mmdit_linear), ("q_norm", C.c_void_p),
                ("k_norm", C.c_void_p)]


class mmdit_double_w(C.Structure):
    _fields_ = [("img", mmdit_stream_w), ("txt", mmdit_stream_w)]


class mmdit_single_w(C.Structure):
    _fields_ = [("mod", mmdit_linear), ("lin1", mmdit_linear), ("lin2", mmdit_linear),
                ("q_norm", C.c_void_p), ("k_norm", C.c_void_p)]


class mmdit_config(C.Structure):
    _fields_ = [("dims", mmdit_dims), ("n_double", C.c_int32), ("n_single", C.c_int32),
                ("in_ch", C.c_int32), ("txt_in_dim", C.c_int32), ("vec_in_dim", C.c_int32),
                ("temb_dim", C.c_int32)]


class mmdit_model_w(C.Structure):
    _fields_ = [("img_in", mmdit_linear), ("txt_in", mmdit_linear), ("time_in0", mmdit_linear),
                ("time_in1", mmdit_linear), ("vec_in0", mmdit_linear), ("vec_in1", mmdit_linear),
                ("final_mod", mmdit_linear), ("final_lin", mmdit_linear),
                ("dbl", C.POINTER(mmdit_double_w)), ("sgl", C.POINTER(mmdit_single_w)),
                ("guidance_in0", mmdit_linear), ("guidance_in1", mmdit_linear)]


class mmdit_step_cache(C.Structure):
    _fields_ = [("buf", C.c_void_p), ("bytes", C.c_size_t), ("valid", C.c_int32), ("ran_blocks", C.c_int32),
                ("acc", C.c_double), ("rel", C.c_double)]


class mmdit_step_opts(C.Structure):
    _fields_ = [("ctx_packed", C.c_void_p), ("ctx_len", C.c_int32), ("has_guidance", C.c_int32),
                ("guidance", C.c_double), ("cache", C.POINTER(mmdit_step_cache)), ("cache_threshold", C.c_double),
                ("dequant", C.c_int32), ("cache_on_device", C.c_int32), ("mods", C.c_void_p),
                ("mods_count", C.c_int32), ("mods_index", C.c_int32)]


# Every function the header declares, with its ctypes signature.
_P = C.c_void_p
_SIGS = {
    "mmdit_double_block_workspace": (C.c_int, [C.POINTER(mmdit_dims), C.POINTER(C.c_size_t)]),
    "mmdit_single_block_workspace": (C.c_int, [C.POINTER(mmdit_dims), C.POINTER(C.c_size_t)]),
    "mmdit_step_workspace": (C.c_int, [C.POINTER(mmdit_config), C.POINTER(C.c_size_t)]),
    "mmdit_step_cache_bytes": (C.c_int, [C.POINTER(mmdit_config), C.POINTER(C.c_size_t)]),
    "mmdit_step_cache_read": (C.c_int, [C.POINTER(mmdit_config), C.POINTER(mmdit_step_cache), _P]),
    "mmdit_step_modulations_bytes": (C.c_int, [C.POINTER(mmdit_config), C.c_int32, C.POINTER(C.c_size_t)]),
    "mmdit_step_modulations": (C.c_int, [C.POINTER(mmdit_config), C.POINTER(mmdit_model_w), _P, C.POINTER(C.c_double),
                                         C.c_int32, C.POINTER(mmdit_step_opts), _P, C.c_size_t, _P]),
    "mmdit_step_workspace_ex": (C.c_int, [C.POINTER(mmdit_config), C.POINTER(mmdit_model_w),
                                          C.POINTER(mmdit_step_opts), C.POINTER(C.c_size_t)]),
    "mmdit_double_block_fwd": (C.c_int, [C.POINTER(mmdit_dims), C.POINTER(mmdit_double_w), _P, _P, _P, _P,
                                         _P, _P, _P, C.c_size_t, _P]),
    "mmdit_single_block_fwd": (C.c_int, [C.POINTER(mmdit_dims), C.POINTER(mmdit_single_w), _P, _P, _P, _P,
                                         _P, C.c_size_t, _P]),
    "mmdit_step": (C.c_int, [C.POINTER(mmdit_config), C.POINTER(mmdit_model_w), _P, _P, _P, _P, _P,
                             C.c_double, C.c_double, _P, C.c_size_t, _P]),
    "mmdit_step_ex": (C.c_int, [C.POINTER(mmdit_config), C.POINTER(mmdit_model_w), _P, _P, _P, _P, _P,
                                C.c_double, C.c_double, C.POINTER(mmdit_step_opts), _P, C.c_size_t, _P]),
    "mmdit_step_noalloc": (C.c_int, [C.POINTER(mmdit_config), C.POINTER(mmdit_model_w), _P, _P, _P, _P, _P,
                                     C.c_double, C.c_double, C.POINTER(mmdit_step_opts), _P]),
    "mmdit_schedule": (C.c_int, [C.c_int32, C.c_int32, C.c_double, C.c_double, C.c_double, C.c_int32, _P]),
    "mmdit_make_ids": (C.c_int, [C.c_int32, C.c_int32, C.c_int32, C.c_int32, _P]),
    "mmdit_pack_latents": (C.c_int, [_P, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, _P]),
    "mmdit_unpack_latents": (C.c_int, [_P, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, _P]),
    "mmdit_rope_table": (C.c_int, [_P, C.c_int32, _P, C.c_double, _P, _P]),
    "mmdit_quantise": (C.c_int, [_P, C.c_int32, C.c_int32, C.c_int32, _P, _P]),
    "mmdit_dequantise": (C.c_int, [_P, _P, C.c_int32, C.c_int32, C.c_int32, _P, _P]),
    "mmdit_adaln_layernorm": (C.c_int, [_P, C.c_int32, _P, C.c_int32, C.c_int32, C.c_int32, _P, C.c_float, _P]),
    "mmdit_linear_workspace": (C.c_int, [C.POINTER(mmdit_linear), C.c_int32, C.c_int32, C.c_int32,
                                         C.POINTER(C.c_size_t)]),
    "mmdit_linear_fwd": (C.c_int, [C.POINTER(mmdit_linear), C.c_int32, _P, C.c_int32, _P, C.c_int32, C.c_int32,
                                   _P, C.c_size_t, _P]),
    "mmdit_profile_begin": (C.c_int, [C.c_int32, C.c_int32]),
    "mmdit_profile_end": (C.c_int, [C.POINTER(C.c_double), C.POINTER(C.c_int32), C.POINTER(C.c_double)]),
    "mmdit_status_str": (C.c_char_p, [C.c_int32]),
    "mmdit_last_error": (C.c_char_p, []),
    "mmdit_version": (C.c_char_p, []),
}


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libmmdit.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m diffusion_transformer_mmdit_amd.build`")
        L = C.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != 0:
        raise MMDiTError(status, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


# ------------------------------------------------------------------ weights --
def _dt(dtype: int):
    import torch
    return torch.bfloat16 if dtype == BF16 else torch.float32


class Linear:
    """Device tensors of one linear layer (keeps them alive)."""

    def __init__(self, w, bias=None, scales=None, fmt=W_DENSE, n_out=None, k_in=None):
        self.w, self.bias, self.scales, self.fmt = w, bias, scales, fmt
        self.n_out = int(n_out if n_out is not None else w.shape[0])
        self.k_in = int(k_in if k_in is not None else w.shape[1])

    def c(self) -> mmdit_linear:
        return mmdit_linear(_ptr(self.w), _ptr(self.scales), _ptr(self.bias), self.fmt, self.n_out, self.k_in)

    @staticmethod
    def from_numpy(w: np.ndarray, b: Optional[np.ndarray], dtype: int, device, bits: int = 0) -> "Linear":
        import torch
        bt = None if b is None else torch.from_numpy(np.ascontiguousarray(b)).to(device).to(_dt(dtype))
        if bits == 0:
            wt = torch.from_numpy(np.ascontiguousarray(w)).to(device).to(_dt(dtype))
            return Linear(wt, bt)
        packed, scales = mmdit_quantise(w, bits)
        st = torch.from_numpy(scales.view(np.int16)).to(device).view(torch.bfloat16)
        pt = torch.from_numpy(packed).to(device)
        fmt = {4: W_Q4G64, 8: W_Q8G64, 1: W_Q1G128, 2: W_TQ2G128}[bits]
        return Linear(pt, bt, st, fmt, w.shape[0], w.shape[1])


def _vec(a, dtype, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(device).to(_dt(dtype))


class StreamW:
    """One stream of a dual block: Linear objects plus RMSNorm scale tensors."""

    def __init__(self, mod, qkv, proj, fc1, fc2, q_norm, k_norm):
        self.mod, self.qkv, self.proj, self.fc1, self.fc2 = mod, qkv, proj, fc1, fc2
        self.q_norm, self.k_norm = q_norm, k_norm

    @classmethod
    def from_numpy(cls, d: Dict[str, np.ndarray], dtype: int, device, quant: Optional[Dict[str, int]] = None):
        q = quant or {}
        lin = lambda n: Linear.from_numpy(d[n + "_w"], d[n + "_b"], dtype, device, q.get(n, 0))  # noqa: E731
        return cls(Linear.from_numpy(d["mod_w"], d["mod_b"], dtype, device), lin("qkv"), lin("proj"), lin("fc1"),
                   lin("fc2"), _vec(d["q_norm"], dtype, device), _vec(d["k_norm"], dtype, device))

    def c(self) -> mmdit_stream_w:
        return mmdit_stream_w(self.mod.c(), self.qkv.c(), self.proj.c(), self.fc1.c(), self.fc2.c(),
                              _ptr(self.q_norm), _ptr(self.k_norm))


class DoubleW:
    def __init__(self, d, dtype: int = None, device=None, quant=None, img=None, txt=None):
        if d is not None:
            img = StreamW.from_numpy(d["img"], dtype, device, quant)
            txt = StreamW.from_numpy(d["txt"], dtype, device, quant)
        self.img, self.txt = img, txt

    def c(self) -> mmdit_double_w:
        return mmdit_double_w(self.img.c(), self.txt.c())


class SingleW:
    def __init__(self, d, dtype: int = None, device=None, quant=None, mod=None, lin1=None, lin2=None,
                 q_norm=None, k_norm=None):
        if d is not None:
            q = quant or {}
            mod = Linear.from_numpy(d["mod_w"], d["mod_b"], dtype, device)
            lin1 = Linear.from_numpy(d["lin1_w"], d["lin1_b"], dtype, device, q.get("lin1", 0))
            lin2 = Linear.from_numpy(d["lin2_w"], d["lin2_b"], dtype, device, q.get("lin2", 0))
            q_norm = _vec(d["q_norm"], dtype, device)
            k_norm = _vec(d["k_norm"], dtype, device)
        self.mod, self.lin1, self.lin2, self.q_norm, self.k_norm = mod, lin1, lin2, q_norm, k_norm

    def c(self) -> mmdit_single_w:
        return mmdit_single_w(self.mod.c(), self.lin1.c(), self.lin2.c(), _ptr(self.q_norm), _ptr(self.k_norm))


# Quantisation policy: the layers writing into the residual stream keep 8
# bits, the inner projections 4 bits (stable-diffusion.rs README).
QUANT_POLICY = {"qkv": 4, "fc1": 4, "lin1": 4, "proj": 8, "fc2": 8, "lin2": 8}
# every block projection ternary (TQ2G128), as the pictor-tokenizer page's
# text-to-image DiT holds its weights; modulation and embedders stay bf16
TERNARY_POLICY = {"qkv": 2, "fc1": 2, "lin1": 2, "proj": 2, "fc2": 2, "lin2": 2}

GLOBAL_LINEARS = ("img_in", "txt_in", "time_in0", "time_in1", "vec_in0", "vec_in1", "final_mod", "final_lin")
GUIDANCE_LINEARS = ("guidance_in0", "guidance_in1")


class ModelW:
    """Whole-model weights: global Linear objects plus lists of block weights."""

    def __init__(self, g: Optional[Dict[str, np.ndarray]], dbl: Sequence, sgl: Sequence, dtype: int = None,
                 device=None, linears: Optional[Dict[str, Linear]] = None):
        if g is not None:
            names = {n: n for n in GLOBAL_LINEARS}
            names["final_lin"] = "final"
            linears = {n: Linear.from_numpy(g[k + "_w"], g[k + "_b"], dtype, device) for n, k in names.items()}
            if g.get("guidance_in0_w") is not None:
                for n in GUIDANCE_LINEARS:
                    linears[n] = Linear.from_numpy(g[n + "_w"], g[n + "_b"], dtype, device)
        for n in GLOBAL_LINEARS:
            setattr(self, n, linears[n])
        # guidance embedder (guidance-distilled models), absent -> zeroed structs
        self.guidance = [linears[n] for n in GUIDANCE_LINEARS] if GUIDANCE_LINEARS[0] in linears else None
        self.dbl: List = list(dbl)
        self.sgl: List = list(sgl)

    def c(self) -> mmdit_model_w:
        self._dbl_arr = (mmdit_double_w * max(1, len(self.dbl)))(*[d.c() for d in self.dbl])
        self._sgl_arr = (mmdit_single_w * max(1, len(self.sgl)))(*[s.c() for s in self.sgl])
        gl = [x.c() for x in self.guidance] if self.guidance else [mmdit_linear(), mmdit_linear()]
        return mmdit_model_w(*[getattr(self, n).c() for n in GLOBAL_LINEARS],
                             C.cast(self._dbl_arr, C.POINTER(mmdit_double_w)),
                             C.cast(self._sgl_arr, C.POINTER(mmdit_single_w)), *gl)


def make_dims(s, dtype: Optional[int] = None, resid: int = RESID_DEFAULT) -> mmdit_dims:
    """mmdit_dims from an inputs.Shape."""
    d = mmdit_dims()
    d.resid = resid
    d.batch, d.hidden, d.heads, d.head_dim = s.batch, s.hidden, s.heads, s.head_dim
    d.mlp_hidden, d.txt_len, d.img_len = s.mlp_hidden, s.txt_len, s.img_len
    d.axes_dim = (C.c_int32 * 3)(*s.axes_dim)
    d.theta, d.ln_eps, d.rms_eps = s.theta, 1e-6, 1e-6
    d.act_dtype = dtype if dtype is not None else (BF16 if s.dtype == "bf16" else F32)
    return d


def make_config(s, dtype: Optional[int] = None, resid: int = RESID_DEFAULT) -> mmdit_config:
    c = mmdit_config()
    c.dims = make_dims(s, dtype, resid)
    c.n_double, c.n_single = s.n_double, s.n_single
    c.in_ch, c.txt_in_dim, c.vec_in_dim, c.temb_dim = s.in_ch, s.txt_in_dim, s.vec_in_dim, s.temb_dim
    return c


# ------------------------------------------------------------------ entry points --
def mmdit_double_block_workspace(dims: mmdit_dims) -> int:
    n = C.c_size_t()
    _check(lib().mmdit_double_block_workspace(C.byref(dims), C.byref(n)), "mmdit_double_block_workspace")
    return n.value


def mmdit_single_block_workspace(dims: mmdit_dims) -> int:
    n = C.c_size_t()
    _check(lib().mmdit_single_block_workspace(C.byref(dims), C.byref(n)), "mmdit_single_block_workspace")
    return n.value


def mmdit_step_workspace(cfg: mmdit_config) -> int:
    n = C.c_size_t()
    _check(lib().mmdit_step_workspace(C.byref(cfg), C.byref(n)), "mmdit_step_workspace")
    return n.value


def mmdit_double_block_fwd(dims, w: mmdit_double_w, img_in, txt_in, img_out, txt_out, vec, ids, ws,
                           stream=None):
    _check(lib().mmdit_double_block_fwd(C.byref(dims), C.byref(w), _ptr(img_in), _ptr(txt_in), _ptr(img_out),
                                        _ptr(txt_out), _ptr(vec), _ptr(ids), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)),
           "mmdit_double_block_fwd")


def mmdit_single_block_fwd(dims, w: mmdit_single_w, x_in, x_out, vec, ids, ws, stream=None):
    _check(lib().mmdit_single_block_fwd(C.byref(dims), C.byref(w), _ptr(x_in), _ptr(x_out), _ptr(vec),
                                        _ptr(ids), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)),
           "mmdit_single_block_fwd")


def mmdit_step(cfg, w: mmdit_model_w, x_packed, v_out, txt_emb, y, ids, sigma: float, sigma_next: float, ws,
               stream=None):
    _check(lib().mmdit_step(C.byref(cfg), C.byref(w), _ptr(x_packed), _ptr(v_out), _ptr(txt_emb), _ptr(y),
                            _ptr(ids), float(sigma), float(sigma_next), _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(stream)),
           "mmdit_step")


def mmdit_step_workspace_ex(cfg: mmdit_config, w: mmdit_model_w, dequant_in_gemm: bool = False) -> int:
    """Workspace bytes of mmdit_step_ex for these weights (no room for decoded
    weights when no layer is decoded)."""
    o = mmdit_step_opts()
    o.dequant = 1 if dequant_in_gemm else 0
    n = C.c_size_t()
    _check(lib().mmdit_step_workspace_ex(C.byref(cfg), C.byref(w), C.byref(o), C.byref(n)),
           "mmdit_step_workspace_ex")
    return n.value


def mmdit_step_cache_bytes(cfg: mmdit_config) -> int:
    n = C.c_size_t()
    _check(lib().mmdit_step_cache_bytes(C.byref(cfg), C.byref(n)), "mmdit_step_cache_bytes")
    return n.value


class StepCache:
    """Step-cache state of one generation: the device buffer (a torch uint8
    tensor) and the mmdit_step_cache struct the library updates. on_device:
    the decision is taken by a kernel (graph-capturable); read() copies it
    back into ran_blocks / rel / acc."""

    def __init__(self, cfg: mmdit_config, device="cuda", on_device: bool = False):
        import torch
        self.cfg = cfg
        self.on_device = on_device
        self.buf = torch.empty(mmdit_step_cache_bytes(cfg), dtype=torch.uint8, device=device)
        self.c = mmdit_step_cache()
        self.c.buf = self.buf.data_ptr()
        self.c.bytes = self.buf.numel()
        self.reset()

    def reset(self):
        """Start a new generation (the next step runs the blocks)."""
        self.c.valid = 0
        self.c.acc = 0.0

    @property
    def ran_blocks(self) -> bool:
        return bool(self.c.ran_blocks)

    @property
    def rel(self) -> float:
        return self.c.rel

    def read(self, stream=None):
        """mmdit_step_cache_read: waits for the stream, then fills ran_blocks,
        acc and rel from the device state."""
        _check(lib().mmdit_step_cache_read(C.byref(self.cfg), C.byref(self.c), _stream(stream)),
               "mmdit_step_cache_read")


def mmdit_step_ex(cfg, w: mmdit_model_w, x_packed, v_out, txt_emb, y, ids, sigma: float, sigma_next: float, ws,
                  ctx_packed=None, ctx_len: int = 0, guidance: Optional[float] = None, stream=None,
                  cache: Optional[StepCache] = None, cache_threshold: float = 0.0, dequant_in_gemm: bool = False,
                  mods=None, mods_count: int = 0, mods_index: int = 0):
    o = mmdit_step_opts()
    o.dequant = 1 if dequant_in_gemm else 0
    o.mods = _ptr(mods)
    o.mods_count = int(mods_count)
    o.mods_index = int(mods_index)
    o.ctx_packed = _ptr(ctx_packed)
    o.ctx_len = int(ctx_len)
    o.has_guidance = 0 if guidance is None else 1
    o.guidance = 0.0 if guidance is None else float(guidance)
    if cache is not None:
        o.cache = C.pointer(cache.c)
        o.cache_threshold = float(cache_threshold)
        o.cache_on_device = 1 if cache.on_device else 0
    _check(lib().mmdit_step_ex(C.byref(cfg), C.byref(w), _ptr(x_packed), _ptr(v_out), _ptr(txt_emb), _ptr(y),
                               _ptr(ids), float(sigma), float(sigma_next), C.byref(o), _ptr(ws),
                               ws.numel() * ws.element_size(), _stream(stream)),
           "mmdit_step_ex")


def mmdit_step_modulations_bytes(cfg: mmdit_config, n_sigma: int) -> int:
    n = C.c_size_t()
    _check(lib().mmdit_step_modulations_bytes(C.byref(cfg), int(n_sigma), C.byref(n)), "mmdit_step_modulations_bytes")
    return n.value


def mmdit_step_modulations(cfg, w: mmdit_model_w, y, sigmas, mods, guidance: Optional[float] = None, stream=None):
    """Modulation vectors for the timesteps `sigmas` in one pass over the
    modulation weights; pass `mods` to mmdit_step_ex with mods_count =
    len(sigmas) and mods_index = j for the step at sigmas[j]."""
    sg = (C.c_double * len(sigmas))(*[float(v) for v in sigmas])
    o = mmdit_step_opts()
    o.has_guidance = 0 if guidance is None else 1
    o.guidance = 0.0 if guidance is None else float(guidance)
    _check(lib().mmdit_step_modulations(C.byref(cfg), C.byref(w), _ptr(y), sg, len(sigmas), C.byref(o), _ptr(mods),
                                        mods.numel() * mods.element_size(), _stream(stream)),
           "mmdit_step_modulations")


NOALLOC_SCRATCH_BYTES = 256 << 20  # the library's scratch per GPU (mmdit_step_noalloc)


def mmdit_step_noalloc(cfg, w: mmdit_model_w, x_packed, v_out, txt_emb, y, ids, sigma: float, sigma_next: float,
                       stream=None):
    """mmdit_step on the library's own scratch (no workspace argument)."""
    _check(lib().mmdit_step_noalloc(C.byref(cfg), C.byref(w), _ptr(x_packed), _ptr(v_out), _ptr(txt_emb), _ptr(y),
                                    _ptr(ids), float(sigma), float(sigma_next), None, _stream(stream)),
           "mmdit_step_noalloc")


def mmdit_schedule(n_steps: int, img_len: int, base_shift=0.5, max_shift=1.15, sigma_terminal=0.0,
                   shift=True) -> np.ndarray:
    out = np.zeros(n_steps + 1, dtype=np.float64)
    _check(lib().mmdit_schedule(n_steps, img_len, base_shift, max_shift, sigma_terminal, int(shift),
                                out.ctypes.data_as(C.c_void_p)), "mmdit_schedule")
    return out


def mmdit_make_ids(grid_h: int, grid_w: int, txt_len: int, frame: int = 0) -> np.ndarray:
    out = np.zeros((txt_len + grid_h * grid_w, 3), dtype=np.int32)
    _check(lib().mmdit_make_ids(grid_h, grid_w, txt_len, frame, out.ctypes.data_as(C.c_void_p)), "mmdit_make_ids")
    return out


def mmdit_pack_latents(z, x, stream=None):
    B, Cc, H, W = z.shape
    _check(lib().mmdit_pack_latents(_ptr(z), _ptr(x), B, Cc, H, W, z.element_size(), _stream(stream)),
           "mmdit_pack_latents")


def mmdit_unpack_latents(x, z, stream=None):
    B, Cc, H, W = z.shape
    _check(lib().mmdit_unpack_latents(_ptr(x), _ptr(z), B, Cc, H, W, z.element_size(), _stream(stream)),
           "mmdit_unpack_latents")


def mmdit_rope_table(ids, axes_dim, theta, table, stream=None):
    ax = np.ascontiguousarray(np.asarray(axes_dim, dtype=np.int32))
    _check(lib().mmdit_rope_table(_ptr(ids), ids.shape[0], ax.ctypes.data_as(C.c_void_p), float(theta),
                                  _ptr(table), _stream(stream)), "mmdit_rope_table")


def mmdit_quantise(w: np.ndarray, bits: int):
    """Returns (packed uint8/int8 codes, scales as uint16 bf16 bits)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    if bits in (1, 2):  # Q1G128 / TQ2G128
        packed = np.zeros((n, k * bits // 8), dtype=np.uint8)
        scales = np.zeros((n, k // 128), dtype=np.uint16)
    else:
        packed = np.zeros((n, k // 2) if bits == 4 else (n, k), dtype=np.uint8 if bits == 4 else np.int8)
        scales = np.zeros((n, k // 64), dtype=np.uint16)
    _check(lib().mmdit_quantise(w.ctypes.data_as(C.c_void_p), n, k, bits, packed.ctypes.data_as(C.c_void_p),
                                scales.ctypes.data_as(C.c_void_p)), "mmdit_quantise")
    return packed, scales


def mmdit_dequantise(w, scales, fmt: int, n_out: int, k_in: int, out, stream=None):
    """Decodes quantised codes `w` with bf16 `scales` (device tensors) into
    the bf16 tensor `out` [n_out, k_in]."""
    _check(lib().mmdit_dequantise(_ptr(w), _ptr(scales), fmt, n_out, k_in, _ptr(out), _stream(stream)),
           "mmdit_dequantise")


def mmdit_adaln_layernorm(x, y, shift_scale, eps: float = 1e-6, stream=None):
    """y = (1 + scale) LN(x) + shift over the last axis; x float32 or in y's
    dtype, shift_scale float32 [2, hidden]."""
    import torch
    act = BF16 if y.dtype == torch.bfloat16 else F32
    rows, hidden = y.numel() // y.shape[-1], y.shape[-1]
    _check(lib().mmdit_adaln_layernorm(_ptr(x), int(x.dtype == torch.float32), _ptr(y), act, rows, hidden,
                                       _ptr(shift_scale), float(eps), _stream(stream)), "mmdit_adaln_layernorm")


def mmdit_linear_workspace(lin: Linear, act_dtype: int, M: int, route: int = ROUTE_AUTO) -> int:
    n = C.c_size_t()
    lc = lin.c()
    _check(lib().mmdit_linear_workspace(C.byref(lc), act_dtype, M, route, C.byref(n)), "mmdit_linear_workspace")
    return n.value


def mmdit_linear_fwd(lin: Linear, x, y, route: int = ROUTE_AUTO, ws=None, stream=None):
    """y [M, n_out] = x [M, k_in] W^T + b; y float32 or x's dtype."""
    import torch
    act = BF16 if x.dtype == torch.bfloat16 else F32
    M = x.numel() // x.shape[-1]
    lc = lin.c()
    _check(lib().mmdit_linear_fwd(C.byref(lc), act, _ptr(x), M, _ptr(y), int(y.dtype == torch.float32), route,
                                  _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)),
           "mmdit_linear_fwd")


def mmdit_profile_begin(kernel_class: int, max_launches: int):
    _check(lib().mmdit_profile_begin(kernel_class, max_launches), "mmdit_profile_begin")


def mmdit_profile_end():
    ms, n, work = C.c_double(), C.c_int32(), C.c_double()
    _check(lib().mmdit_profile_end(C.byref(ms), C.byref(n), C.byref(work)), "mmdit_profile_end")
    return ms.value, n.value, work.value


def mmdit_status_str(status: int) -> str:
    return lib().mmdit_status_str(status).decode()


def mmdit_last_error() -> str:
    return lib().mmdit_last_error().decode()


def mmdit_version() -> str:
    return lib().mmdit_version().decode()
