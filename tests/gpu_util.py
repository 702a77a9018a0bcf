"""Helpers for the GPU parity tests: device upload, comparison metrics and
the tolerance of each precision."""
import numpy as np

from diffusion_transformer_mmdit_amd import binding as bd


def torch():
    import torch as t
    return t


def dev():
    return torch().device("cuda:0")


def up(a, dtype: str):
    """numpy float32 -> device tensor in the workload dtype (exact for bf16-valued data)."""
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())
    return x.to(t.bfloat16) if dtype == "bf16" else x


def up_i32(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev())


def down(x) -> np.ndarray:
    return x.detach().float().cpu().numpy()


def rel_l2(got, ref) -> float:
    g = np.asarray(got, np.float64)
    r = np.asarray(ref, np.float64)
    return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))


def cosine(got, ref) -> float:
    g = np.asarray(got, np.float64).ravel()
    r = np.asarray(ref, np.float64).ravel()
    return float(np.dot(g, r) / max(np.linalg.norm(g) * np.linalg.norm(r), 1e-300))


# Tolerances: fp32 rel-L2 <= 1e-5; bf16 and quantised rel-L2 <= 2e-2 with
# cosine >= 0.999 (the pictor README's per-stage cosine gate).
TOL = {"f32": dict(rel=1e-5, cos=None), "bf16": dict(rel=2e-2, cos=0.999)}


def assert_parity(got, ref, dtype: str, what: str = ""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    r = rel_l2(got, ref)
    tol = TOL[dtype]
    msg = f"{what}: rel_l2 {r:.3e} (tol {tol['rel']})"
    assert r <= tol["rel"], msg
    if tol["cos"] is not None:
        c = cosine(got, ref)
        assert c >= tol["cos"], f"{what}: cosine {c:.6f} < {tol['cos']}"
    print(msg, flush=True)
    return r


def workspace(nbytes: int):
    t = torch()
    return t.empty(max(nbytes, 256), dtype=t.uint8, device=dev())


def sync():
    torch().cuda.synchronize()


def dtype_code(s: str) -> int:
    return bd.BF16 if s == "bf16" else bd.F32
