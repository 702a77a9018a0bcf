"""Error-budget diagnostic of the full denoising step (not a test; run by
hand on a machine with the GPU):

    python tests/error_budget.py [--tokens 4608|320] [--out FILE]

For every depth k = 1 .. 57 (the first k blocks of the 19 dual + 38 single
blocks of the seeded random-init 1024^2 model), v_k is the final layer
applied to the image tokens after block k. Three v_k are compared:
  * the float64 oracle (the reference),
  * the float32 oracle,
  * the GPU step run with the model cut to its first k blocks (bf16 operands,
    float32 residual).
Printed per depth: rel-L2 of the float32 oracle and of the GPU against the
float64 oracle, and of the GPU against the float32 oracle. The oracle side
composes the oracle's own functions in the order oracle.step applies them.
"""
import argparse
import dataclasses
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from diffusion_transformer_mmdit_amd import binding as bd  # noqa: E402
from diffusion_transformer_mmdit_amd import inputs as I  # noqa: E402
from tests.test_gpu_depth import _inputs, double_np, global_np, single_np  # noqa: E402


def rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--tokens", type=int, default=4608, choices=(4608, 320))
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "error_budget.json"))
    a = ap.parse_args()
    import torch
    from diffusion_transformer_mmdit_amd import random_init as RI
    S = I.CFG4 if a.tokens == 4608 else dataclasses.replace(I.CFG4, txt_len=64, grid_h=16, grid_w=16)
    dev = torch.device("cuda:0")
    M = RI.model(S, seed=42, device=dev)
    X, T, y, ids, sig = _inputs(S)
    s0, s1 = sig[1], sig[2]
    nd, ns = S.n_double, S.n_single
    # GPU: v after the first k blocks, k = 1 .. nd + ns
    Xd = torch.from_numpy(X).to(dev)
    Td = torch.from_numpy(T).to(dev).to(torch.bfloat16)
    yd = torch.from_numpy(y).to(dev).to(torch.bfloat16)
    idd = torch.from_numpy(ids).to(dev)
    ws = torch.empty(bd.mmdit_step_workspace(bd.make_config(S)), dtype=torch.uint8, device=dev)
    v_gpu = []
    for k in range(1, nd + ns + 1):
        kd, ks = min(k, nd), max(0, k - nd)
        Sk = dataclasses.replace(S, n_double=kd, n_single=ks)
        Mk = bd.ModelW(None, M.dbl[:kd], M.sgl[:ks], linears={n: getattr(M, n) for n in bd.GLOBAL_LINEARS})
        Xr = Xd.clone()
        v = torch.empty_like(Xr)
        bd.mmdit_step(bd.make_config(Sk), Mk.c(), Xr, v, Td, yd, idd, s0, s1, ws)
        torch.cuda.synchronize()
        v_gpu.append(v.cpu().numpy())
    print(f"GPU: {len(v_gpu)} truncated steps done", flush=True)
    # oracle in float32 and float64, one block at a time
    g = global_np(M)
    st = {}
    for dt in (np.float32, np.float64):
        Xc, Tc, yc = X.astype(dt), T.astype(dt), y.astype(dt)
        st[dt] = dict(img=oracle.linear(Xc, g["img_in_w"], g["img_in_b"]),
                      txt=oracle.linear(Tc, g["txt_in_w"], g["txt_in_b"]),
                      vec=oracle.conditioning_vec(g, s0, yc, temb_dim=S.temb_dim))
    rows = []
    Lt = S.txt_len
    t0 = time.time()
    for k in range(1, nd + ns + 1):
        w = double_np(M.dbl[k - 1]) if k <= nd else single_np(M.sgl[k - 1 - nd])
        v_or = {}
        for dt, s in st.items():
            if k <= nd:
                s["img"], s["txt"] = oracle.double_block(w, s["img"], s["txt"], s["vec"], ids, S.heads, S.axes_dim,
                                                         S.theta)
                img = s["img"]
            else:
                if k == nd + 1:
                    s["x"] = np.concatenate([s["txt"], s["img"]], axis=1)
                s["x"] = oracle.single_block(w, s["x"], s["vec"], ids, S.heads, S.axes_dim, S.theta)
                img = s["x"][:, Lt:]
            v_or[dt] = oracle.final_layer(g, img, s["vec"])
        r = dict(depth=k, kind="dual" if k <= nd else "single",
                 f32_vs_f64=rel(v_or[np.float32], v_or[np.float64]),
                 gpu_vs_f64=rel(v_gpu[k - 1], v_or[np.float64]),
                 gpu_vs_f32=rel(v_gpu[k - 1], v_or[np.float32].astype(np.float64)))
        rows.append(r)
        print(f"depth {k:2d} ({r['kind']:6s}) f32-oracle vs f64 {r['f32_vs_f64']:.3e}  GPU vs f64 "
              f"{r['gpu_vs_f64']:.3e}  GPU vs f32-oracle {r['gpu_vs_f32']:.3e}  ({time.time() - t0:.0f} s)",
              flush=True)
    os.makedirs(os.path.dirname(a.out), exist_ok=True)
    with open(a.out, "w") as f:
        json.dump(dict(tokens=S.seq_len, sigma=[s0, s1], rows=rows), f, indent=1)
    print(f"wrote {a.out}", flush=True)


if __name__ == "__main__":
    main()
