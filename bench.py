#!/usr/bin/env python3
"""Benchmark of the FLUX-style MMDiT denoising step on one MI355X.

Workload: one denoising step at 1024x1024 (64x64 patch grid = 4096 image
tokens, 512 text tokens, joint sequence 4608), 19 dual-stream + 38
single-stream blocks, hidden 3072, 24 heads x 128, MLP 12288, bf16 operands
with float32 accumulation, batch 1, random-init weights drawn on the GPU.
A step = conditioning vector, all modulations, input projections, the 57
blocks, the final layer and the fused Euler update (mmdit_step).

Prints ONE JSON line. `value` is the step latency in ms (lower is better).
Extra fields: HIP-graph replay latency, block TFLOP/s for one dual and one
single block at 4608 tokens, the quantised-weight step latency, the roofline
of the dominant GEMM kernel (timed with HIP events on the library's stream)
and the CPU oracle on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import dataclasses
import json
import os
import sys
import time

METRIC = "MMDiT step latency (ms) + block TFLOP/s at 1024² (4096 img+512 txt tok), bf16"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def block_flops(s):
    """Algorithmic FLOPs of one dual (== single) block at s: projections
    2 L sum(K N) + attention 4 H L^2 d."""
    h, m, L, H = s.hidden, s.mlp_hidden, s.seq_len, s.heads
    kn_dual = h * 3 * h + h * h + h * m + m * h
    kn_single = h * (3 * h + m) + (h + m) * h
    assert kn_dual == kn_single
    return 2.0 * L * kn_dual + 4.0 * H * L * L * s.head_dim


def step_flops(s):
    h = s.hidden
    Li, Lt = s.img_len, s.txt_len
    blocks = (s.n_double + s.n_single) * block_flops(s)
    io = 2.0 * Li * s.in_ch * h + 2.0 * Lt * s.txt_in_dim * h + 2.0 * Li * h * s.in_ch
    return blocks + io


def lin1_traffic():
    """HBM bytes per launch of the linear1 GEMM from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (scaled by a 1 GiB copy's counts), or None
    when the kernel's sources have changed since those counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        rec = json.load(open(os.path.join(here, "profiles", "gemm_lin1_traffic.json")))
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(here, "diffusion_transformer_mmdit_amd", "csrc", src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def vendor_reference(s):
    """Context only: the ROCm libraries torch calls, on this path's two
    dominant shapes. torch's bf16 linear (hipBLASLt) on the single-block
    linear1 GEMM, and torch's flash SDPA on the joint attention (the flash
    backend is forced: no math-path fallback)."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    res = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    M, K, N = s.seq_len, s.hidden, 3 * s.hidden + s.mlp_hidden
    A = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    W = (torch.randn(N, K, device="cuda", generator=g) * 0.02).to(torch.bfloat16)

    def t_ms(fn, n=10):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n
    ms = t_ms(lambda: torch.nn.functional.linear(A, W))
    res["torch_linear_linear1"] = {"shape": [M, N, K], "avg_us": round(ms * 1e3, 1),
                                   "tflops": round(2.0 * M * N * K / ms / 1e9, 1)}
    del A, W
    H, L, D = s.heads, s.seq_len, s.head_dim
    q, k, v = (torch.randn(1, H, L, D, device="cuda", generator=g).to(torch.bfloat16) for _ in range(3))
    try:
        with sdpa_kernel(SDPBackend.FLASH_ATTENTION):
            ms = t_ms(lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v))
        res["torch_flash_sdpa"] = {"shape": [1, H, L, D], "avg_us": round(ms * 1e3, 1),
                                   "tflops": round(4.0 * H * L * L * D / ms / 1e9, 1)}
    except RuntimeError as e:
        res["torch_flash_sdpa"] = {"unavailable": str(e)[:120]}
    torch.cuda.synchronize()
    return res


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def lin1_clock():
    """Sustained shader clock (GHz) of the linear1 GEMM from the committed
    GRBM_GUI_ACTIVE pass, or None when the kernel's sources have changed."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        rec = json.load(open(os.path.join(here, "profiles", "gemm_lin1_clock.json")))
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(here, "diffusion_transformer_mmdit_amd", "csrc", src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return float(rec["clock_ghz"]), float(rec["max_clock_ghz"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(s):
    """The oracle on the host cores: one dual and one single block at the
    full 4608-token size (config-3 weights), scaled to 19 + 38 blocks."""
    import numpy as np
    import threadpoolctl

    import oracle
    from diffusion_transformer_mmdit_amd import inputs as I
    sb = dataclasses.replace(I.CFG3, txt_len=s.txt_len, grid_h=s.grid_h, grid_w=s.grid_w)
    x = I.block_inputs(sb)
    ids = oracle.make_ids(sb.grid_h, sb.grid_w, sb.txt_len)
    wd = I.double_block_weights(sb, 0)
    t0 = time.perf_counter()
    oracle.double_block(wd, x["x_img"], x["x_txt"], x["vec"], ids, sb.heads)
    t_dual = time.perf_counter() - t0
    del wd
    ws = I.single_block_weights(sb, 0)
    t0 = time.perf_counter()
    oracle.single_block(ws, x["x"], x["vec"], ids, sb.heads)
    t_single = time.perf_counter() - t0
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    est_ms = 1e3 * (s.n_double * t_dual + s.n_single * t_single)
    # one core: one dual block at 1280 tokens (256 text + 32x32 image)
    s2 = I.CFG2
    x2 = I.block_inputs(s2)
    w2 = I.double_block_weights(s2, 0)
    ids2 = oracle.make_ids(s2.grid_h, s2.grid_w, s2.txt_len)
    with threadpoolctl.threadpool_limits(1):
        t0 = time.perf_counter()
        oracle.double_block(w2, x2["x_img"], x2["x_txt"], x2["vec"], ids2, s2.heads)
        t_one = time.perf_counter() - t0
        one_threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()
                           if i.get("user_api") == "blas"] or [1])
    flops2 = block_flops(s2)
    one_core = {"block": "dual, 256 text + 1024 image tokens, h 3072", "blas_threads": int(one_threads),
                "seconds": round(t_one, 2),
                "gflops": round(flops2 / t_one / 1e9, 1)}
    return {"value": round(est_ms, 1), "unit": "ms", "cores": int(threads), "kind": "oracle",
            "gflops": round(step_flops(s) / (est_ms * 1e-3) / 1e9, 1), "one_core": one_core,
            "sample": (f"numpy float32 oracle, 1 dual block ({t_dual:.2f} s) + 1 single block ({t_single:.2f} s) "
                       f"at 4608 tokens, scaled to {s.n_double}+{s.n_single} blocks; BLAS "
                       f"{info[0].get('internal_api', '?') if info else '?'}, affinity "
                       f"{len(os.sched_getaffinity(0))} cores")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=12)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip block, graph and quantised timings")
    ap.add_argument("--cache-threshold", type=float, default=0.25,
                    help="step-cache threshold of the cached 50-step generation")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run one plain device copy of this many MiB (calibrates HBM byte counters)")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}): the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from diffusion_transformer_mmdit_amd import binding as bd
    from diffusion_transformer_mmdit_amd import inputs as I
    from diffusion_transformer_mmdit_amd import random_init as RI

    bd.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.copy_probe_mib > 0:
        n = a.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {a.copy_probe_mib} MiB read + {a.copy_probe_mib} MiB written")
        del src, dst
    s = I.CFG4
    log(f"building random-init model: {s.n_double}+{s.n_single} blocks, h {s.hidden}, bf16")
    t0 = time.perf_counter()
    M = RI.model(s, seed=42, device=dev)
    mc = M.c()
    cfg = bd.make_config(s)
    torch.cuda.synchronize()
    log(f"  weights ready in {time.perf_counter() - t0:.1f} s")

    inp_z = I.box_muller(s.batch * 16 * 4 * s.grid_h * s.grid_w).reshape(s.batch, 16, 2 * s.grid_h, 2 * s.grid_w)
    z = torch.from_numpy(inp_z).to(dev)
    X = torch.empty((s.batch, s.img_len, s.in_ch), dtype=torch.float32, device=dev)
    bd.mmdit_pack_latents(z, X)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    T = torch.randn((s.batch, s.txt_len, s.txt_in_dim), generator=g, device=dev).to(torch.bfloat16)
    y = torch.randn((s.batch, s.vec_in_dim), generator=g, device=dev).to(torch.bfloat16)
    ids = torch.from_numpy(bd.mmdit_make_ids(s.grid_h, s.grid_w, s.txt_len)).to(dev)
    sig = bd.mmdit_schedule(4, s.img_len)
    v = torch.empty_like(X)
    ws = torch.empty(bd.mmdit_step_workspace(cfg), dtype=torch.uint8, device=dev)

    def step(i, model_c=mc, xx=X):
        j = i % 4
        bd.mmdit_step(cfg, model_c, xx, v, T, y, ids, sig[j], sig[j + 1], ws)

    def timed(fn, n):
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / n

    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    ms = timed(step, a.steps)
    log(f"step: {ms:.2f} ms")
    # spread: each of a.steps further steps timed alone with events on the stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        step(i)
        e1.record()
    torch.cuda.synchronize()
    per = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    spread = {"median": round(float(np.median(per)), 3), "p10": round(float(np.percentile(per, 10)), 3),
              "p90": round(float(np.percentile(per, 90)), 3), "n": int(per.size)}
    log(f"step spread: median {spread['median']:.2f} ms, p10 {spread['p10']:.2f}, p90 {spread['p90']:.2f}")
    # the 4-step loop of the schedule, from the same latent each time
    X0 = X.clone()

    def loop4(_):
        X.copy_(X0)
        for j in range(4):
            step(j)
    loop4(0)
    loop_ms = timed(loop4, max(2, a.steps // 4))
    log(f"4-step loop: {loop_ms:.2f} ms")
    flops = step_flops(s)

    # roofline of the dominant kernels, timed with HIP events around each launch
    prof = {}
    for name, cls in (("gemm_lin1", bd.PC_GEMM_LIN1), ("gemm_all", bd.PC_GEMM), ("attention", bd.PC_ATTN)):
        bd.mmdit_profile_begin(cls, 400 * max(1, a.steps))
        for i in range(a.steps):
            step(i)
        tot_ms, n, work = bd.mmdit_profile_end()
        prof[name] = dict(ms_total=tot_ms, launches=n, flops=work,
                          avg_us=1e3 * tot_ms / max(n, 1), tflops=work / max(tot_ms, 1e-9) / 1e9)
        log(f"{name}: {n} launches, avg {prof[name]['avg_us']:.1f} us, {prof[name]['tflops']:.1f} TFLOP/s")
    # HBM-bound kernels: work counted in algorithmic bytes
    mem = {}
    for name, cls in (("layernorm", bd.PC_LN), ("qk_norm_rope", bd.PC_QKNORM), ("gemv", bd.PC_GEMV)):
        bd.mmdit_profile_begin(cls, 400 * max(1, a.steps))
        for i in range(a.steps):
            step(i)
        tot_ms, n, work = bd.mmdit_profile_end()
        gbps = work / max(tot_ms, 1e-9) / 1e6
        mem[name] = dict(ms_per_step=round(tot_ms / max(a.steps, 1), 4), launches_per_step=n // max(a.steps, 1),
                         avg_us=round(1e3 * tot_ms / max(n, 1), 2), gbps=round(gbps, 1),
                         frac=round(gbps / PEAK_HBM_GBS, 4))
        log(f"{name}: {mem[name]['ms_per_step']:.3f} ms/step in {mem[name]['launches_per_step']} launches, "
            f"{mem[name]['gbps']:.0f} GB/s")
    dom = "gemm_lin1"
    p = prof[dom]
    traffic = lin1_traffic()
    roofline = {"bound": "mfma", "kernel": "k_gemm_dma 256x256 direct-to-LDS, split epilogue with fused QK "
                "RMSNorm + RoPE (single-block linear1, M 4608 N 21504 K 3072)", "achieved": round(p["tflops"], 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(p["tflops"] / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                "avg_launch_us": round(p["avg_us"], 2), "flops_per_launch": p["flops"] / max(p["launches"], 1)}
    clk = lin1_clock()
    if clk:
        pk = PEAK_BF16_TFLOPS * clk[0] / clk[1]
        roofline.update({"clock_ghz_measured": clk[0], "peak_at_measured_clock": round(pk, 1),
                         "frac_at_measured_clock": round(p["tflops"] / pk, 4)})

    out = {"metric": METRIC, "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": round(ms, 3), "higher_is_better": False, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded random-init weights and inputs)",
           "config": {"workload": "FLUX-style MMDiT denoising step at 1024x1024: 19 dual + 38 single blocks, "
                                  "hidden 3072, 24x128 heads, MLP 12288, 4096 image + 512 text tokens, batch 1",
                      "global_batch": 1, "seq_len": s.seq_len, "image_tokens": s.img_len, "text_tokens": s.txt_len,
                      "parallelism": "single GPU"},
           "step_spread_ms": spread, "loop_4_steps_ms": round(loop_ms, 3),
           "device": {"name": torch.cuda.get_device_name(0), "hip": torch.version.hip,
                      "torch": torch.__version__},
           "step_tflops": round(flops / ms / 1e9, 1),
           "step_frac_of_bf16_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
           "roofline": roofline,
           "kernels": {k: {"avg_us": round(v_["avg_us"], 2), "tflops": round(v_["tflops"], 1),
                           "frac": round(v_["tflops"] / PEAK_BF16_TFLOPS, 4),
                           "launches_per_step": v_["launches"] // max(a.steps, 1)} for k, v_ in prof.items()},
           "hbm_kernels": mem}

    if not a.no_extras:
        # HIP graphs: one captured graph per schedule position (sigma differs)
        graphs = []
        try:
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            for j in range(4):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=cap):
                    step(j)
                graphs.append(gr)
            torch.cuda.synchronize()
            for i in range(4):
                graphs[i % 4].replay()
            gms = timed(lambda i: graphs[i % 4].replay(), a.steps)
            out["graph_ms_per_step"] = round(gms, 3)
            log(f"graph step: {gms:.2f} ms")
        except Exception as e:  # report, do not hide the main number
            out["graph_ms_per_step"] = None
            out["graph_error"] = str(e)[:200]
        del graphs

        # block TFLOP/s at 4608 tokens, two weight sets alternating
        s3 = I.CFG3
        dims = bd.make_dims(s3)
        dbl = [RI.double_block(s3, 100 + i, dev) for i in range(2)]
        sgl = [RI.single_block(s3, 200 + i, dev) for i in range(2)]
        dblc = [d.c() for d in dbl]
        sglc = [x.c() for x in sgl]
        img = torch.randn((1, s3.img_len, s3.hidden), generator=g, device=dev).to(torch.bfloat16)
        txt = torch.randn((1, s3.txt_len, s3.hidden), generator=g, device=dev).to(torch.bfloat16)
        xj = torch.randn((1, s3.seq_len, s3.hidden), generator=g, device=dev).to(torch.bfloat16)
        vec = torch.randn((1, s3.hidden), generator=g, device=dev).to(torch.bfloat16)
        ids3 = torch.from_numpy(bd.mmdit_make_ids(s3.grid_h, s3.grid_w, s3.txt_len)).to(dev)
        wsb = torch.empty(max(bd.mmdit_double_block_workspace(dims), bd.mmdit_single_block_workspace(dims)),
                          dtype=torch.uint8, device=dev)
        io, to = torch.empty_like(img), torch.empty_like(txt)
        xo = torch.empty_like(xj)
        fd = lambda i: bd.mmdit_double_block_fwd(dims, dblc[i % 2], img, txt, io, to, vec, ids3, wsb)  # noqa
        fs = lambda i: bd.mmdit_single_block_fwd(dims, sglc[i % 2], xj, xo, vec, ids3, wsb)  # noqa
        for i in range(4):
            fd(i)
            fs(i)
        nb = max(2 * a.steps, 8)
        dms = timed(fd, nb)
        sms = timed(fs, nb)
        bf = block_flops(s3)
        out["block"] = {"dual_ms": round(dms, 4), "single_ms": round(sms, 4),
                        "dual_tflops": round(bf / dms / 1e9, 1), "single_tflops": round(bf / sms / 1e9, 1),
                        "dual_block_fwd_per_s": round(1e3 / dms, 1), "single_block_fwd_per_s": round(1e3 / sms, 1),
                        "flops_per_block": bf}
        log(f"blocks: dual {dms:.3f} ms ({bf / dms / 1e9:.0f} TFLOP/s), single {sms:.3f} ms "
            f"({bf / sms / 1e9:.0f} TFLOP/s)")
        del dbl, sgl, dblc, sglc

        # quantised-weight step (4-bit inner projections, 8-bit residual-writing layers)
        Mq = RI.model(I.CFG5, seed=43, device=dev, quant=bd.QUANT_POLICY)
        mqc = Mq.c()
        Xq = X.clone()
        for i in range(a.warmup):
            step(i, mqc, Xq)
        qms = timed(lambda i: step(i, mqc, Xq), a.steps)
        out["quantised_ms_per_step"] = round(qms, 3)
        log(f"quantised step: {qms:.2f} ms")
        # at 4608 rows each quantised layer is decoded to bf16 once per launch
        bd.mmdit_profile_begin(bd.PC_DEQUANT, 400 * max(1, a.steps))
        for i in range(a.steps):
            step(i, mqc, Xq)
        dq_ms, dq_n, dq_b = bd.mmdit_profile_end()
        out["quantised_decode"] = {"ms_per_step": round(dq_ms / max(a.steps, 1), 3),
                                   "launches_per_step": dq_n // max(a.steps, 1),
                                   "gbps": round(dq_b / max(dq_ms, 1e-9) / 1e6, 1)}
        log(f"quantised decode: {out['quantised_decode']['ms_per_step']:.3f} ms/step in "
            f"{out['quantised_decode']['launches_per_step']} launches, {out['quantised_decode']['gbps']:.0f} GB/s")
        # the same step with every quantised layer dequantised inside its GEMM
        qstep = lambda i: bd.mmdit_step_ex(cfg, mqc, Xq, v, T, y, ids, sig[i % 4], sig[i % 4 + 1], ws,  # noqa
                                           dequant_in_gemm=True)
        for i in range(2):
            qstep(i)
        qgms = timed(qstep, a.steps)
        out["quantised_in_gemm_ms_per_step"] = round(qgms, 3)
        log(f"quantised step, dequantised inside the GEMMs: {qgms:.2f} ms")
        del Mq, mqc

        # ternary-weight step (TQ2G128 in every block projection)
        Mt = RI.model(I.CFG5, seed=45, device=dev, quant=bd.TERNARY_POLICY)
        mtc = Mt.c()
        Xt = X.clone()
        for i in range(2):
            step(i, mtc, Xt)
        tms = timed(lambda i: step(i, mtc, Xt), max(a.steps // 2, 3))
        out["ternary_ms_per_step"] = round(tms, 3)
        log(f"ternary step: {tms:.2f} ms")
        del Mt, mtc, Xt

        # reference-image (Kontext-style) step: 4096 context tokens with frame
        # id 1 after the 4096 generated ones, L = 512 + 8192 = 8704
        ck = bd.make_config(s)
        Lc = s.img_len
        ck.dims.img_len = s.img_len + Lc
        Xk = X.clone()
        Xc = torch.randn((s.batch, Lc, s.in_ch), generator=g, device=dev)
        idk = torch.from_numpy(np.concatenate([bd.mmdit_make_ids(s.grid_h, s.grid_w, s.txt_len),
                                               bd.mmdit_make_ids(s.grid_h, s.grid_w, 0, frame=1)])).to(dev)
        wsk = torch.empty(bd.mmdit_step_workspace(ck), dtype=torch.uint8, device=dev)

        def kstep(i):
            j = i % 4
            bd.mmdit_step_ex(ck, mc, Xk, v, T, y, idk, sig[j], sig[j + 1], wsk, ctx_packed=Xc, ctx_len=Lc)
        for i in range(2):
            kstep(i)
        kn = max(a.steps // 2, 3)
        kms = timed(kstep, kn)
        kfl = step_flops(dataclasses.replace(s, grid_w=2 * s.grid_w))
        out["kontext_step"] = {"ms_per_step": round(kms, 3), "seq_len": s.txt_len + 2 * s.img_len,
                               "context_tokens": Lc, "tflops": round(kfl / kms / 1e9, 1),
                               "frac_of_bf16_peak": round(kfl / kms / 1e9 / PEAK_BF16_TFLOPS, 4)}
        log(f"kontext step (L {s.txt_len + 2 * s.img_len}): {kms:.2f} ms ({kfl / kms / 1e9:.0f} TFLOP/s)")
        del wsk, Xk, Xc

        # guidance-distilled (dev) generation: the same blocks plus a guidance
        # embedder, 50 shifted steps at guidance 4.0, timed as one loop
        Gd = RI._Gen(44, dev)
        dt16 = torch.bfloat16
        M.guidance = [RI._linear(Gd, s.hidden, s.temb_dim, dt16), RI._linear(Gd, s.hidden, s.hidden, dt16)]
        keep = (M._dbl_arr, M._sgl_arr)  # mc's block arrays stay alive: M.c() builds new ones
        mdc = M.c()
        nd = 50
        sigd = bd.mmdit_schedule(nd, s.img_len)
        Xd = X.clone()
        bd.mmdit_step_ex(cfg, mdc, Xd, v, T, y, ids, sigd[0], sigd[1], ws, guidance=4.0)
        Xd.copy_(X)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(nd):
            bd.mmdit_step_ex(cfg, mdc, Xd, v, T, y, ids, sigd[i], sigd[i + 1], ws, guidance=4.0)
        torch.cuda.synchronize()
        dsec = time.perf_counter() - t1
        out["dev_generation"] = {"steps": nd, "guidance": 4.0, "seconds": round(dsec, 3),
                                 "ms_per_step": round(dsec * 1e3 / nd, 3)}
        log(f"dev generation: {nd} steps in {dsec:.2f} s ({dsec * 1e3 / nd:.2f} ms/step)")

        # the same generation with step caching: steps whose summed change of
        # the first block's modulated input stays below the threshold reuse
        # the block residual
        Xq = X.clone()
        cache = bd.StepCache(cfg)
        ran = 0
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(nd):
            bd.mmdit_step_ex(cfg, mdc, Xq, v, T, y, ids, sigd[i], sigd[i + 1], ws, guidance=4.0, cache=cache,
                             cache_threshold=a.cache_threshold)
            ran += int(cache.ran_blocks)
        torch.cuda.synchronize()
        csec = time.perf_counter() - t1
        drift = float((Xq - Xd).norm() / Xd.norm())
        out["cached_dev_generation"] = {"steps": nd, "threshold": a.cache_threshold, "steps_running_blocks": ran,
                                        "seconds": round(csec, 3), "speedup": round(dsec / csec, 3),
                                        "rel_l2_vs_uncached": round(drift, 5)}
        log(f"cached dev generation (threshold {a.cache_threshold}): {ran}/{nd} steps ran the blocks, "
            f"{csec:.2f} s ({dsec / csec:.2f}x), final latent rel-L2 {drift:.4f} vs uncached")
        M.guidance = None
        del Xd, Xq, mdc, keep, cache

    if not a.no_extras:
        out["vendor_reference"] = vendor_reference(s)
        log(f"vendor reference: {out['vendor_reference']}")

    if not a.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(s)
        log(f"  {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
