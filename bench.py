#!/usr/bin/env python3
"""Benchmark of the FLUX-style MMDiT denoising step on one MI355X.

Workload: one denoising step at 1024x1024 (64x64 patch grid = 4096 image
tokens, 512 text tokens, joint sequence 4608), 19 dual-stream + 38
single-stream blocks, hidden 3072, 24 heads x 128, MLP 12288, bf16 operands
with float32 accumulation, batch 1, random-init weights drawn on the GPU.
A step = conditioning vector, all modulations, input projections, the 57
blocks, the final layer and the fused Euler update (mmdit_step).

Prints ONE JSON line. `value` is the step latency in ms (lower is better).
Extra fields: every MFMA kernel class of the step (launches per step, average
launch time from HIP events on the library's stream, TFLOP/s, fraction of the
bf16 peak, share of the step); `roofline` for the class with the largest
share; the HBM-bound kernels in the step and alone (cold and warm Infinity
Cache); weight streaming of a quantised layer at 1 and 16 rows; HIP-graph
replay; block TFLOP/s (4608 tokens) and the configuration-2 block (1280
tokens); the bf16-residual, quantised, ternary, reference-image and guided
variants; the 4-step loop and the guided generation with the modulation
vectors of 4 timesteps computed in one pass; the cached guided generation
with the decision on the host, on the device, and replayed from HIP graphs;
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


def _profile_record(name):
    """A committed counter record profiles/<name>.json, or None when missing
    or when the kernel's sources have changed since the counters were taken
    (SHA-256 of the listed sources)."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    try:
        rec = json.load(open(os.path.join(here, "profiles", name + ".json")))
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(here, "diffusion_transformer_mmdit_amd", "csrc", src), "rb") as f:
                h.update(f.read())
        return rec if h.hexdigest() == rec["sources_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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
            "value_is": "extrapolated: the timed sample scaled to the full step's block count",
            "gflops": round(step_flops(s) / (est_ms * 1e-3) / 1e9, 1), "one_core": one_core,
            "sample": (f"numpy float32 oracle timed on 1 dual block ({t_dual:.2f} s) + 1 single block "
                       f"({t_single:.2f} s) at 4608 tokens; value = {s.n_double} x dual + {s.n_single} x single "
                       f"(the embedders and final layer, under 0.1% of the FLOPs, are not timed); BLAS "
                       f"{info[0].get('internal_api', '?') if info else '?'}, affinity "
                       f"{len(os.sched_getaffinity(0))} cores")}


def time_config2(dev, g, steps):
    """One dual block at 512x512 (256 text + 1024 image tokens, h 3072), two
    weight sets alternating (680 MB each), timed back to back."""
    import torch

    from diffusion_transformer_mmdit_amd import binding as bd
    from diffusion_transformer_mmdit_amd import inputs as I
    from diffusion_transformer_mmdit_amd import random_init as RI
    s2 = I.CFG2
    dims2 = bd.make_dims(s2)
    d2 = [RI.double_block(s2, 300 + i, dev) for i in range(2)]
    d2c = [d.c() for d in d2]
    img2 = torch.randn((1, s2.img_len, s2.hidden), generator=g, device=dev).to(torch.bfloat16)
    txt2 = torch.randn((1, s2.txt_len, s2.hidden), generator=g, device=dev).to(torch.bfloat16)
    vec2 = torch.randn((1, s2.hidden), generator=g, device=dev).to(torch.bfloat16)
    ids2 = torch.from_numpy(bd.mmdit_make_ids(s2.grid_h, s2.grid_w, s2.txt_len)).to(dev)
    ws2 = torch.empty(bd.mmdit_double_block_workspace(dims2), dtype=torch.uint8, device=dev)
    io2, to2 = torch.empty_like(img2), torch.empty_like(txt2)
    f2 = lambda i: bd.mmdit_double_block_fwd(dims2, d2c[i % 2], img2, txt2, io2, to2, vec2, ids2, ws2)  # noqa
    for i in range(4):
        f2(i)
    n = max(4 * steps, 16)
    torch.cuda.synchronize()
    t = time.perf_counter()
    for i in range(n):
        f2(i)
    torch.cuda.synchronize()
    c2ms = (time.perf_counter() - t) * 1e3 / n
    bf2 = block_flops(s2)
    log(f"config-2 dual block (1280 tokens): {c2ms:.4f} ms ({bf2 / c2ms / 1e9:.0f} TFLOP/s)")
    return {"ms": round(c2ms, 4), "tflops": round(bf2 / c2ms / 1e9, 1),
            "frac": round(bf2 / c2ms / 1e9 / PEAK_BF16_TFLOPS, 4),
            "block_fwd_per_s": round(1e3 / c2ms, 1), "flops": bf2, "tokens": s2.seq_len}


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
    ap.add_argument("--config2-only", action="store_true",
                    help="time only the 1280-token dual block and print its figures as the JSON line")
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
    if a.config2_only:
        r = time_config2(dev, torch.Generator(device=dev).manual_seed(7), a.steps)
        print(json.dumps({"metric": "dual_block_ms_1280_tokens", "value": r["ms"], "unit": "ms",
                          "higher_is_better": False, "dtype": "bf16", "data": "synthetic", "config2": r}))
        return
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
    # the same loop with the modulation vectors of its 4 timesteps computed in
    # one pass over the modulation weights (mmdit_step_modulations), inside
    # the timed region; the final latent must equal the plain loop's
    mods4 = torch.empty(bd.mmdit_step_modulations_bytes(cfg, 4), dtype=torch.uint8, device=dev)
    x_plain = X.clone()

    def loop4_shared(_):
        X.copy_(X0)
        bd.mmdit_step_modulations(cfg, mc, y, sig[:4], mods4)
        for j in range(4):
            bd.mmdit_step_ex(cfg, mc, X, v, T, None, ids, sig[j], sig[j + 1], ws, mods=mods4, mods_count=4,
                             mods_index=j)
    loop4_shared(0)
    torch.cuda.synchronize()
    same = bool(torch.equal(X, x_plain))
    loop_shared_ms = timed(loop4_shared, max(2, a.steps // 4))
    log(f"4-step loop, modulations shared: {loop_shared_ms:.2f} ms (final latent equal to the plain loop's: {same})")
    del mods4, x_plain
    flops = step_flops(s)

    # every MFMA-bound kernel class of the step, timed with HIP events around
    # each launch on the library's stream (mmdit_profile_begin/end)
    kdesc = {
        "gemm_res": ("k_gemm_dma<2> gated-residual epilogue: out-projection (K 3072), fc2 (K 12288), linear2 "
                     "(K 15360); N 3072, M 4608", bd.PC_GEMM_RES),
        "gemm_lin1": ("k_gemm_dma<6> single-block linear1, split GELU + fused QK RMSNorm/RoPE epilogue; "
                      "M 4608 N 21504 K 3072", bd.PC_GEMM_LIN1),
        "attention": ("k_attn_bf16 joint flash attention, 24 heads x 4608 tokens", bd.PC_ATTN),
        "gemm_fc1": ("k_gemm_dma<1> dual-block fc1, GELU epilogue; M 512+4096 N 12288 K 3072", bd.PC_GEMM_FC1),
        "gemm_qkv": ("k_gemm_dma<5> dual-block QKV, fused QK RMSNorm/RoPE epilogue; M 512+4096 N 9216 K 3072",
                     bd.PC_GEMM_QKV),
    }
    prof = {}
    for name, (desc, cls) in kdesc.items():
        bd.mmdit_profile_begin(cls, 400 * max(1, a.steps))
        for i in range(a.steps):
            step(i)
        tot_ms, n, work = bd.mmdit_profile_end()
        tf = work / max(tot_ms, 1e-9) / 1e9
        prof[name] = {"kernel": desc, "launches_per_step": n // max(a.steps, 1),
                      "avg_us": round(1e3 * tot_ms / max(n, 1), 2), "tflops": round(tf, 1),
                      "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                      "flops_per_launch": work / max(n, 1),
                      "ms_per_step": round(tot_ms / max(a.steps, 1), 3),
                      "share_of_step": round(tot_ms / max(a.steps, 1) / ms, 4)}
        log(f"{name}: {prof[name]['launches_per_step']}/step, avg {prof[name]['avg_us']:.1f} us, "
            f"{tf:.1f} TFLOP/s ({prof[name]['frac']:.3f}), {100 * prof[name]['share_of_step']:.1f}% of the step")
    # HBM-bound kernels inside the step: algorithmic bytes. The modulation
    # GEMVs stream 6.49 GB of weights per step (25x the 256 MB Infinity
    # Cache), so their in-step rate is a cold-cache rate; the LayerNorm reads
    # a residual the previous GEMM has just written (warm) and is also timed
    # cold below.
    mem = {}
    for name, cls in (("layernorm_in_step", bd.PC_LN), ("gemv_in_step", bd.PC_GEMV)):
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
    # the roofline line names the MFMA kernel class with the largest share of the step
    dom = max(prof, key=lambda k: prof[k]["share_of_step"])
    p = prof[dom]
    rec = _profile_record(f"{dom}_traffic")
    roofline = {"bound": "mfma", "kernel": p["kernel"], "class": dom, "achieved": p["tflops"],
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": p["frac"],
                "traffic": int(rec["traffic_bytes_per_launch"]) if rec else None,
                "avg_launch_us": p["avg_us"], "flops_per_launch": p["flops_per_launch"],
                "share_of_step": p["share_of_step"]}
    clk = _profile_record(f"{dom}_clock")
    if clk:
        pk = PEAK_BF16_TFLOPS * float(clk["clock_ghz"]) / float(clk["max_clock_ghz"])
        roofline.update({"clock_ghz_measured": float(clk["clock_ghz"]), "peak_at_measured_clock": round(pk, 1),
                         "frac_at_measured_clock": round(p["tflops"] / pk, 4)})

    out = {"metric": METRIC, "value": round(ms, 3), "unit": "ms", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": round(ms, 3), "higher_is_better": False, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded random-init weights and inputs)",
           "config": {"workload": "FLUX-style MMDiT denoising step at 1024x1024: 19 dual + 38 single blocks, "
                                  "hidden 3072, 24x128 heads, MLP 12288, 4096 image + 512 text tokens, batch 1",
                      "global_batch": 1, "seq_len": s.seq_len, "image_tokens": s.img_len, "text_tokens": s.txt_len,
                      "parallelism": "single GPU"},
           "step_spread_ms": spread, "loop_4_steps_ms": round(loop_ms, 3),
           "loop_4_steps_shared_modulations": {"ms": round(loop_shared_ms, 3), "final_latent_identical": same},
           "device": {"name": torch.cuda.get_device_name(0), "hip": torch.version.hip,
                      "torch": torch.__version__},
           "step_tflops": round(flops / ms / 1e9, 1),
           "step_frac_of_bf16_peak": round(flops / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
           "roofline": roofline,
           "kernels": {k: {kk: vv for kk, vv in v_.items() if kk != "flops_per_launch"} for k, v_ in prof.items()},
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
        del dbl, sgl, dblc, sglc, wsb

        out["config2_dual_block"] = time_config2(dev, g, a.steps)

        # the step with its residual stream held in bf16 (dims.resid)
        cfg16 = bd.make_config(s, resid=bd.RESID_BF16)
        ws16 = torch.empty(bd.mmdit_step_workspace(cfg16), dtype=torch.uint8, device=dev)
        X16 = X.clone()
        st16 = lambda i: bd.mmdit_step(cfg16, mc, X16, v, T, y, ids, sig[i % 4], sig[i % 4 + 1], ws16)  # noqa
        for i in range(2):
            st16(i)
        out["bf16_residual_ms_per_step"] = round(timed(st16, a.steps), 3)
        log(f"bf16-residual step: {out['bf16_residual_ms_per_step']:.2f} ms")
        del ws16, X16

        # HBM-bound kernels alone, cold and warm. Cold: a pass that reads a
        # 512 MB buffer evicts the 256 MB Infinity Cache before each call (a
        # write pass would leave dirty lines whose write-back then overlaps
        # the timed call); warm: the call repeated on the same buffers. All
        # calls of a measurement are enqueued back to back (arguments
        # marshalled once, raw C calls) before one synchronisation, so that
        # no start event waits for the host.
        import ctypes as C
        evict = torch.ones(128 << 20, dtype=torch.float32, device=dev)
        evict_sink = torch.empty((), dtype=torch.float32, device=dev)
        stream_h = C.c_void_p(torch.cuda.current_stream().cuda_stream)

        def evict_pass():
            torch.sum(evict, dim=0, out=evict_sink)

        def kernel_times(calls, pre=None):
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in calls]
            evict.fill_(7)  # head start: the GPU is busy while the host enqueues
            sts = []
            for (e0, e1), c in zip(ev, calls):
                if pre is not None:
                    pre()
                e0.record()
                sts.append(c())
                e1.record()
            torch.cuda.synchronize()
            assert all(st == 0 for st in sts), sts
            return [e0.elapsed_time(e1) for e0, e1 in ev]

        def rate(ts, nbytes):
            t = float(np.median(ts))
            return {"us": round(1e3 * t, 2), "gbps": round(nbytes / t / 1e6, 1),
                    "frac": round(nbytes / t / 1e6 / PEAK_HBM_GBS, 4)}

        def cold_warm(call, nbytes, n=12):
            call()
            return {"cold": rate(kernel_times([call] * n, pre=evict_pass), nbytes),
                    "warm": rate(kernel_times([call] * n), nbytes), "bytes": int(nbytes)}
        hbm = {}
        rows, h = s.seq_len, s.hidden
        xl = torch.randn((rows, h), generator=g, device=dev)
        yl = torch.empty((rows, h), dtype=torch.bfloat16, device=dev)
        modl = torch.randn((2, h), generator=g, device=dev) * 0.3
        f_ln = bd.lib().mmdit_adaln_layernorm
        ln_args = (xl.data_ptr(), 1, yl.data_ptr(), bd.BF16, rows, h, modl.data_ptr(), C.c_float(1e-6), stream_h)
        hbm["layernorm"] = cold_warm(lambda: f_ln(*ln_args), rows * h * 6)
        hbm["layernorm"]["shape"] = f"{rows} x {h}, float32 in, bf16 out"
        del xl, yl
        qd = RI._linear(RI._Gen(47, dev), 3 * h + s.mlp_hidden, h, torch.bfloat16, 4)
        wd = torch.empty((qd.n_out, qd.k_in), dtype=torch.bfloat16, device=dev)
        nq = qd.n_out * qd.k_in
        f_dq = bd.lib().mmdit_dequantise
        dq_args = (qd.w.data_ptr(), qd.scales.data_ptr(), bd.W_Q4G64, qd.n_out, qd.k_in, wd.data_ptr(), stream_h)
        hbm["dequant_q4"] = cold_warm(lambda: f_dq(*dq_args), nq * 0.5 + nq / 64 * 2 + nq * 2)
        hbm["dequant_q4"]["shape"] = f"{qd.n_out} x {qd.k_in} 4-bit codes -> bf16"
        del qd, wd
        out["hbm_alone"] = hbm
        log(f"HBM kernels alone: {hbm}")

        f_lin = bd.lib().mmdit_linear_fwd

        def lin_call(lin, xm, ym, route, ws=None):
            lc = lin.c()
            args = (C.byref(lc), bd.BF16, xm.data_ptr(), xm.shape[0], ym.data_ptr(),
                    int(ym.dtype == torch.float32), route, None if ws is None else ws.data_ptr(),
                    0 if ws is None else ws.numel(), stream_h)
            return lambda: f_lin(*args) if lc is not None else -1

        # weight streaming: one linear layer (linear1's shape, 21504 x 3072)
        # at 1 and 16 rows, every format, on the weight-streaming route; the
        # calls cycle through enough copies of the layer (>= 512 MB) that each
        # reads its weights from HBM. GB/s counts codes + scales.
        n_out, k_in = 3 * h + s.mlp_hidden, h
        stream = {}
        wbytes = {0: 2.0, 4: 0.5 + 2 / 64, 8: 1.0 + 2 / 64, 1: 0.125 + 2 / 128, 2: 0.25 + 2 / 128}
        for fname, bits in (("dense", 0), ("q4g64", 4), ("q8g64", 8), ("q1g128", 1), ("tq2g128", 2)):
            per = n_out * k_in * wbytes[bits]
            copies = max(2, int(np.ceil((512 << 20) / per)))
            G = RI._Gen(50 + bits, dev)
            pool = [RI._linear(G, n_out, k_in, torch.bfloat16, bits) for _ in range(copies)]
            stream[fname] = {"weight_bytes": int(per), "copies": copies}
            for rows_m in (1, 16):
                xm = torch.randn((rows_m, k_in), generator=g, device=dev).to(torch.bfloat16)
                ym = torch.empty((rows_m, n_out), dtype=torch.float32, device=dev)
                calls = [lin_call(pool[i % copies], xm, ym, bd.ROUTE_STREAM) for i in range(4 * copies)]
                kernel_times(calls[:copies])
                stream[fname][f"M{rows_m}"] = rate(kernel_times(calls)[copies:], per)
            del pool
            # one layer 8x as wide (172032 x 3072): the per-launch start-up,
            # a few microseconds, weighs less against the weight bytes
            G = RI._Gen(70 + bits, dev)
            big = [RI._linear(G, 8 * n_out, k_in, torch.bfloat16, bits) for _ in range(max(2, copies // 8))]
            xm = torch.randn((1, k_in), generator=g, device=dev).to(torch.bfloat16)
            ym = torch.empty((1, 8 * n_out), dtype=torch.float32, device=dev)
            calls = [lin_call(big[i % len(big)], xm, ym, bd.ROUTE_STREAM) for i in range(4 * len(big))]
            kernel_times(calls[:len(big)])
            stream[fname]["M1_8x_wide"] = rate(kernel_times(calls)[len(big):], 8 * per)
            del big
        out["weight_streaming"] = stream
        log(f"weight streaming (21504 x 3072): {stream}")

        # routes of a 4-bit layer (linear1's shape) against the row count:
        # weight streaming (M <= 16), dequantisation inside the tiled GEMM,
        # and decoding the layer once to bf16 before the dense GEMM
        G = RI._Gen(60, dev)
        lq = RI._linear(G, n_out, k_in, torch.bfloat16, 4)
        wsr = torch.empty(bd.mmdit_linear_workspace(lq, bd.BF16, 4608, bd.ROUTE_DECODE), dtype=torch.uint8,
                          device=dev)
        routes = {}
        for rows_m in (1, 16, 256, 1024, 4608):
            xm = torch.randn((rows_m, k_in), generator=g, device=dev).to(torch.bfloat16)
            ym = torch.empty((rows_m, n_out), dtype=torch.bfloat16, device=dev)
            r = {}
            for rname, rt in (("stream", bd.ROUTE_STREAM), ("tiled", bd.ROUTE_TILED), ("decode", bd.ROUTE_DECODE)):
                if rt == bd.ROUTE_STREAM and rows_m > 16:
                    continue
                c = lin_call(lq, xm, ym, rt, wsr)
                c()
                r[rname + "_us"] = round(1e3 * float(np.median(kernel_times([c] * 8, pre=evict_pass))), 2)
            routes[f"M{rows_m}"] = r
        out["q4_routes_vs_rows"] = routes
        log(f"4-bit routes against rows (cold): {routes}")
        del lq, wsr, evict

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

        # the same generation with the modulation vectors of each group of 4
        # timesteps computed in one pass over the modulation weights
        mods4 = torch.empty(bd.mmdit_step_modulations_bytes(cfg, 4), dtype=torch.uint8, device=dev)
        Xm = X.clone()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i0 in range(0, nd, 4):
            cnt = min(4, nd - i0)
            bd.mmdit_step_modulations(cfg, mdc, y, sigd[i0:i0 + cnt], mods4, guidance=4.0)
            for j in range(cnt):
                bd.mmdit_step_ex(cfg, mdc, Xm, v, T, None, ids, sigd[i0 + j], sigd[i0 + j + 1], ws, mods=mods4,
                                 mods_count=cnt, mods_index=j)
        torch.cuda.synchronize()
        msec = time.perf_counter() - t1
        out["dev_generation_shared_modulations"] = {
            "seconds": round(msec, 3), "ms_per_step": round(msec * 1e3 / nd, 3),
            "final_latent_identical": bool(torch.equal(Xm, Xd))}
        log(f"dev generation, modulations shared by groups of 4 steps: {msec:.2f} s, "
            f"same latent {torch.equal(Xm, Xd)}")
        del Xm, mods4

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

        # decided on the device (no wait per step; a reused step still
        # enqueues the blocks' launches, which return at once), eagerly and
        # replayed from HIP graphs (one per schedule position after the first)
        def dev_cached(replay=None):
            Xe = X.clone()
            ce = bd.StepCache(cfg, on_device=True)
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for i in range(nd):
                if replay is None or i == 0:
                    bd.mmdit_step_ex(cfg, mdc, Xe, v, T, y, ids, sigd[i], sigd[i + 1], ws, guidance=4.0,
                                     cache=ce, cache_threshold=a.cache_threshold)
                else:
                    replay[i - 1].replay()
            torch.cuda.synchronize()
            return time.perf_counter() - t1, Xe, ce

        esec, Xe, ce = dev_cached()
        out["cached_dev_generation_device"] = {
            "seconds": round(esec, 3), "speedup": round(dsec / esec, 3),
            "bit_identical_to_host_decision": bool(torch.equal(Xe, Xq))}
        log(f"cached dev generation, device decision: {esec:.2f} s, same latent {torch.equal(Xe, Xq)}")
        try:
            # capture with the cache of a started generation; each replay
            # continues the generation whose first step ran eagerly
            Xe.copy_(X)
            Xg = Xe
            cg = ce
            cg.reset()
            bd.mmdit_step_ex(cfg, mdc, Xg, v, T, y, ids, sigd[0], sigd[1], ws, guidance=4.0, cache=cg,
                             cache_threshold=a.cache_threshold)
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            graphs = []
            for i in range(1, nd):
                gr = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gr, stream=cap):
                    bd.mmdit_step_ex(cfg, mdc, Xg, v, T, y, ids, sigd[i], sigd[i + 1], ws, guidance=4.0,
                                     cache=cg, cache_threshold=a.cache_threshold)
                graphs.append(gr)
            torch.cuda.synchronize()
            Xg.copy_(X)
            cg.reset()
            # the eager first step inside the timing starts the generation
            t1 = time.perf_counter()
            bd.mmdit_step_ex(cfg, mdc, Xg, v, T, y, ids, sigd[0], sigd[1], ws, guidance=4.0, cache=cg,
                             cache_threshold=a.cache_threshold)
            for gr in graphs:
                gr.replay()
            torch.cuda.synchronize()
            gsec = time.perf_counter() - t1
            out["cached_dev_generation_graph"] = {
                "seconds": round(gsec, 3), "speedup": round(dsec / gsec, 3),
                "bit_identical_to_host_decision": bool(torch.equal(Xg, Xq))}
            log(f"cached dev generation from graphs: {gsec:.2f} s, same latent {torch.equal(Xg, Xq)}")
            del graphs
        except Exception as e:  # report, do not hide the main number
            out["cached_dev_generation_graph"] = {"error": str(e)[:200]}
        M.guidance = None
        del Xd, Xq, Xe, mdc, keep, cache, ce

    if not a.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        out["cpu_baseline"] = cpu_baseline(s)
        log(f"  {out['cpu_baseline']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
