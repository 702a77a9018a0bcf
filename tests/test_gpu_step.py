"""GPU parity of the denoising step (mmdit_step) and of the packing / RoPE
helpers against the CPU oracle."""
import dataclasses

import numpy as np
import pytest

import oracle
from diffusion_transformer_mmdit_amd import binding as bd
from diffusion_transformer_mmdit_amd import inputs as I
from tests.gpu_util import assert_parity, down, dtype_code, rel_l2, sync, torch, up, up_i32, workspace

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------- helpers ------
def test_pack_unpack_bit_exact():
    t = torch()
    rng = np.random.default_rng(3)
    for nbytes, npdt, tdt in ((4, np.uint32, t.int32), (2, np.uint16, t.int16)):
        z = rng.integers(0, 2 ** (8 * nbytes), size=(2, 16, 128, 96), dtype=np.uint64).astype(npdt)
        zd = t.from_numpy(z.view(np.int32 if nbytes == 4 else np.int16)).cuda()
        xd = t.empty((2, 64 * 48, 64), dtype=tdt, device="cuda")
        print(f"pack elem_bytes={nbytes}", flush=True)
        bd.mmdit_pack_latents(zd, xd)
        back = t.empty_like(zd)
        bd.mmdit_unpack_latents(xd, back)
        sync()
        X = xd.cpu().numpy().view(npdt)
        assert np.array_equal(X, oracle.pack_latents(z))
        assert np.array_equal(back.cpu().numpy().view(npdt), z)


def test_rope_table_matches_oracle():
    t = torch()
    ids = oracle.make_ids(64, 64, 512, frame=3)
    ids[:512, 1] = np.arange(512)
    tab = t.empty((ids.shape[0], 64, 2), dtype=t.float32, device="cuda")
    bd.mmdit_rope_table(up_i32(ids), (16, 56, 56), 10000.0, tab)
    sync()
    cos, sin = oracle.rope_table(ids)
    got = tab.cpu().numpy()
    err = max(np.abs(got[..., 0] - cos).max(), np.abs(got[..., 1] - sin).max())
    print(f"rope table max abs err {err:.2e}, exact {np.mean(got[..., 0] == cos):.4f}", flush=True)
    assert err <= 2e-6


# ---------------------------------------------------------------- step -------
def model_numpy(s: I.Shape):
    g = I.global_weights(s)
    dbl = [I.double_block_weights(s, i) for i in range(s.n_double)]
    sgl = [I.single_block_weights(s, i) for i in range(s.n_single)]
    return g, dbl, sgl


def run_step(s: I.Shape, g, dbl, sgl, inp, sig_i: int, n_steps: int = 4, quant=None, repeat: int = 1,
             dequant_in_gemm: bool = False):
    t = torch()
    dt = dtype_code(s.dtype)
    cfg = bd.make_config(s)
    M = bd.ModelW(g, [bd.DoubleW(d, dt, "cuda", quant) for d in dbl],
                  [bd.SingleW(w, dt, "cuda", quant) for w in sgl], dt, "cuda")
    mc = M.c()
    z = t.from_numpy(inp["z"]).cuda()
    X = t.empty((s.batch, s.img_len, s.in_ch), dtype=t.float32, device="cuda")
    bd.mmdit_pack_latents(z, X)
    ids = up_i32(bd.mmdit_make_ids(s.grid_h, s.grid_w, s.txt_len))
    sig = bd.mmdit_schedule(n_steps, s.img_len)
    T = up(inp["T"], s.dtype)
    y = up(inp["y"], s.dtype)
    v = t.empty_like(X)
    ws = workspace(bd.mmdit_step_workspace(cfg))
    outs = []
    for _ in range(repeat):
        Xr = X.clone()
        print(f"step B={s.batch} h={s.hidden} {s.n_double}+{s.n_single} blocks L={s.seq_len} {s.dtype} "
              f"sigma {sig[sig_i]:.4f}->{sig[sig_i + 1]:.4f}", flush=True)
        if dequant_in_gemm:
            bd.mmdit_step_ex(cfg, mc, Xr, v, T, y, ids, sig[sig_i], sig[sig_i + 1], ws, dequant_in_gemm=True)
        else:
            bd.mmdit_step(cfg, mc, Xr, v, T, y, ids, sig[sig_i], sig[sig_i + 1], ws)
        sync()
        outs.append((down(Xr), down(v)))
    return outs if repeat > 1 else outs[0]


def oracle_step(s: I.Shape, g, dbl, sgl, inp, sig_i: int, n_steps: int = 4):
    X = oracle.pack_latents(inp["z"])
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    sig = oracle.schedule(n_steps, s.img_len)
    return oracle.step(g, dbl, sgl, X, inp["T"], inp["y"], ids, sig[sig_i], sig[sig_i + 1], s.heads,
                       s.axes_dim, s.theta)


TINY_F32 = I.Shape(hidden=256, heads=2, mlp_hidden=512, txt_len=16, grid_h=8, grid_w=8, dtype="f32",
                   cfg_id=41, n_double=2, n_single=2, txt_in_dim=256, vec_in_dim=256)


@pytest.mark.parametrize("sig_i", [0, 3])
def test_step_f32_tiny(sig_i):
    s = TINY_F32
    g, dbl, sgl = model_numpy(s)
    inp = I.step_inputs(s)
    Xg, vg = run_step(s, g, dbl, sgl, inp, sig_i)
    Xr, vr = oracle_step(s, g, dbl, sgl, inp, sig_i)
    assert_parity(vg, vr, "f32", "step v")
    assert_parity(Xg, Xr, "f32", "step x_next")


def test_step_f32_batch2_no_text():
    s = dataclasses.replace(TINY_F32, batch=2, txt_len=0, grid_h=6, grid_w=10, cfg_id=42)
    g, dbl, sgl = model_numpy(s)
    inp = I.step_inputs(s)
    Xg, vg = run_step(s, g, dbl, sgl, inp, 1)
    Xr, vr = oracle_step(s, g, dbl, sgl, inp, 1)
    assert_parity(vg, vr, "f32", "step v (B=2, Lt=0)")


def test_step_f32_batch2_ragged():
    s = dataclasses.replace(TINY_F32, batch=2, txt_len=21, grid_h=5, grid_w=9, cfg_id=43)
    g, dbl, sgl = model_numpy(s)
    inp = I.step_inputs(s)
    _, vg = run_step(s, g, dbl, sgl, inp, 2)
    _, vr = oracle_step(s, g, dbl, sgl, inp, 2)
    assert_parity(vg, vr, "f32", "step v (B=2 ragged)")


def test_step_bf16_full_tokens_two_plus_two_blocks():
    # 1024^2 workload (4096 image + 512 text tokens, h 3072) at depth 2 + 2
    s = dataclasses.replace(I.CFG4, n_double=2, n_single=2)
    g, dbl, sgl = model_numpy(s)
    inp = I.step_inputs(s)
    Xg, vg = run_step(s, g, dbl, sgl, inp, 0)
    Xr, vr = oracle_step(s, g, dbl, sgl, inp, 0)
    assert_parity(vg, vr, "bf16", "bf16 step v")
    assert_parity(Xg, Xr, "bf16", "bf16 step x_next")


def ctx_ids(s: I.Shape, cgh: int, cgw: int) -> np.ndarray:
    """[txt; generated (frame 0); context (frame 1)] ids."""
    return np.concatenate([oracle.make_ids(s.grid_h, s.grid_w, s.txt_len),
                           oracle.make_ids(cgh, cgw, 0, frame=1)]).astype(np.int32)


def run_step_ex(s: I.Shape, cgh: int, cgw: int, sig_i: int, guidance=None, n_steps: int = 4):
    """mmdit_step_ex with a context latent of cgh x cgw packed tokens (none
    when 0) and an optional guidance value (the model then has a guidance
    embedder) against the oracle step with the same options."""
    t = torch()
    g, dbl, sgl = model_numpy(s)
    if guidance is not None:
        g = dict(g, **I.guidance_weights(s))
    inp = I.step_inputs(s)
    Lc = cgh * cgw
    Xc = np.random.default_rng(1000 + s.cfg_id).standard_normal((s.batch, Lc, s.in_ch)).astype(np.float32)
    ids = ctx_ids(s, cgh, cgw) if Lc else oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    sig = oracle.schedule(n_steps, s.img_len)
    dt = dtype_code(s.dtype)
    cfg = bd.make_config(s)
    cfg.dims.img_len = s.img_len + Lc
    M = bd.ModelW(g, [bd.DoubleW(d, dt, "cuda") for d in dbl], [bd.SingleW(w, dt, "cuda") for w in sgl], dt, "cuda")
    z = t.from_numpy(inp["z"]).cuda()
    X = t.empty((s.batch, s.img_len, s.in_ch), dtype=t.float32, device="cuda")
    bd.mmdit_pack_latents(z, X)
    v = t.empty_like(X)
    ws = workspace(bd.mmdit_step_workspace(cfg))
    print(f"step_ex B={s.batch} h={s.hidden} {s.n_double}+{s.n_single} blocks Lt={s.txt_len} Lg={s.img_len} "
          f"Lc={Lc} guidance={guidance} {s.dtype}", flush=True)
    bd.mmdit_step_ex(cfg, M.c(), X, v, up(inp["T"], s.dtype), up(inp["y"], s.dtype), up_i32(ids), sig[sig_i],
                     sig[sig_i + 1], ws, ctx_packed=t.from_numpy(Xc).cuda() if Lc else None, ctx_len=Lc,
                     guidance=guidance)
    sync()
    Xr, vr = oracle.step(g, dbl, sgl, oracle.pack_latents(inp["z"]), inp["T"], inp["y"], ids, sig[sig_i],
                         sig[sig_i + 1], s.heads, s.axes_dim, s.theta, Xc=Xc if Lc else None, guidance=guidance)
    return (down(X), down(v)), (Xr, vr)


def test_step_ctx_f32_tiny_batch2():
    s = dataclasses.replace(TINY_F32, batch=2, txt_len=11, grid_h=6, grid_w=5, cfg_id=45)
    (Xg, vg), (Xr, vr) = run_step_ex(s, 4, 7, 1)
    assert_parity(vg, vr, "f32", "step_ctx v")
    assert_parity(Xg, Xr, "f32", "step_ctx x_next")


def test_step_ctx_bf16_width3072():
    # h 3072 / 24 heads, 256 text + 32x32 generated + 32x32 context tokens
    s = dataclasses.replace(I.CFG4, n_double=1, n_single=1, txt_len=256, grid_h=32, grid_w=32, cfg_id=46)
    (Xg, vg), (Xr, vr) = run_step_ex(s, 32, 32, 0)
    assert_parity(vg, vr, "bf16", "bf16 step_ctx v")
    assert_parity(Xg, Xr, "bf16", "bf16 step_ctx x_next")


def test_step_guidance_f32_tiny():
    s = dataclasses.replace(TINY_F32, txt_len=9, grid_h=5, grid_w=7, cfg_id=47)
    (Xg, vg), (Xr, vr) = run_step_ex(s, 0, 0, 2, guidance=3.5)
    assert_parity(vg, vr, "f32", "guided step v")
    assert_parity(Xg, Xr, "f32", "guided step x_next")


def test_step_guidance_with_context_bf16_width3072():
    # guidance plus reference-image tokens (instruction editing with a
    # guidance-distilled model), h 3072, 128 + 24x24 generated + 24x24 context
    s = dataclasses.replace(I.CFG4, n_double=1, n_single=1, txt_len=128, grid_h=24, grid_w=24, cfg_id=48)
    (Xg, vg), (Xr, vr) = run_step_ex(s, 24, 24, 1, guidance=2.5)
    assert_parity(vg, vr, "bf16", "bf16 guided step_ex v")
    assert_parity(Xg, Xr, "bf16", "bf16 guided step_ex x_next")


# ----------------------------------------------------------- step caching ---
def cached_oracle(s, g, dbl, sgl, inp, ids, sig, thr, Xc=None):
    """oracle.step_cached over the schedule: (X, v, ran_blocks, rel, acc) per step."""
    st = oracle.new_cache_state()
    X = oracle.pack_latents(inp["z"])
    out = []
    for i in range(len(sig) - 1):
        X, v, run, rel = oracle.step_cached(g, dbl, sgl, X, inp["T"], inp["y"], ids, sig[i], sig[i + 1], s.heads,
                                            st, thr, s.axes_dim, s.theta, Xc=Xc)
        out.append((X, v, run, rel, st["acc"]))
    return out


def cached_gpu(s, g, dbl, sgl, inp, ids, sig, thr, Xc=None, mode="host"):
    """mmdit_step_ex with a step cache over the schedule, same tuple per step.

    mode "host": the host decides (the state is in the struct after each
    call); "device": a kernel decides, read back with mmdit_step_cache_read;
    "graph": the first step eager, the others captured into HIP graphs (one
    per schedule position) and replayed, the whole generation twice, with
    eager work and synchronisations between the replays: both passes must
    agree bit for bit."""
    t = torch()
    dt = dtype_code(s.dtype)
    Lc = 0 if Xc is None else Xc.shape[1]
    cfg = bd.make_config(s)
    cfg.dims.img_len = s.img_len + Lc
    M = bd.ModelW(g, [bd.DoubleW(d, dt, "cuda") for d in dbl], [bd.SingleW(w, dt, "cuda") for w in sgl], dt, "cuda")
    mc = M.c()
    z = t.from_numpy(inp["z"]).cuda()
    X0 = t.empty((s.batch, s.img_len, s.in_ch), dtype=t.float32, device="cuda")
    bd.mmdit_pack_latents(z, X0)
    X = X0.clone()
    v = t.empty_like(X)
    T, y, ids_d = up(inp["T"], s.dtype), up(inp["y"], s.dtype), up_i32(ids)
    xc = None if Xc is None else t.from_numpy(Xc).cuda()
    ws = workspace(bd.mmdit_step_workspace(cfg))
    cache = bd.StepCache(cfg, on_device=mode != "host")

    def step(i):
        bd.mmdit_step_ex(cfg, mc, X, v, T, y, ids_d, sig[i], sig[i + 1], ws, ctx_packed=xc, ctx_len=Lc,
                         cache=cache, cache_threshold=thr)

    def record():
        sync()
        if mode != "host":
            cache.read()
        return (down(X), down(v), cache.ran_blocks, cache.rel, cache.c.acc)

    tag = f"B={s.batch} h={s.hidden} Lt={s.txt_len} Lg={s.img_len} Lc={Lc} {s.dtype} threshold {thr:.4g} {mode}"
    if mode != "graph":
        out = []
        for i in range(len(sig) - 1):
            print(f"cached step {i} {tag}", flush=True)
            step(i)
            out.append(record())
        return out
    print(f"cached step 0 (eager) {tag}", flush=True)
    step(0)
    sync()
    graphs = []
    cap = t.cuda.Stream()
    cap.wait_stream(t.cuda.current_stream())
    for i in range(1, len(sig) - 1):
        print(f"capturing cached step {i}", flush=True)
        gr = t.cuda.CUDAGraph()
        with t.cuda.graph(gr, stream=cap):
            step(i)
        graphs.append(gr)
    sync()
    passes = []
    for k in range(2):
        X.copy_(X0)
        v.fill_(float("nan"))
        cache.reset()
        print(f"pass {k}: cached step 0 (eager)", flush=True)
        step(0)
        out = [record()]
        for i, gr in enumerate(graphs, 1):
            print(f"pass {k}: replay of cached step {i}", flush=True)
            gr.replay()
            out.append(record())
        passes.append(out)
    for a, b in zip(*passes):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2:] == b[2:]
    return passes[1]


def check_cached(s, cgh=0, cgw=0, n_steps=5, rel_tol=1e-4):
    g, dbl, sgl = model_numpy(s)
    inp = I.step_inputs(s)
    Lc = cgh * cgw
    Xc = np.random.default_rng(2000 + s.cfg_id).standard_normal((s.batch, Lc, s.in_ch)).astype(np.float32) if Lc else None
    ids = ctx_ids(s, cgh, cgw) if Lc else oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    sig = oracle.schedule(n_steps, s.img_len)
    # threshold between the second step's change and the sum of the second
    # and third steps' changes (never-recompute trajectory): the second step
    # reuses the residual, the third runs the blocks again
    ref_inf = cached_oracle(s, g, dbl, sgl, inp, ids, sig[:4], np.inf, Xc)
    thr = ref_inf[1][3] + 0.5 * ref_inf[2][3]
    ref = cached_oracle(s, g, dbl, sgl, inp, ids, sig, thr, Xc)
    runs = [r[2] for r in ref]
    assert runs[:3] == [True, False, True], runs
    prev_acc = 0.0
    for i, r in enumerate(ref):  # every decision clear of the threshold
        if i > 0:
            assert abs(prev_acc + r[3] - thr) > 0.02 * thr, (i, prev_acc + r[3], thr)
        prev_acc = r[4]
    got = cached_gpu(s, g, dbl, sgl, inp, ids, sig, thr, Xc)
    assert [r[2] for r in got] == runs
    for i, (a, b) in enumerate(zip(got, ref)):
        assert abs(a[3] - b[3]) <= rel_tol * max(b[3], 1e-30), (i, a[3], b[3])
        assert abs(a[4] - b[4]) <= rel_tol * max(b[4], 1e-30) or a[4] == b[4] == 0.0, (i, a[4], b[4])
        assert_parity(a[1], b[1], s.dtype, f"cached step {i} v (ran blocks {b[2]})")
        assert_parity(a[0], b[0], s.dtype, f"cached step {i} x_next")
    # the decision taken on the device, eagerly and from HIP graphs: the same
    # decisions, and the same kernels on the same data, so x and v bit for
    # bit those of the host decision (rel and acc summed in another order)
    for mode in ("device", "graph"):
        dv = cached_gpu(s, g, dbl, sgl, inp, ids, sig, thr, Xc, mode=mode)
        for i, (a, b) in enumerate(zip(dv, got)):
            assert a[2] == b[2], (mode, i, a[2], b[2])
            assert abs(a[3] - b[3]) <= 1e-9 * max(b[3], 1e-30), (mode, i, a[3], b[3])
            assert abs(a[4] - b[4]) <= 1e-9 * max(b[4], 1e-30) or a[4] == b[4] == 0.0, (mode, i, a[4], b[4])
            assert np.array_equal(a[1], b[1]), f"{mode} step {i}: v differs from the host decision's"
            assert np.array_equal(a[0], b[0]), f"{mode} step {i}: x differs from the host decision's"


def test_step_cache_f32_tiny_batch2():
    check_cached(dataclasses.replace(TINY_F32, batch=2, txt_len=11, grid_h=6, grid_w=5, cfg_id=49))


def test_step_cache_bf16_width3072_with_context():
    s = dataclasses.replace(I.CFG4, n_double=1, n_single=1, txt_len=128, grid_h=16, grid_w=16, cfg_id=50)
    check_cached(s, 16, 16, rel_tol=2e-2)


@pytest.mark.parametrize("in_gemm", [False, True])
def test_step_quantised_full_tokens_one_plus_one_blocks(in_gemm):
    # 4608 tokens: layers decoded once to bf16 (automatic), or dequantised
    # inside the GEMMs while staging weight tiles (dequant = 1)
    s = dataclasses.replace(I.CFG5, n_double=1, n_single=1)
    g, dbl, sgl = model_numpy(s)
    inp = I.step_inputs(s)
    _, vg = run_step(s, g, dbl, sgl, inp, 1, quant=bd.QUANT_POLICY, dequant_in_gemm=in_gemm)
    from tests.test_gpu_blocks import dequantised
    _, vr = oracle_step(s, g, [dequantised(d, bd.QUANT_POLICY) for d in dbl],
                        [dequantised(w, bd.QUANT_POLICY) for w in sgl], inp, 1)
    assert_parity(vg, vr, "bf16", "quantised step v")


def test_step_is_deterministic():
    s = dataclasses.replace(I.CFG4, n_double=1, n_single=1, txt_len=128, grid_h=32, grid_w=32, cfg_id=44)
    g, dbl, sgl = model_numpy(s)
    inp = I.step_inputs(s)
    (x1, v1), (x2, v2) = run_step(s, g, dbl, sgl, inp, 0, repeat=2)
    assert np.array_equal(v1, v2) and np.array_equal(x1, x2)


def test_step_graph_replays_match_eager():
    # The step captured into a HIP graph (torch's graph API on a side stream,
    # as bench.py times it) and replayed three times, with eager copies and
    # synchronisations between the replays: every replay must give the
    # eager step's x and v bit for bit (the library issues no memsets, so
    # the graph holds kernels only).
    t = torch()
    s = dataclasses.replace(I.CFG4, n_double=1, n_single=1, txt_len=128, grid_h=32, grid_w=32, cfg_id=52)
    g, dbl, sgl = model_numpy(s)
    inp = I.step_inputs(s)
    dt = dtype_code(s.dtype)
    cfg = bd.make_config(s)
    M = bd.ModelW(g, [bd.DoubleW(d, dt, "cuda") for d in dbl], [bd.SingleW(w, dt, "cuda") for w in sgl], dt, "cuda")
    mc = M.c()
    X0 = t.empty((s.batch, s.img_len, s.in_ch), dtype=t.float32, device="cuda")
    bd.mmdit_pack_latents(t.from_numpy(inp["z"]).cuda(), X0)
    ids = up_i32(bd.mmdit_make_ids(s.grid_h, s.grid_w, s.txt_len))
    sig = bd.mmdit_schedule(4, s.img_len)
    T = up(inp["T"], s.dtype)
    y = up(inp["y"], s.dtype)
    ws = workspace(bd.mmdit_step_workspace(cfg))
    X = X0.clone()
    v = t.empty_like(X)
    print("eager step", flush=True)
    bd.mmdit_step(cfg, mc, X, v, T, y, ids, sig[1], sig[2], ws)
    sync()
    x_ref, v_ref = down(X), down(v)
    X.copy_(X0)
    v.zero_()
    sync()
    print("capturing the step", flush=True)
    gr = t.cuda.CUDAGraph()
    cap = t.cuda.Stream()
    cap.wait_stream(t.cuda.current_stream())
    with t.cuda.graph(gr, stream=cap):
        bd.mmdit_step(cfg, mc, X, v, T, y, ids, sig[1], sig[2], ws)
    sync()
    for k in range(3):
        X.copy_(X0)
        v.fill_(float("nan"))
        sync()
        print(f"replay {k}", flush=True)
        gr.replay()
        sync()
        assert np.array_equal(down(X), x_ref), f"replay {k}: x differs"
        assert np.array_equal(down(v), v_ref), f"replay {k}: v differs"


@pytest.mark.parametrize("bits", [4, 8])
def test_step_quantised_final_layer(bits):
    # the final projection (h -> 64, fused Euler update) held as group-quantised
    # codes: the Euler epilogue dequantises its weight tiles like the others
    s = dataclasses.replace(I.CFG4, hidden=512, heads=4, mlp_hidden=1024, txt_len=24, grid_h=8, grid_w=8,
                            n_double=1, n_single=1, txt_in_dim=256, vec_in_dim=256, cfg_id=58)
    g, dbl, sgl = model_numpy(s)
    inp = I.step_inputs(s)
    t = torch()
    cfg = bd.make_config(s)
    M = bd.ModelW(g, [bd.DoubleW(d, bd.BF16, "cuda") for d in dbl], [bd.SingleW(w, bd.BF16, "cuda") for w in sgl],
                  bd.BF16, "cuda")
    M.final_lin = bd.Linear.from_numpy(g["final_w"], g["final_b"], bd.BF16, "cuda", bits)
    X = t.from_numpy(oracle.pack_latents(inp["z"])).cuda()
    v = t.empty_like(X)
    ids = bd.mmdit_make_ids(s.grid_h, s.grid_w, s.txt_len)
    sig = bd.mmdit_schedule(4, s.img_len)
    ws = workspace(bd.mmdit_step_workspace(cfg))
    print(f"step with a {bits}-bit final layer", flush=True)
    bd.mmdit_step(cfg, M.c(), X, v, up(inp["T"], "bf16"), up(inp["y"], "bf16"), up_i32(ids), sig[0], sig[1], ws)
    sync()
    q, sc = oracle.quantise(g["final_w"], bits)
    go = dict(g)
    go["final_w"] = oracle.dequantise(q, sc)
    Xr, vr = oracle.step(go, dbl, sgl, oracle.pack_latents(inp["z"]), inp["T"], inp["y"], ids, sig[0], sig[1],
                         s.heads, s.axes_dim, s.theta)
    assert_parity(down(v), vr, "bf16", f"{bits}-bit final layer: v")
    assert_parity(down(X), Xr, "bf16", f"{bits}-bit final layer: x_next")


# ------------------------------------------- modulations of several steps ---
def check_shared_modulations(s: I.Shape, n_sigma: int, guidance=None):
    """Every step of a schedule run with the modulation vectors that
    mmdit_step_modulations computed for n_sigma timesteps in one pass gives
    the plain step's x and v bit for bit (the same GEMVs per row), and the
    plain step matches the oracle."""
    t = torch()
    g, dbl, sgl = model_numpy(s)
    if guidance is not None:
        g = dict(g, **I.guidance_weights(s))
    inp = I.step_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    sig = oracle.schedule(n_sigma, s.img_len)
    dt = dtype_code(s.dtype)
    cfg = bd.make_config(s)
    M = bd.ModelW(g, [bd.DoubleW(d, dt, "cuda") for d in dbl], [bd.SingleW(w, dt, "cuda") for w in sgl], dt, "cuda")
    mc = M.c()
    z = t.from_numpy(inp["z"]).cuda()
    X0 = t.empty((s.batch, s.img_len, s.in_ch), dtype=t.float32, device="cuda")
    bd.mmdit_pack_latents(z, X0)
    T, y, ids_d = up(inp["T"], s.dtype), up(inp["y"], s.dtype), up_i32(ids)
    ws = workspace(bd.mmdit_step_workspace(cfg))
    mods = t.empty(bd.mmdit_step_modulations_bytes(cfg, n_sigma), dtype=t.uint8, device="cuda")
    print(f"modulations of {n_sigma} steps, B={s.batch} h={s.hidden} {s.dtype} guidance={guidance}", flush=True)
    bd.mmdit_step_modulations(cfg, mc, y, sig[:n_sigma], mods, guidance=guidance)
    Xp, Xs = X0.clone(), X0.clone()
    vp, vs = t.empty_like(X0), t.empty_like(X0)
    for j in range(n_sigma):
        bd.mmdit_step_ex(cfg, mc, Xp, vp, T, y, ids_d, sig[j], sig[j + 1], ws, guidance=guidance)
        # the shared-modulation step reads neither y nor the guidance value
        bd.mmdit_step_ex(cfg, mc, Xs, vs, T, None, ids_d, sig[j], sig[j + 1], ws, mods=mods, mods_count=n_sigma,
                         mods_index=j)
        sync()
        assert np.array_equal(down(vp), down(vs)), f"step {j}: v differs"
        assert np.array_equal(down(Xp), down(Xs)), f"step {j}: x differs"
        if j == 0:
            Xr, vr = oracle.step(g, dbl, sgl, oracle.pack_latents(inp["z"]), inp["T"], inp["y"], ids, sig[0], sig[1],
                                 s.heads, s.axes_dim, s.theta, guidance=guidance)
            assert_parity(down(vs), vr, s.dtype, "first step with shared modulations: v")


def test_shared_modulations_f32_batch2():
    check_shared_modulations(dataclasses.replace(TINY_F32, batch=2, txt_len=11, grid_h=6, grid_w=5, cfg_id=62), 2)


def test_shared_modulations_bf16_guided_four_steps():
    s = dataclasses.replace(I.CFG4, n_double=2, n_single=2, txt_len=64, grid_h=16, grid_w=16, cfg_id=63)
    check_shared_modulations(s, 4, guidance=3.5)


def test_shared_modulations_with_context_and_device_cache():
    # the options together: reference-image tokens, shared modulation
    # vectors, and the step cache decided on the device; every step equals
    # the plain cached step (modulations computed in the step, decision on
    # the host) bit for bit, decisions included
    t = torch()
    s = dataclasses.replace(I.CFG4, n_double=1, n_single=1, txt_len=64, grid_h=12, grid_w=12, cfg_id=65)
    cgh = cgw = 12
    g, dbl, sgl = model_numpy(s)
    inp = I.step_inputs(s)
    Lc = cgh * cgw
    Xc = np.random.default_rng(3000).standard_normal((s.batch, Lc, s.in_ch)).astype(np.float32)
    ids = ctx_ids(s, cgh, cgw)
    n = 4
    sig = oracle.schedule(n, s.img_len)
    dt = dtype_code(s.dtype)
    cfg = bd.make_config(s)
    cfg.dims.img_len = s.img_len + Lc
    M = bd.ModelW(g, [bd.DoubleW(d, dt, "cuda") for d in dbl], [bd.SingleW(w, dt, "cuda") for w in sgl], dt, "cuda")
    mc = M.c()
    X0 = t.empty((s.batch, s.img_len, s.in_ch), dtype=t.float32, device="cuda")
    bd.mmdit_pack_latents(t.from_numpy(inp["z"]).cuda(), X0)
    T, y, ids_d = up(inp["T"], s.dtype), up(inp["y"], s.dtype), up_i32(ids)
    xc = t.from_numpy(Xc).cuda()
    ws = workspace(bd.mmdit_step_workspace(cfg))
    mods = t.empty(bd.mmdit_step_modulations_bytes(cfg, n), dtype=t.uint8, device="cuda")
    bd.mmdit_step_modulations(cfg, mc, y, sig[:n], mods)
    # threshold between the second step's change and the sum of the second
    # and third (read from a pass that never reruns the blocks), so the
    # second step reuses the residual and the third runs the blocks
    probe = bd.StepCache(cfg)
    Xp, vp = X0.clone(), t.empty_like(X0)
    rel = []
    for j in range(3):
        bd.mmdit_step_ex(cfg, mc, Xp, vp, T, y, ids_d, sig[j], sig[j + 1], ws, ctx_packed=xc, ctx_len=Lc,
                         cache=probe, cache_threshold=float("inf"))
        sync()
        rel.append(probe.rel)
    thr = rel[1] + 0.5 * rel[2]
    ch, cd = bd.StepCache(cfg), bd.StepCache(cfg, on_device=True)
    Xh, Xd = X0.clone(), X0.clone()
    vh, vd = t.empty_like(X0), t.empty_like(X0)
    runs = []
    for j in range(n):
        print(f"step {j}: plain host-cached step against shared modulations + device cache", flush=True)
        bd.mmdit_step_ex(cfg, mc, Xh, vh, T, y, ids_d, sig[j], sig[j + 1], ws, ctx_packed=xc, ctx_len=Lc,
                         cache=ch, cache_threshold=thr)
        bd.mmdit_step_ex(cfg, mc, Xd, vd, T, None, ids_d, sig[j], sig[j + 1], ws, ctx_packed=xc, ctx_len=Lc,
                         cache=cd, cache_threshold=thr, mods=mods, mods_count=n, mods_index=j)
        sync()
        cd.read()
        assert cd.ran_blocks == ch.ran_blocks, (j, cd.ran_blocks, ch.ran_blocks)
        runs.append(ch.ran_blocks)
        assert np.array_equal(down(vh), down(vd)), f"step {j}: v differs"
        assert np.array_equal(down(Xh), down(Xd)), f"step {j}: x differs"
    print(f"blocks ran at steps: {runs}", flush=True)
    assert runs[:3] == [True, False, True], runs
