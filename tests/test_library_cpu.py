"""CPU checks of libmmdit.so: exported symbols, ABI layout of the structs,
host helpers bit-exact against the oracle, and argument errors returned
before any device work. No GPU is touched."""
import ctypes as C
import dataclasses
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from diffusion_transformer_mmdit_amd import binding as bd
from diffusion_transformer_mmdit_amd import inputs as I

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mmdit.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.lib_path()):
        pytest.fail("libmmdit.so is not built (python -m diffusion_transformer_mmdit_amd.build)")
    return bd.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mmdit_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(lib, n), n
        assert n in bd._SIGS, f"binding lacks a signature for {n}"
    assert bd.mmdit_version().startswith("mmdit")


def test_struct_layout_matches_c_compiler(lib):
    structs = {"mmdit_dims": bd.mmdit_dims, "mmdit_linear": bd.mmdit_linear,
               "mmdit_stream_w": bd.mmdit_stream_w, "mmdit_double_w": bd.mmdit_double_w,
               "mmdit_single_w": bd.mmdit_single_w, "mmdit_config": bd.mmdit_config,
               "mmdit_model_w": bd.mmdit_model_w, "mmdit_step_opts": bd.mmdit_step_opts,
               "mmdit_step_cache": bd.mmdit_step_cache}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for name, cls in structs.items():
        lines.append(f'printf("{name} size %zu\\n", sizeof({name}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{name} {f} %zu\\n", offsetof({name}, {f}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "l.c")
        exe = os.path.join(d, "l")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-o", exe, src], check=True)
        out = subprocess.run([exe], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for ln in out:
        if ln:
            a, b, v = ln.split()
            got[(a, b)] = int(v)
    for name, cls in structs.items():
        assert got[(name, "size")] == C.sizeof(cls), name
        for f, _ in cls._fields_:
            assert got[(name, f)] == getattr(cls, f).offset, (name, f)


@pytest.mark.parametrize("n,li,term,shift", [(4, 4096, 0.0, True), (4, 4096, 0.02, True), (50, 4096, 0.0, True),
                                             (1, 1024, 0.0, True), (7, 300, 0.0, True), (9, 4096, 0.0, False),
                                             (3, 256, 0.02, True)])
def test_schedule_bit_exact(lib, n, li, term, shift):
    got = bd.mmdit_schedule(n, li, 0.5, 1.15, term, shift)
    ref = oracle.schedule(n, li, 0.5, 1.15, sigma_terminal=term, shift=shift)
    assert np.array_equal(got, ref)


def test_make_ids_bit_exact(lib):
    for gh, gw, lt, fr in [(64, 64, 512, 0), (8, 8, 16, 0), (3, 7, 0, 2), (1, 1, 5, 1)]:
        assert np.array_equal(bd.mmdit_make_ids(gh, gw, lt, fr), oracle.make_ids(gh, gw, lt, fr))


@pytest.mark.parametrize("bits", [4, 8])
def test_quantiser_bit_exact(lib, bits):
    w = I.normal((96, 320), (999, 0, bits), std=0.02)
    w[5, 64:128] = 0.0
    w[7, :64] *= 1e-30                      # subnormal-scale group
    w[9, 3] = 0.5                           # one outlier
    packed, scales = bd.mmdit_quantise(w, bits)
    q, s = oracle.quantise(w, bits)
    assert np.array_equal(scales, I.bf16_bits(s))
    if bits == 4:
        assert np.array_equal(packed, oracle.pack_int4(q))
    else:
        assert np.array_equal(packed, q)


@pytest.mark.parametrize("bits", [1, 2])
def test_quantiser_g128_bit_exact(lib, bits):
    w = I.normal((40, 384), (998, 0, bits), std=0.02)
    w[5, 128:256] = 0.0
    w[7, :128] *= 1e-30                     # subnormal-scale group
    w[9, 3] = 0.5                           # one outlier
    w[11, 7] = -0.0
    packed, scales = bd.mmdit_quantise(w, bits)
    c, s = oracle.quantise_g128(w, bits)
    assert np.array_equal(scales, I.bf16_bits(s))
    assert np.array_equal(packed, oracle.pack_g128(c, bits))


def _dims(**kw):
    s = I.Shape(**{**dict(hidden=256, heads=2, mlp_hidden=512, txt_len=16, grid_h=8, grid_w=8,
                          dtype="bf16"), **kw})
    return bd.make_dims(s)


@pytest.mark.parametrize("change,status", [
    (dict(head_dim=64), 5), (dict(hidden=384), 2), (dict(mlp_hidden=100), 2), (dict(batch=0), 2),
    (dict(img_len=0), 2), (dict(act_dtype=7), 3), (dict(txt_len=-1), 2)])
def test_dims_errors(lib, change, status):
    d = _dims()
    for k, v in change.items():
        setattr(d, k, v)
    n = C.c_size_t(0)
    assert lib.mmdit_double_block_workspace(C.byref(d), C.byref(n)) == status
    assert n.value == 0
    assert len(bd.mmdit_last_error()) > 0


def test_axes_must_sum_to_head_dim(lib):
    d = _dims()
    d.axes_dim = (C.c_int32 * 3)(16, 56, 54)
    n = C.c_size_t(0)
    assert lib.mmdit_single_block_workspace(C.byref(d), C.byref(n)) == 2


def _fake_linear(n, k, fmt=0, scales=True):
    return bd.mmdit_linear(0x1000, 0x2000 if scales else None, 0x3000, fmt, n, k)


def _fake_stream(h, m, **over):
    parts = dict(mod=_fake_linear(6 * h, h), qkv=_fake_linear(3 * h, h), proj=_fake_linear(h, h),
                 fc1=_fake_linear(m, h), fc2=_fake_linear(h, m))
    parts.update(over)
    return bd.mmdit_stream_w(parts["mod"], parts["qkv"], parts["proj"], parts["fc1"], parts["fc2"], 0x4000, 0x4000)


def _call_double(lib, d, w, ws_bytes, ws_ptr=0x5000):
    # Fake, never-dereferenced pointers: every check below fails before any launch.
    return lib.mmdit_double_block_fwd(C.byref(d), C.byref(w), 0x6000, 0x6000, 0x6000, 0x6000, 0x6000, 0x6000,
                                      ws_ptr, ws_bytes, None)


def test_block_errors_before_launch(lib):
    d = _dims()
    h, m = 256, 512
    good = bd.mmdit_double_w(_fake_stream(h, m), _fake_stream(h, m))
    need = bd.mmdit_double_block_workspace(d)
    assert need > 0
    assert _call_double(lib, d, good, need - 1) == 4                       # workspace
    assert _call_double(lib, d, good, need, ws_ptr=None) == 4
    bad = bd.mmdit_double_w(_fake_stream(h, m, qkv=_fake_linear(3 * h, h + 64)), _fake_stream(h, m))
    assert _call_double(lib, d, bad, need) == 2                            # shape
    bad = bd.mmdit_double_w(_fake_stream(h, m), _fake_stream(h, m, fc1=_fake_linear(m, h, fmt=1, scales=False)))
    assert _call_double(lib, d, bad, need) == 1                            # null scales
    bad = bd.mmdit_double_w(_fake_stream(h, m), _fake_stream(h, m, fc1=_fake_linear(m, h, fmt=9)))
    assert _call_double(lib, d, bad, need) == 3                            # format
    d32 = _dims(dtype="f32")
    d32.act_dtype = bd.F32
    q = bd.mmdit_double_w(_fake_stream(h, m, fc1=_fake_linear(m, h, fmt=1)), _fake_stream(h, m))
    assert _call_double(lib, d32, q, 1 << 40) == 3                         # quantised needs bf16
    bad = bd.mmdit_double_w(_fake_stream(h, m, mod=_fake_linear(6 * h, h, fmt=2)), _fake_stream(h, m))
    assert _call_double(lib, d, bad, need) == 3                            # modulation must be dense
    assert lib.mmdit_double_block_fwd(C.byref(d), None, 0x6000, 0x6000, 0x6000, 0x6000, 0x6000, 0x6000,
                                      0x5000, need, None) == 1


def test_step_ex_errors_before_launch(lib):
    # option checks run before any weight is read or kernel launched: the
    # model below has only a (fake) guidance embedder pointer
    s = I.Shape(hidden=256, heads=2, mlp_hidden=512, txt_len=16, grid_h=8, grid_w=8, dtype="f32", cfg_id=41,
                n_double=1, n_single=1, txt_in_dim=256, vec_in_dim=256)
    cfg = bd.make_config(s)
    w = bd.mmdit_model_w()
    w.guidance_in0.w = 0x1000
    fake = 0x6000

    def call(opts):
        return lib.mmdit_step_ex(C.byref(cfg), C.byref(w), fake, None, fake, fake, fake, 1.0, 0.5, opts, fake,
                                 1 << 40, None)
    assert call(None) == 1                                                  # guidance model, no value
    assert lib.mmdit_step(C.byref(cfg), C.byref(w), fake, None, fake, fake, fake, 1.0, 0.5, fake, 1 << 40,
                          None) == 1
    o = bd.mmdit_step_opts(has_guidance=1, guidance=float("nan"))
    assert call(C.byref(o)) == 2                                            # non-finite guidance
    o = bd.mmdit_step_opts(ctx_packed=fake, ctx_len=s.img_len, has_guidance=1, guidance=3.5)
    assert call(C.byref(o)) == 2                                            # no generated tokens left
    o = bd.mmdit_step_opts(ctx_packed=None, ctx_len=4, has_guidance=1, guidance=3.5)
    assert call(C.byref(o)) == 1                                            # NULL context latent
    o = bd.mmdit_step_opts(ctx_packed=fake, ctx_len=-1)
    assert call(C.byref(o)) == 2
    o = bd.mmdit_step_opts(has_guidance=1, guidance=3.5, dequant=2)
    assert call(C.byref(o)) == 2                                            # unknown dequant route
    # step cache options
    need = bd.mmdit_step_cache_bytes(cfg)
    cache = bd.mmdit_step_cache(buf=fake, bytes=need)
    for thr, want in ((float("nan"), 2), (-0.1, 2)):
        o = bd.mmdit_step_opts(has_guidance=1, guidance=3.5, cache=C.pointer(cache), cache_threshold=thr)
        assert call(C.byref(o)) == want
    o = bd.mmdit_step_opts(has_guidance=1, guidance=3.5, cache=C.pointer(bd.mmdit_step_cache(bytes=need)),
                           cache_threshold=0.1)
    assert call(C.byref(o)) == 1                                            # NULL cache buffer
    o = bd.mmdit_step_opts(has_guidance=1, guidance=3.5,
                           cache=C.pointer(bd.mmdit_step_cache(buf=fake, bytes=need - 1)), cache_threshold=0.1)
    assert call(C.byref(o)) == 4                                            # cache buffer too small
    o = bd.mmdit_step_opts(has_guidance=1, guidance=3.5, cache=C.pointer(cache), cache_threshold=0.1,
                           cache_on_device=2)
    assert call(C.byref(o)) == 2                                            # unknown decision mode
    cfg0 = bd.make_config(dataclasses.replace(s, n_double=0))
    o = bd.mmdit_step_opts(has_guidance=1, guidance=3.5, cache=C.pointer(cache), cache_threshold=0.1)
    assert lib.mmdit_step_ex(C.byref(cfg0), C.byref(w), fake, None, fake, fake, fake, 1.0, 0.5, C.byref(o), fake,
                             1 << 40, None) == 2                            # no dual block to read
    assert cache.valid == 0


def test_step_cache_bytes(lib):
    s = I.CFG4
    n = bd.mmdit_step_cache_bytes(bd.make_config(s))
    # a_prev and the residual in float32, two floats per image row, 32 bytes
    # of decision state
    lo = 2 * s.img_len * s.hidden * 4 + s.img_len * 8 + 32
    assert lo <= n <= lo + 1024


def test_step_cache_read_errors(lib):
    # checked before the device copy: the buffer pointer is never used
    cfg = bd.make_config(I.CFG4)
    need = bd.mmdit_step_cache_bytes(cfg)
    fake = 0x6000
    assert lib.mmdit_step_cache_read(C.byref(cfg), None, None) == 1
    c = bd.mmdit_step_cache(buf=None, bytes=need, valid=1)
    assert lib.mmdit_step_cache_read(C.byref(cfg), C.byref(c), None) == 1     # NULL buffer
    c = bd.mmdit_step_cache(buf=fake, bytes=need - 1, valid=1)
    assert lib.mmdit_step_cache_read(C.byref(cfg), C.byref(c), None) == 4     # buffer too small
    c = bd.mmdit_step_cache(buf=fake, bytes=need, valid=0)
    assert lib.mmdit_step_cache_read(C.byref(cfg), C.byref(c), None) == 2     # no step has run


def test_dequantise_argument_errors(lib):
    # checked on the host before any device work (the pointers are never used)
    w, sc, out = 0x10000, 0x20000, 0x30000
    call = lambda *a: lib.mmdit_dequantise(*a, None)  # noqa: E731
    assert call(None, sc, bd.W_Q4G64, 4, 64, out) == 1                  # NULL weights
    assert call(w, sc, bd.W_Q4G64, 4, 64, None) == 1                    # NULL output
    assert call(w, sc, bd.W_DENSE, 4, 64, out) == 3                     # not a quantised format
    assert call(w, sc, 9, 4, 64, out) == 3
    assert call(w, sc, bd.W_Q8G64, 4, 96, out) == 2                     # k_in not a multiple of 64
    assert call(w, sc, bd.W_Q1G128, 4, 64, out) == 2                    # sub-byte groups are 128
    assert call(w, sc, bd.W_TQ2G128, -1, 128, out) == 2                 # negative rows
    assert call(w + 8, sc, bd.W_Q4G64, 4, 64, out) == 2                 # codes not 16-byte aligned
    assert call(w + 4, sc, bd.W_TQ2G128, 4, 128, out) == 2              # ternary codes need 8
    assert call(w, sc + 1, bd.W_Q8G64, 4, 64, out) == 2                 # odd scale address
    assert call(w, sc, bd.W_Q8G64, 4, 64, out + 8) == 2                 # output not 16-byte aligned
    assert "aligned" in bd.mmdit_last_error() or "misaligned" in bd.mmdit_last_error()


def test_workspace_holds_decoded_weights_from_1024_rows(lib):
    # bf16 at 1024 rows and more: room for the largest launch's weights in
    # bf16 (both streams' fc1 at h 3072, m 12288: 2 * 12288 * 3072 weights)
    below = bd.mmdit_double_block_workspace(_dims(hidden=3072, heads=24, mlp_hidden=12288, txt_len=0,
                                                  grid_h=31, grid_w=33))
    at = bd.mmdit_double_block_workspace(_dims(hidden=3072, heads=24, mlp_hidden=12288, txt_len=0,
                                               grid_h=32, grid_w=32))
    assert 2 * 12288 * 3072 * 2 <= at - below <= 2 * 12288 * 3072 * 2 + 4 * 2**20
    f32 = bd.mmdit_double_block_workspace(_dims(hidden=3072, heads=24, mlp_hidden=12288, txt_len=0,
                                                grid_h=32, grid_w=32, dtype="f32"))
    below32 = bd.mmdit_double_block_workspace(_dims(hidden=3072, heads=24, mlp_hidden=12288, txt_len=0,
                                                    grid_h=31, grid_w=33, dtype="f32"))
    assert f32 - below32 < 4 * 2**20


def test_workspace_sizes_scale_with_tokens(lib):
    small = bd.mmdit_double_block_workspace(_dims(grid_h=8, grid_w=8))
    big = bd.mmdit_double_block_workspace(_dims(grid_h=16, grid_w=16))
    assert big > small > 0
    cfg = bd.make_config(I.CFG4)
    n = bd.mmdit_step_workspace(cfg)
    # f32 residual (56.6 MB) + block scratch; well under a GB at 1024^2
    assert 200e6 < n < 1.5e9


def test_step_noalloc_refuses_configurations_beyond_its_scratch(lib):
    # the 1024^2 step needs more workspace than the library's 256 MiB scratch:
    # refused with MMDIT_ERR_WORKSPACE before any device work (dummy pointers)
    cfg = bd.make_config(I.CFG4)
    M = bd.mmdit_model_w()
    dbl = (bd.mmdit_double_w * I.CFG4.n_double)()
    sgl = (bd.mmdit_single_w * I.CFG4.n_single)()
    M.dbl = C.cast(dbl, C.POINTER(bd.mmdit_double_w))
    M.sgl = C.cast(sgl, C.POINTER(bd.mmdit_single_w))
    # dense weights: no room for decoded layers, and still above 256 MiB
    assert bd.mmdit_step_workspace_ex(cfg, M) > bd.NOALLOC_SCRATCH_BYTES
    assert bd.mmdit_step_workspace_ex(cfg, M) < bd.mmdit_step_workspace(cfg)
    dummy = C.c_void_p(4096)
    st = lib.mmdit_step_noalloc(C.byref(cfg), C.byref(M), dummy, dummy, dummy, dummy, dummy, 1.0, 0.5, None, None)
    assert st == 4
    assert "256" in bd.mmdit_last_error() or "268435456" in bd.mmdit_last_error()
    # a NULL config is an argument error, also before any device work
    assert lib.mmdit_step_noalloc(None, C.byref(M), dummy, dummy, dummy, dummy, dummy, 1.0, 0.5, None, None) == 1


def test_step_workspace_ex_leaves_out_decoded_weight_room_for_dense_models(lib):
    # h 3072, 1280 tokens: a dense model needs no room for decoded weights
    # (2 * 3072 * 12288 bf16 = 151 MB); a quantised one does unless every
    # layer is dequantised inside its GEMM
    s = I.CFG2
    cfg = bd.make_config(dataclasses.replace(s, n_double=1, n_single=1))
    M = bd.mmdit_model_w()
    dbl = (bd.mmdit_double_w * 1)()
    sgl = (bd.mmdit_single_w * 1)()
    M.dbl = C.cast(dbl, C.POINTER(bd.mmdit_double_w))
    M.sgl = C.cast(sgl, C.POINTER(bd.mmdit_single_w))
    full = bd.mmdit_step_workspace(cfg)
    dense = bd.mmdit_step_workspace_ex(cfg, M)
    assert full - dense >= 2 * 3072 * 12288 * 2
    sgl[0].lin1.fmt = bd.W_Q4G64
    assert bd.mmdit_step_workspace_ex(cfg, M) == full
    assert bd.mmdit_step_workspace_ex(cfg, M, dequant_in_gemm=True) == dense


def test_resid_field_is_checked(lib):
    n = C.c_size_t()
    d = bd.make_dims(I.CFG2, resid=7)
    assert lib.mmdit_double_block_workspace(C.byref(d), C.byref(n)) == 3
    d = bd.make_dims(I.CFG1, resid=bd.RESID_BF16)  # float32 activations
    assert lib.mmdit_double_block_workspace(C.byref(d), C.byref(n)) == 3
    d = bd.make_dims(I.CFG2, resid=bd.RESID_BF16)
    assert lib.mmdit_double_block_workspace(C.byref(d), C.byref(n)) == 0
    # the step's bf16 residual halves the residual buffer
    c32 = bd.make_config(I.CFG4)
    c16 = bd.make_config(I.CFG4, resid=bd.RESID_BF16)
    assert bd.mmdit_step_workspace(c32) - bd.mmdit_step_workspace(c16) >= I.CFG4.seq_len * 3072 * 2


def test_linear_entry_point_errors_before_launch(lib):
    # argument errors of mmdit_linear_fwd / mmdit_linear_workspace return
    # before any device work (dummy device pointers are never touched)
    dummy = C.c_void_p(4096)
    lin = bd.mmdit_linear(w=4096, scales=4096, bias=None, fmt=bd.W_Q4G64, n_out=328, k_in=384)
    n = C.c_size_t()
    assert lib.mmdit_linear_workspace(C.byref(lin), bd.BF16, 300, bd.ROUTE_DECODE, C.byref(n)) == 0
    assert n.value >= 328 * 384 * 2
    assert lib.mmdit_linear_workspace(C.byref(lin), bd.BF16, 300, bd.ROUTE_TILED, C.byref(n)) == 0 and n.value == 0
    assert lib.mmdit_linear_workspace(C.byref(lin), bd.BF16, 5, bd.ROUTE_AUTO, C.byref(n)) == 0 and n.value == 0
    # the streaming route needs M <= 16
    assert lib.mmdit_linear_fwd(C.byref(lin), bd.BF16, dummy, 17, dummy, 1, bd.ROUTE_STREAM, None, 0, None) == 2
    # the decoding route needs its workspace
    assert lib.mmdit_linear_fwd(C.byref(lin), bd.BF16, dummy, 300, dummy, 1, bd.ROUTE_DECODE, None, 0, None) == 4
    # quantised weights need bf16 activations; unknown route
    assert lib.mmdit_linear_fwd(C.byref(lin), bd.F32, dummy, 8, dummy, 1, bd.ROUTE_AUTO, None, 0, None) == 3
    assert lib.mmdit_linear_fwd(C.byref(lin), bd.BF16, dummy, 8, dummy, 1, 7, None, 0, None) == 2
    dense = bd.mmdit_linear(w=4096, scales=None, bias=None, fmt=bd.W_DENSE, n_out=328, k_in=384)
    assert lib.mmdit_linear_fwd(C.byref(dense), bd.BF16, dummy, 300, dummy, 1, bd.ROUTE_DECODE, dummy, 1 << 20,
                                None) == 2
    # the streaming route reads 16-byte pieces of 4-bit rows and 4-byte scale pairs
    odd = bd.mmdit_linear(w=4096 + 8, scales=4096, bias=None, fmt=bd.W_Q4G64, n_out=328, k_in=384)
    assert lib.mmdit_linear_fwd(C.byref(odd), bd.BF16, dummy, 4, dummy, 1, bd.ROUTE_STREAM, None, 0, None) == 2
    odd = bd.mmdit_linear(w=4096, scales=4096 + 2, bias=None, fmt=bd.W_Q4G64, n_out=328, k_in=384)
    assert lib.mmdit_linear_fwd(C.byref(odd), bd.BF16, dummy, 4, dummy, 1, bd.ROUTE_STREAM, None, 0, None) == 2
    # M = 0 is a no-op, NULL weights an error
    assert lib.mmdit_linear_fwd(C.byref(dense), bd.BF16, None, 0, None, 1, bd.ROUTE_AUTO, None, 0, None) == 0
    assert lib.mmdit_linear_fwd(None, bd.BF16, dummy, 4, dummy, 1, bd.ROUTE_AUTO, None, 0, None) == 1


def test_adaln_layernorm_errors_before_launch(lib):
    dummy = C.c_void_p(4096)
    assert lib.mmdit_adaln_layernorm(dummy, 1, dummy, bd.BF16, 10, 300, dummy, C.c_float(1e-6), None) == 2
    assert lib.mmdit_adaln_layernorm(dummy, 1, dummy, 5, 10, 256, dummy, C.c_float(1e-6), None) == 3
    assert lib.mmdit_adaln_layernorm(None, 1, dummy, bd.BF16, 10, 256, dummy, C.c_float(1e-6), None) == 1
    assert lib.mmdit_adaln_layernorm(None, 1, None, bd.BF16, 0, 256, None, C.c_float(1e-6), None) == 0


def test_step_modulations_errors_before_launch(lib):
    # argument errors return before any device work (dummy pointers unused)
    s = I.Shape(hidden=256, heads=2, mlp_hidden=512, txt_len=16, grid_h=8, grid_w=8, dtype="f32", cfg_id=64,
                n_double=1, n_single=1, txt_in_dim=256, vec_in_dim=256)
    cfg = bd.make_config(s)
    n = C.c_size_t()
    assert lib.mmdit_step_modulations_bytes(C.byref(cfg), 0, C.byref(n)) == 2
    assert lib.mmdit_step_modulations_bytes(C.byref(cfg), 5, C.byref(n)) == 2          # at most 4 rows
    assert lib.mmdit_step_modulations_bytes(C.byref(cfg), 4, C.byref(n)) == 0
    # 4 timesteps of (12 + 3 + 2) h floats each, plus the conditioning scratch
    assert n.value >= 4 * 17 * 256 * 4
    cfg2 = bd.make_config(dataclasses.replace(s, batch=2))
    assert lib.mmdit_step_modulations_bytes(C.byref(cfg2), 3, C.byref(n)) == 2         # 3 x 2 rows
    need = bd.mmdit_step_modulations_bytes(cfg, 2)
    w = bd.mmdit_model_w()
    fake = 0x6000
    sg = (C.c_double * 2)(1.0, 0.5)
    call = lambda mods, nbytes, sig=sg, y=fake: lib.mmdit_step_modulations(  # noqa: E731
        C.byref(cfg), C.byref(w), y, sig, 2, None, mods, nbytes, None)
    assert call(fake, need, y=None) == 1                                                # NULL y
    assert call(None, need) == 1                                                        # NULL buffer
    assert call(fake + 8, need) == 2                                                    # misaligned buffer
    assert call(fake, need - 1) == 4                                                    # buffer too small
    assert call(fake, need, sig=(C.c_double * 2)(1.0, float("nan"))) == 2              # non-finite sigma
    # a step given modulations checks which timestep it is
    o = bd.mmdit_step_opts(mods=fake, mods_count=2, mods_index=2)
    assert lib.mmdit_step_ex(C.byref(cfg), C.byref(w), fake, None, fake, None, fake, 1.0, 0.5, C.byref(o), fake,
                             1 << 40, None) == 2
    o = bd.mmdit_step_opts(mods=fake + 4, mods_count=2, mods_index=1)
    assert lib.mmdit_step_ex(C.byref(cfg), C.byref(w), fake, None, fake, None, fake, 1.0, 0.5, C.byref(o), fake,
                             1 << 40, None) == 2
