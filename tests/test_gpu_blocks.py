"""GPU parity of the block entry points against the CPU oracle.

Every case runs the HIP path through the C ABI and compares with the oracle
on the same seeded inputs: float32 to rel-L2 <= 1e-5, bf16 to rel-L2 <= 2e-2
and cosine >= 0.999, integer/bit work exactly."""
import numpy as np
import pytest

import oracle
from diffusion_transformer_mmdit_amd import binding as bd
from diffusion_transformer_mmdit_amd import inputs as I
from tests.gpu_util import (assert_parity, down, dtype_code, sync, torch, up, up_i32, workspace)

pytestmark = pytest.mark.gpu


def run_double(s: I.Shape, w_np, x, ids, frame_ids=None, quant=None, inplace=False):
    t = torch()
    dims = bd.make_dims(s)
    W = bd.DoubleW(w_np, dtype_code(s.dtype), "cuda", quant)
    wc = W.c()
    img = up(x["x_img"], s.dtype)
    txt = up(x["x_txt"], s.dtype)
    vec = up(x["vec"], s.dtype)
    ids_d = up_i32(ids)
    ws = workspace(bd.mmdit_double_block_workspace(dims))
    if inplace:
        img_o, txt_o = img, txt
    else:
        img_o, txt_o = t.empty_like(img), t.empty_like(txt)
    print(f"double block B={s.batch} h={s.hidden} Lt={s.txt_len} Li={s.img_len} {s.dtype}", flush=True)
    bd.mmdit_double_block_fwd(dims, wc, img, txt, img_o, txt_o, vec, ids_d, ws)
    sync()
    return down(img_o), down(txt_o)


def run_single(s: I.Shape, w_np, x, ids, quant=None, inplace=False):
    t = torch()
    dims = bd.make_dims(s)
    W = bd.SingleW(w_np, dtype_code(s.dtype), "cuda", quant)
    wc = W.c()
    xin = up(x["x"], s.dtype)
    vec = up(x["vec"], s.dtype)
    ids_d = up_i32(ids)
    ws = workspace(bd.mmdit_single_block_workspace(dims))
    out = xin if inplace else t.empty_like(xin)
    print(f"single block B={s.batch} h={s.hidden} L={s.seq_len} {s.dtype}", flush=True)
    bd.mmdit_single_block_fwd(dims, wc, xin, out, vec, ids_d, ws)
    sync()
    return down(out)


def oracle_double(s, w, x, ids):
    return oracle.double_block(w, x["x_img"], x["x_txt"], x["vec"], ids, s.heads, s.axes_dim, s.theta)


def oracle_single(s, w, x, ids):
    return oracle.single_block(w, x["x"], x["vec"], ids, s.heads, s.axes_dim, s.theta)


def dequantised(w, quant):
    """Copy of block weights holding the dequantised values of the layers the
    policy quantises (the oracle's quantised GEMM is the float32 GEMM on them)."""
    if "txt" in w:
        return {k: dequantised(v, quant) for k, v in w.items()}
    out = dict(w)
    for name, bits in quant.items():
        if name + "_w" in w:
            if bits in (1, 2):
                c, sc = oracle.quantise_g128(w[name + "_w"], bits)
                out[name + "_w"] = oracle.dequantise_g128(c, sc, bits)
            else:
                q, sc = oracle.quantise(w[name + "_w"], bits)
                out[name + "_w"] = oracle.dequantise(q, sc)
    return out


# 1-bit and ternary weights (groups of 128): ternary inner projections,
# 1-bit residual-writing layers, so one block runs both formats
SUB_BYTE_MIX = {"qkv": 2, "fc1": 2, "lin1": 2, "proj": 1, "fc2": 1, "lin2": 1}


# ------------------------------------------------------------- float32 ------
def test_double_block_cfg1_f32():
    s = I.CFG1
    w = I.double_block_weights(s, 0)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "f32", "cfg1 img")
    assert_parity(txt, rtxt, "f32", "cfg1 txt")


def test_single_block_cfg1_f32():
    s = I.CFG1
    w = I.single_block_weights(s, 0)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    assert_parity(run_single(s, w, x, ids), oracle_single(s, w, x, ids), "f32", "cfg1 single")


def test_blocks_f32_width1024():
    # float32 at h 1024 (8 heads): the LayerNorm takes its one-block-per-row
    # form (h a multiple of 1024) with float32 input and output
    s = I.Shape(hidden=1024, heads=8, mlp_hidden=2048, txt_len=24, grid_h=6, grid_w=7, batch=2, dtype="f32",
                cfg_id=55)
    w = I.double_block_weights(s, 0)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "f32", "h 1024 img")
    assert_parity(txt, rtxt, "f32", "h 1024 txt")
    ws_ = I.single_block_weights(s, 0)
    assert_parity(run_single(s, ws_, x, ids), oracle_single(s, ws_, x, ids), "f32", "h 1024 single")


@pytest.mark.parametrize("txt_len,gh,gw,batch", [(0, 5, 7, 1), (13, 9, 11, 2), (130, 3, 3, 1)])
def test_blocks_f32_ragged(txt_len, gh, gw, batch):
    s = I.Shape(hidden=256, heads=2, mlp_hidden=320, txt_len=txt_len, grid_h=gh, grid_w=gw, batch=batch,
                dtype="f32", cfg_id=31)
    w = I.double_block_weights(s, 1)
    x = I.block_inputs(s)
    ids = oracle.make_ids(gh, gw, txt_len, frame=1)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "f32", "ragged img")
    if txt_len:
        assert_parity(txt, rtxt, "f32", "ragged txt")
    ws_ = I.single_block_weights(s, 1)
    assert_parity(run_single(s, ws_, x, ids), oracle_single(s, ws_, x, ids), "f32", "ragged single")


# ---------------------------------------------------------------- bf16 ------
def test_double_block_cfg2_bf16():
    s = I.CFG2
    w = I.double_block_weights(s, 0)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "bf16", "cfg2 img")
    assert_parity(txt, rtxt, "bf16", "cfg2 txt")


def _sharpened(w, a):
    """Copy of bf16 block weights with the QK RMSNorm scales multiplied by a
    (rounded to bf16, so both sides get the same values)."""
    if "txt" in w:
        return {k: _sharpened(v, a) for k, v in w.items()}
    out = dict(w)
    for n in ("q_norm", "k_norm"):
        out[n] = I.round_bf16(np.asarray(w[n], np.float32) * np.float32(a))
    return out


def test_blocks_bf16_sharp_attention():
    # The seeded norm scales (about 1) give scores with a standard deviation
    # of about 1.4 in log2 units, so the running max of the online softmax
    # settles on the first key tile. Scales of 3 make it about 13: over the
    # 1280 keys, about half the queries' max exceeds their first tile's max
    # by more than 12 (a probability above 2^12), so later tiles take the
    # path that moves the running max and rescales O and the row sums.
    s = I.CFG2
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    w = _sharpened(I.double_block_weights(s, 0), 3.0)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "bf16", "sharp attention img")
    assert_parity(txt, rtxt, "bf16", "sharp attention txt")
    ws_ = _sharpened(I.single_block_weights(s, 0), 3.0)
    assert_parity(run_single(s, ws_, x, ids), oracle_single(s, ws_, x, ids), "bf16", "sharp attention single")


@pytest.mark.parametrize("txt_len,gh,gw,batch", [(77, 9, 13, 2), (0, 16, 12, 1), (200, 1, 1, 1), (5, 3, 4, 1), (40, 5, 5, 2)])
def test_blocks_bf16_ragged(txt_len, gh, gw, batch):
    s = I.Shape(hidden=512, heads=4, mlp_hidden=1024, txt_len=txt_len, grid_h=gh, grid_w=gw, batch=batch,
                dtype="bf16", cfg_id=32)
    w = I.double_block_weights(s, 2)
    x = I.block_inputs(s)
    ids = oracle.make_ids(gh, gw, txt_len, frame=0)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "bf16", "ragged img")
    if txt_len:
        assert_parity(txt, rtxt, "bf16", "ragged txt")
    ws_ = I.single_block_weights(s, 2)
    assert_parity(run_single(s, ws_, x, ids), oracle_single(s, ws_, x, ids), "bf16", "ragged single")


def test_blocks_bf16_max_width():
    # the widest model the library takes: h 4096 (32 heads), MLP 16384, with
    # 40 text + 12x13 image tokens (the LayerNorm's four chunks per thread,
    # 4096-wide modulation GEMVs)
    s = I.Shape(hidden=4096, heads=32, mlp_hidden=16384, txt_len=40, grid_h=12, grid_w=13, dtype="bf16",
                cfg_id=53)
    w = I.double_block_weights(s, 0)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "bf16", "max-width img")
    assert_parity(txt, rtxt, "bf16", "max-width txt")
    ws_ = I.single_block_weights(s, 0)
    assert_parity(run_single(s, ws_, x, ids), oracle_single(s, ws_, x, ids), "bf16", "max-width single")


def test_blocks_bf16_reference_image_length():
    # the reference-image sequence at its full length: 512 text + 4096
    # generated + 4096 context tokens (L 8704; the context rows carry frame
    # id 1), dual and single blocks against the oracle on every output
    s = I.Shape(txt_len=512, grid_h=64, grid_w=128, dtype="bf16", cfg_id=54)
    x = I.block_inputs(s)
    ids = np.concatenate([oracle.make_ids(64, 64, 512), oracle.make_ids(64, 64, 0, frame=1)])
    w = I.double_block_weights(s, 0)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "bf16", "L 8704 dual img")
    assert_parity(txt, rtxt, "bf16", "L 8704 dual txt")
    del w, rimg, rtxt
    ws_ = I.single_block_weights(s, 0)
    assert_parity(run_single(s, ws_, x, ids), oracle_single(s, ws_, x, ids), "bf16", "L 8704 single")


@pytest.fixture(scope="module")
def cfg3():
    s = I.CFG3
    return s, I.block_inputs(s), oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)


def test_double_block_cfg3_bf16_full_size(cfg3):
    s, x, ids = cfg3
    w = I.double_block_weights(s, 0)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "bf16", "cfg3 dual img")
    assert_parity(txt, rtxt, "bf16", "cfg3 dual txt")


def test_single_block_cfg3_bf16_full_size(cfg3):
    s, x, ids = cfg3
    w = I.single_block_weights(s, 0)
    assert_parity(run_single(s, w, x, ids), oracle_single(s, w, x, ids), "bf16", "cfg3 single")


@pytest.mark.parametrize("quant", [None, "policy", "sub_byte"])
def test_blocks_bf16_full_width_ragged_rows(quant):
    # h 3072 with 77 text + 40x41 image tokens: the projections take the
    # 256x256 direct-to-LDS GEMM with partial row tiles in both streams
    # (dense weights; 4/8-bit or 1-bit/ternary weights, which at 1717 rows
    # are decoded to bf16 a layer at a time first)
    s = I.Shape(txt_len=77, grid_h=40, grid_w=41, dtype="bf16", cfg_id=38)
    q = {None: None, "policy": bd.QUANT_POLICY, "sub_byte": SUB_BYTE_MIX}[quant]
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    w = I.double_block_weights(s, 0)
    img, txt = run_double(s, w, x, ids, quant=q)
    wo = dequantised(w, q) if q else w
    rimg, rtxt = oracle_double(s, wo, x, ids)
    assert_parity(img, rimg, "bf16", f"ragged-rows dual img {quant}")
    assert_parity(txt, rtxt, "bf16", f"ragged-rows dual txt {quant}")
    ws_ = I.single_block_weights(s, 0)
    wso = dequantised(ws_, q) if q else ws_
    assert_parity(run_single(s, ws_, x, ids, quant=q), oracle_single(s, wso, x, ids), "bf16",
                  f"ragged-rows single {quant}")


@pytest.mark.parametrize("quant", ["policy", "sub_byte"])
def test_blocks_quantised_full_width_below_decoding_rows(quant):
    # h 3072 with 77 text + 28x30 image tokens (917 rows, under the 1024 from
    # which whole layers are decoded to bf16 first): the GEMM kernels
    # dequantise weight tiles as they stage them, on the 256x256
    # direct-to-LDS kernel (fc1: 240 tiles, linear1: 336) and on the
    # register-staged one (qkv, out-projection, fc2, linear2)
    s = I.Shape(txt_len=77, grid_h=28, grid_w=30, dtype="bf16", cfg_id=51)
    q = {"policy": bd.QUANT_POLICY, "sub_byte": SUB_BYTE_MIX}[quant]
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    w = I.double_block_weights(s, 0)
    img, txt = run_double(s, w, x, ids, quant=q)
    rimg, rtxt = oracle_double(s, dequantised(w, q), x, ids)
    assert_parity(img, rimg, "bf16", f"fused-dequant dual img {quant}")
    assert_parity(txt, rtxt, "bf16", f"fused-dequant dual txt {quant}")
    ws_ = I.single_block_weights(s, 0)
    assert_parity(run_single(s, ws_, x, ids, quant=q), oracle_single(s, dequantised(ws_, q), x, ids), "bf16",
                  f"fused-dequant single {quant}")


def test_blocks_bf16_full_width_two_batches():
    # h 3072, batch 2, 77 text + 48x48 image tokens: the 256x256 GEMM's gated
    # residual rows cross a batch boundary inside a tile (image rows per batch
    # 2304), and the joint attention runs over two (batch, head) sets
    s = I.Shape(txt_len=77, grid_h=48, grid_w=48, batch=2, dtype="bf16", cfg_id=39)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    w = I.double_block_weights(s, 0)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "bf16", "two-batch dual img")
    assert_parity(txt, rtxt, "bf16", "two-batch dual txt")
    ws_ = I.single_block_weights(s, 0)
    assert_parity(run_single(s, ws_, x, ids), oracle_single(s, ws_, x, ids), "bf16", "two-batch single")


@pytest.mark.parametrize("policy", ["q4q8", "sub_byte"])
def test_blocks_quantised_weights_bf16(policy):
    # h 1024: small problems, the register-staged GEMM dequantises B
    s = I.Shape(hidden=1024, heads=8, mlp_hidden=4096, txt_len=64, grid_h=16, grid_w=16, dtype="bf16",
                cfg_id=35)
    qp = bd.QUANT_POLICY if policy == "q4q8" else SUB_BYTE_MIX
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    w = I.double_block_weights(s, 0)
    img, txt = run_double(s, w, x, ids, quant=qp)
    rimg, rtxt = oracle_double(s, dequantised(w, qp), x, ids)
    assert_parity(img, rimg, "bf16", f"{policy} dual img")
    assert_parity(txt, rtxt, "bf16", f"{policy} dual txt")
    ws_ = I.single_block_weights(s, 0)
    got = run_single(s, ws_, x, ids, quant=qp)
    assert_parity(got, oracle_single(s, dequantised(ws_, qp), x, ids), "bf16", f"{policy} single")


# ------------------------------------------------------------ properties ----
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gate_zero_is_bit_exact_identity(dtype):
    s = I.Shape(hidden=512, heads=4, mlp_hidden=1024, txt_len=40, grid_h=8, grid_w=10, dtype=dtype, cfg_id=33)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    img, txt = run_double(s, I.zero_modulation(I.double_block_weights(s, 0)), x, ids)
    assert np.array_equal(img, x["x_img"]) and np.array_equal(txt, x["x_txt"])
    out = run_single(s, I.zero_modulation(I.single_block_weights(s, 0)), x, ids)
    assert np.array_equal(out, x["x"])


def test_in_place_equals_out_of_place():
    s = I.Shape(hidden=512, heads=4, mlp_hidden=1024, txt_len=33, grid_h=7, grid_w=9, dtype="bf16", cfg_id=34)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    w = I.double_block_weights(s, 0)
    a = run_double(s, w, x, ids)
    b = run_double(s, w, x, ids, inplace=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    ws_ = I.single_block_weights(s, 0)
    assert np.array_equal(run_single(s, ws_, x, ids), run_single(s, ws_, x, ids, inplace=True))


def test_blocks_are_deterministic():
    s = I.Shape(hidden=1024, heads=8, mlp_hidden=2048, txt_len=100, grid_h=20, grid_w=20, dtype="bf16", cfg_id=36)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    w = I.double_block_weights(s, 0)
    a = run_double(s, w, x, ids)
    b = run_double(s, w, x, ids)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_small_workspace_leaves_outputs_untouched():
    t = torch()
    s = I.Shape(hidden=256, heads=2, mlp_hidden=512, txt_len=8, grid_h=4, grid_w=4, dtype="bf16", cfg_id=37)
    dims = bd.make_dims(s)
    W = bd.SingleW(I.single_block_weights(s, 0), bd.BF16, "cuda")
    wc = W.c()
    x = I.block_inputs(s)
    xin = up(x["x"], "bf16")
    out = t.full_like(xin, 7.0)
    need = bd.mmdit_single_block_workspace(dims)
    ws = workspace(need - 256)
    with pytest.raises(bd.MMDiTError) as e:
        bd.mmdit_single_block_fwd(dims, wc, xin, out, up(x["vec"], "bf16"),
                                  up_i32(oracle.make_ids(4, 4, 8)), ws)
    assert e.value.status == 4
    sync()
    assert bool((out == 7.0).all())


# ------------------------------------------------- attention in isolation ----
# With the second gate (dual) or the MLP half of linear2 (single) zeroed and
# the out-projection bias zero, a block's output minus its input is the
# attention branch alone, linear in the attention output O. The block input
# is scaled by 2^-6 (exact in bf16; LayerNorm is scale-invariant, so the
# attention inputs are the same up to the epsilon), which keeps the bf16
# rounding of the output small against that difference. A relative error e
# in O then shows as about e in the difference (tests/test_attention_isolation.py
# pins this on the oracle), where the whole block's output moves by only
# about 0.4 e.
def _small_inputs(x):
    return {k: (v * np.float32(2.0 ** -6) if k != "vec" else v) for k, v in x.items()}


def _delta_parity(got_out, ref_out, x_in, what):
    d_got = np.asarray(got_out, np.float64) - x_in
    d_ref = np.asarray(ref_out, np.float64) - x_in
    return assert_parity(d_got, d_ref, "bf16", what)


ISO_CASES = {
    "cfg3": I.CFG3,
    "cfg2_sharp": I.CFG2,
    # 512 text + 4096 generated + 4096 context tokens (L 8704, 24 heads: 816
    # units, the last 48 split along the keys over 256 workers and merged)
    "ref8704": I.Shape(txt_len=512, grid_h=64, grid_w=128, dtype="bf16", cfg_id=54),
    # h 1024 (8 heads), 77 + 40x41 = 1717 tokens: a ragged last key tile in
    # split units (56 tail units)
    "split_ragged": I.Shape(hidden=1024, heads=8, mlp_hidden=2048, txt_len=77, grid_h=40, grid_w=41,
                            dtype="bf16", cfg_id=59),
}


@pytest.mark.parametrize("case", list(ISO_CASES))
def test_attention_branch_isolated(case):
    # cfg3: 512 text + 4096 image tokens (L 4608); cfg2_sharp: 1280 tokens
    # with QK RMSNorm scales times 3 (the online softmax's rescaling path)
    s = ISO_CASES[case]
    x = _small_inputs(I.block_inputs(s))
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    if case == "ref8704":
        ids = np.concatenate([oracle.make_ids(64, 64, 512), oracle.make_ids(64, 64, 0, frame=1)])
    w = I.attention_only(I.double_block_weights(s, 0))
    if case == "cfg2_sharp":
        w = _sharpened(w, 3.0)
    img, txt = run_double(s, w, x, ids)
    rimg, rtxt = oracle_double(s, w, x, ids)
    _delta_parity(img, rimg, x["x_img"], f"{case} dual attention branch, image rows")
    _delta_parity(txt, rtxt, x["x_txt"], f"{case} dual attention branch, text rows")
    del w, rimg, rtxt
    ws_ = I.attention_only(I.single_block_weights(s, 0))
    if case == "cfg2_sharp":
        ws_ = _sharpened(ws_, 3.0)
    _delta_parity(run_single(s, ws_, x, ids), oracle_single(s, ws_, x, ids), x["x"],
                  f"{case} single attention branch")


def test_blocks_mixed_stream_formats_below_decoding_rows():
    # text stream dense, image stream 4-bit / 8-bit (and the reverse), 320
    # rows: the register-staged GEMM runs each format as its own launch
    s = I.Shape(hidden=1024, heads=8, mlp_hidden=4096, txt_len=64, grid_h=16, grid_w=16, dtype="bf16",
                cfg_id=57)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    w = I.double_block_weights(s, 0)
    for qs in ("img", "txt"):
        t = torch()
        dims = bd.make_dims(s)
        streams = {st: bd.StreamW.from_numpy(w[st], bd.BF16, "cuda", bd.QUANT_POLICY if st == qs else None)
                   for st in ("img", "txt")}
        W = bd.DoubleW(None, img=streams["img"], txt=streams["txt"])
        img, txt = up(x["x_img"], "bf16"), up(x["x_txt"], "bf16")
        img_o, txt_o = t.empty_like(img), t.empty_like(txt)
        ws = workspace(bd.mmdit_double_block_workspace(dims))
        print(f"mixed formats: {qs} stream quantised", flush=True)
        bd.mmdit_double_block_fwd(dims, W.c(), img, txt, img_o, txt_o, up(x["vec"], "bf16"), up_i32(ids), ws)
        sync()
        wo = dict(w)
        wo[qs] = dequantised(w[qs], bd.QUANT_POLICY)
        rimg, rtxt = oracle_double(s, wo, x, ids)
        assert_parity(down(img_o), rimg, "bf16", f"mixed formats ({qs} quantised) img")
        assert_parity(down(txt_o), rtxt, "bf16", f"mixed formats ({qs} quantised) txt")


def test_blocks_float32_residual_with_bf16_operands():
    # dims.resid = MMDIT_RESID_F32: bf16 operands, float32 block inputs and
    # outputs (the residual the step keeps), 256 text + 32x32 image tokens
    t = torch()
    s = I.CFG2
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    dims = bd.make_dims(s, resid=bd.RESID_F32)
    w = I.double_block_weights(s, 0)
    W = bd.DoubleW(w, bd.BF16, "cuda")
    img, txt = up(x["x_img"], "f32"), up(x["x_txt"], "f32")
    vec = up(x["vec"], "bf16")
    ws = workspace(bd.mmdit_double_block_workspace(dims))
    print("double block, float32 residual", flush=True)
    bd.mmdit_double_block_fwd(dims, W.c(), img, txt, img, txt, vec, up_i32(ids), ws)
    sync()
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert img.dtype == t.float32
    assert_parity(down(img), rimg, "bf16", "f32-residual dual img")
    assert_parity(down(txt), rtxt, "bf16", "f32-residual dual txt")
    ws_ = I.single_block_weights(s, 0)
    S_ = bd.SingleW(ws_, bd.BF16, "cuda")
    xin = up(x["x"], "f32")
    out = t.empty_like(xin)
    print("single block, float32 residual", flush=True)
    bd.mmdit_single_block_fwd(dims, S_.c(), xin, out, vec, up_i32(ids), ws)
    sync()
    assert_parity(down(out), oracle_single(s, ws_, x, ids), "bf16", "f32-residual single")


# Gated-residual GEMMs with fewer than 128 tiles of 256 x 256 are split along
# k (float32 partial sums, then a reduce that applies bias, gate and
# residual). Ways per launch (k-ranges) in these shapes:
# - h 1536, m 3072, 77 + 600 tokens: out-projection 3 (1536 / 64 k-tiles
#   allow no more), fc2 4, linear2 4;
# - h 1024, m 4096, no text, 2 x 320 image tokens, float32 residual:
#   out-projection 2, fc2 4, linear2 4 (the text problem is empty).
SPLIT_K_CASES = {
    "three_ways_ragged": (I.Shape(hidden=1536, heads=12, mlp_hidden=3072, txt_len=77, grid_h=24, grid_w=25,
                                  dtype="bf16", cfg_id=81), False),
    "two_ways_f32_residual_batch2": (I.Shape(hidden=1024, heads=8, mlp_hidden=4096, txt_len=0, grid_h=16,
                                             grid_w=20, batch=2, dtype="bf16", cfg_id=82), True),
}


@pytest.mark.parametrize("case", sorted(SPLIT_K_CASES))
def test_blocks_split_k_gated_residual(case):
    t = torch()
    s, f32_resid = SPLIT_K_CASES[case]
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    dims = bd.make_dims(s, resid=bd.RESID_F32) if f32_resid else bd.make_dims(s)
    rd = "f32" if f32_resid else "bf16"
    w = I.double_block_weights(s, 0)
    W = bd.DoubleW(w, bd.BF16, "cuda")
    img, txt = up(x["x_img"], rd), up(x["x_txt"], rd)
    img_o, txt_o = t.empty_like(img), t.empty_like(txt)
    vec = up(x["vec"], "bf16")
    ws = workspace(bd.mmdit_double_block_workspace(dims))
    print(f"split-k double block {case}", flush=True)
    bd.mmdit_double_block_fwd(dims, W.c(), img, txt, img_o, txt_o, vec, up_i32(ids), ws)
    sync()
    rimg, rtxt = oracle_double(s, w, x, ids)
    assert_parity(down(img_o), rimg, "bf16", f"split-k {case} img")
    if s.txt_len:
        assert_parity(down(txt_o), rtxt, "bf16", f"split-k {case} txt")
    ws_ = I.single_block_weights(s, 0)
    S_ = bd.SingleW(ws_, bd.BF16, "cuda")
    xin = up(x["x"], rd)
    out = t.empty_like(xin)
    wss = workspace(bd.mmdit_single_block_workspace(dims))
    print(f"split-k single block {case}", flush=True)
    bd.mmdit_single_block_fwd(dims, S_.c(), xin, out, vec, up_i32(ids), wss)
    sync()
    assert_parity(down(out), oracle_single(s, ws_, x, ids), "bf16", f"split-k {case} single")


def test_blocks_full_width_between_128_and_200_tiles():
    # h 3072, no text, 20 x 32 image tokens (640 rows): fc1 has 144 tiles of
    # 256 x 256 and takes the direct-to-LDS kernel with the GELU epilogue in
    # one partial round; QKV has 108 (register-staged kernel, separate QK
    # pass); the out-projection, fc2 and linear2 (36 tiles each) are split
    # along k in 4 ranges; linear1 has 252 (fused QK and split GELU)
    s = I.Shape(txt_len=0, grid_h=20, grid_w=32, dtype="bf16", cfg_id=83)
    x = I.block_inputs(s)
    ids = oracle.make_ids(s.grid_h, s.grid_w, s.txt_len)
    w = I.double_block_weights(s, 0)
    img, _ = run_double(s, w, x, ids)
    rimg, _ = oracle_double(s, w, x, ids)
    assert_parity(img, rimg, "bf16", "640-row dual img")
    ws_ = I.single_block_weights(s, 0)
    assert_parity(run_single(s, ws_, x, ids), oracle_single(s, ws_, x, ids), "bf16", "640-row single")
