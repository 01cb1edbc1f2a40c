"""Parity of the HIP path with the fp64 CPU oracle (needs an MI355X).

Every comparison calls the product through the C ABI (the Python binding is
argument marshalling only) and the oracle on the same seeded inputs:
- integer / byte work (code packing) must be bit-exact;
- floating point must be within 2e-3 max normwise relative error
  (max |gpu - oracle| / max |oracle|) of the fp64 oracle, for the GEMV both
  against the oracle fed the GPU's own fp16 rotated activation and against the
  pure fp64 path from the raw activation;
- inputs built so that every partial sum is exact (dyadic codewords, +-1
  activations) must give bit-identical results.
"""
import numpy as np
import pytest
import torch

import additive_codebook_gemv_amd as aqd
import oracle
import workloads as wl
from tests.gpu_util import TOL, dev, normwise, record, rms_rel, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    o = oracle.load()
    o.set_threads(16)
    return o


def _layer_dev(codes, cb, s):
    return to_dev(codes), to_dev(cb), to_dev(s)


def _f16_ulp(v: np.ndarray) -> np.ndarray:
    a = np.abs(v).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)


# ---------------------------------------------------------------------------
# packing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_out,d_in,M", [(256, 256, 2), (4096, 14336, 4), (1000, 1000, 3), (1, 8, 1), (17, 520, 8)])
def test_pack_bit_exact(orc, d_out, d_in, M):
    g = wl.rng(7, kind="codes", extra=d_out + d_in + M)
    codes = wl.gen_codes(g, d_out, d_in, M)
    packed = aqd.aqd_pack_codes(to_dev(codes))
    ref = orc.pack(codes)
    got = packed.cpu().numpy()
    assert got.size == ref.size
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8].tolist()}"
    back = aqd.aqd_unpack_codes(packed, d_out, d_in, M).cpu().numpy()
    assert np.array_equal(back, codes)
    # the first k planes are exactly the packing of the first k codebooks
    plane = got.size // M
    for k in range(1, M + 1):
        pk = aqd.aqd_pack_codes(to_dev(np.ascontiguousarray(codes[:, :, :k]))).cpu().numpy()
        assert np.array_equal(pk, got[: k * plane]), k


# ---------------------------------------------------------------------------
# rotation
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("block", [64, 128, 256])
def test_rotation_matches_oracle(orc, block):
    d_in = 14336 if block == 256 else 4096
    x = wl.gen_x(wl.rng(11, extra=block), 8, d_in, "f16")
    xd = to_dev(x)
    ref = orc.rotate(x, block)
    f32 = aqd.aqd_hadamard_rotate(xd, block, aqd.AQD_F32).cpu().numpy()
    err32 = normwise(f32, ref)
    assert err32 < 1e-6, err32
    f16 = aqd.aqd_hadamard_rotate(xd, block, aqd.AQD_F16).cpu().numpy().astype(np.float64)
    assert np.all(np.abs(f16 - ref) <= _f16_ulp(ref)), "fp16 output more than one ulp from the exact rotation"
    x2 = aqd.aqd_hadamard_rotate(xd, block, aqd.AQD_BF16X2).float().cpu().numpy().astype(np.float64)
    err2 = normwise(x2[0] + x2[1], ref)
    assert err2 < 2.0 ** -15, err2
    record(test="rotation", block=block, err_f32=err32, err_bf16x2=err2)


@pytest.mark.parametrize("block", [64, 256])
def test_rotation_bit_exact_on_integers(orc, block):
    """Integer inputs with b = 64 or 256 (1/sqrt(b) a power of two): every sum is exact."""
    g = wl.rng(12, extra=block)
    x = g.integers(-8, 9, size=(3, 4 * block)).astype(np.float16)
    got = aqd.aqd_hadamard_rotate(to_dev(x), block, aqd.AQD_F16).cpu().numpy().view(np.uint16)
    ref = orc.encode(orc.rotate(x, block), "f16")
    assert np.array_equal(got, ref)


def test_rotation_bf16_input_and_in_place(orc):
    x = wl.gen_x(wl.rng(13), 4, 1024, "bf16")
    ref = orc.rotate(x, 128, "bf16")
    got = aqd.aqd_hadamard_rotate(to_dev(x, bf16_bits=True), 128, aqd.AQD_F32).cpu().numpy()
    assert normwise(got, ref) < 1e-6
    xf = wl.gen_x(wl.rng(14), 2, 512, "f16")
    t = to_dev(xf)
    out = aqd.aqd_hadamard_rotate(t, 64, aqd.AQD_F16, out=t)        # in place
    assert out.data_ptr() == t.data_ptr()
    assert np.all(np.abs(t.cpu().numpy().astype(np.float64) - orc.rotate(xf, 64)) <= _f16_ulp(orc.rotate(xf, 64)))


def _eps(signs: np.ndarray, d_in: int) -> np.ndarray:
    return 1.0 - 2.0 * np.unpackbits(signs, bitorder="little")[:d_in].astype(np.float64)


@pytest.mark.parametrize("block", [64, 128, 256])
def test_signed_rotation_matches_oracle(orc, block):
    """H diag(eps) / sqrt(b): the oracle's randomized rotation within rounding, and the bits of the
    unsigned rotation of the sign-flipped input (a negation is exact)."""
    d_in = 14336 if block == 256 else 4096
    g = wl.rng(15, extra=block)
    x = wl.gen_x(g, 4, d_in, "f16")
    signs = wl.gen_signs(g, d_in)
    xd, sd = to_dev(x), to_dev(signs)
    ref = orc.rotate_signed(x, signs, block)
    f32 = aqd.aqd_hadamard_rotate_signed(xd, block, sd, aqd.AQD_F32).cpu().numpy()
    err32 = normwise(f32, ref)
    assert err32 < 1e-6, err32
    f16 = aqd.aqd_hadamard_rotate_signed(xd, block, sd, aqd.AQD_F16)
    assert np.all(np.abs(f16.cpu().numpy().astype(np.float64) - ref) <= _f16_ulp(ref))
    flipped = to_dev((x.astype(np.float64) * _eps(signs, d_in)).astype(np.float16))
    assert torch.equal(f16, aqd.aqd_hadamard_rotate(flipped, block, aqd.AQD_F16))
    zero = torch.zeros_like(sd)
    assert torch.equal(aqd.aqd_hadamard_rotate_signed(xd, block, zero, aqd.AQD_F16),
                       aqd.aqd_hadamard_rotate(xd, block, aqd.AQD_F16))
    t = xd.clone()
    aqd.aqd_hadamard_rotate_signed(t, block, sd, aqd.AQD_F16, out=t)        # in place
    assert torch.equal(t, f16)
    record(test="signed_rotation", block=block, err_f32=err32)


@pytest.mark.parametrize("block", [64, 256])
def test_signed_rotation_bit_exact_on_integers(orc, block):
    g = wl.rng(16, extra=block)
    x = g.integers(-8, 9, size=(3, 4 * block)).astype(np.float16)
    signs = wl.gen_signs(g, 4 * block)
    got = aqd.aqd_hadamard_rotate_signed(to_dev(x), block, to_dev(signs), aqd.AQD_F16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, orc.encode(orc.rotate_signed(x, signs, block), "f16"))


# ---------------------------------------------------------------------------
# GEMV (batch 1..8)
# ---------------------------------------------------------------------------

def _check_gemv_layer(orc, cid, lin, rows=None):
    bmax = max(lin.batches)
    codes, cb, s, x = wl.layer_inputs(cid, lin, batch=bmax)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    xr = aqd.aqd_hadamard_rotate(to_dev(x), lin.block, aqd.AQD_F16)
    xr_np = xr.cpu().numpy()
    sel = slice(None) if rows is None else rows
    c_o, s_o = (codes, s) if rows is None else (codes[rows], s[rows])
    for k in lin.ks:
        ref_lin = orc.linear(c_o, cb, s_o, k, xr_np)
        ref_full = orc.forward(c_o, cb, s_o, k, x, lin.block)
        for B in lin.batches:
            y = aqd.aqd_gemv(packed, cbdev, sdev, k, xr[:B].contiguous(), lin.d_out, lin.d_in, lin.M)
            y = y.cpu().numpy().astype(np.float64)[:, sel]
            e_lin = normwise(y, ref_lin[:B])
            e_full = normwise(y, ref_full[:B])
            record(test="gemv", cfg=cid, layer=lin.name, k=k, batch=B, err=e_full, err_same_input=e_lin,
                   rms=rms_rel(y, ref_full[:B]), sampled_rows=None if rows is None else len(rows))
            assert e_lin <= TOL and e_full <= TOL, (lin.name, k, B, e_lin, e_full)


@pytest.mark.parametrize("cid", [1, 2])
def test_gemv_config(orc, cid):
    for lin in wl.config(cid):
        _check_gemv_layer(orc, cid, lin)


@pytest.mark.parametrize("name", ["gate14336x4096", "up14336x4096", "down4096x14336"])
def test_gemv_mlp_config(orc, name):
    lin = [l for l in wl.config(3) if l.name == name][0]
    _check_gemv_layer(orc, 3, lin)


def test_gemv_stack_sampled(orc):
    """32-layer stack: three layers, all seven projections, at their seeded k; 96 sampled rows each."""
    lins = wl.config(4)
    g = np.random.Generator(np.random.PCG64(404))
    for lin in [l for l in lins if l.layer in (0, 17, 31)]:
        rows = np.sort(g.choice(lin.d_out, size=96, replace=False))
        _check_gemv_layer(orc, 4, lin, rows=rows)


@pytest.mark.parametrize("d_out,d_in,M,batches", [
    (1000, 1000, 3, (1, 2, 3, 8)),    # ragged rows (not a multiple of 16) and groups (not a multiple of 64)
    (1, 8, 1, (1, 2)),                # one row, one group
    (33, 4096, 8, (1, 2, 5)),         # M = 8 codebooks, every k
    (2048, 512, 2, (7,)),
    (16, 65536, 4, (1, 2, 4)),        # at k = 4 too long for the batch-2 tables (k * d_in / 512 > 510); batch 4:
                                      # four-column tables at k = 1 (128 slices), other routes above
    (16, 130560, 4, (1, 2, 3)),       # 255 table slices, the most a row sum counts: batch 1 at k = 4, batch 2 at k = 2,
                                      # batch 3 at k = 1
])
def test_gemv_edge_shapes(orc, d_out, d_in, M, batches):
    g = wl.rng(21, extra=d_out * 7 + d_in + M)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    xr = wl.gen_x(g, max(batches), d_in, "f16")          # stands for an already rotated activation
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    for k in range(1, M + 1):
        ref = orc.linear(codes, cb, s, k, xr)
        for B in batches:
            y = aqd.aqd_gemv(packed, cbdev, sdev, k, to_dev(xr[:B]), d_out, d_in, M).cpu().numpy()
            e = normwise(y, ref[:B])
            record(test="gemv_edge", shape=[d_out, d_in, M], k=k, batch=B, err=e)
            assert e <= TOL, (k, B, e)


def test_gemv_tall_layer_many_rounds(orc):
    """2^20 rows over 512 inputs: the batch-1, batch-2, four-column and matrix-core routes all plan
    several rounds of workgroups (1024 or more for the table routes, with four row tiles per wave).
    Sampled rows, the first and the last among them, against the oracle."""
    d_out, d_in, M = 1 << 20, 512, 2
    g = wl.rng(41, extra=d_out)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    x = wl.gen_x(g, 8, d_in, "f16")                      # stands for an already rotated activation
    packed = aqd.aqd_pack_codes(to_dev(codes))
    cbd, sd = to_dev(cb), to_dev(s)
    pick = np.random.Generator(np.random.PCG64(42)).choice(d_out, size=254, replace=False)
    rows = np.unique(np.concatenate([[0, d_out - 1], pick]))
    for k in (1, 2):
        ref = orc.linear(codes[rows], cb, s[rows], k, x)
        for B in (1, 2, 4, 8):
            y = aqd.aqd_gemv(packed, cbd, sd, k, to_dev(x[:B]), d_out, d_in, M).cpu().numpy()[:, rows]
            e = normwise(y, ref[:B])
            record(test="gemv_tall", shape=[d_out, d_in, M], k=k, batch=B, err=e)
            assert e <= TOL, (k, B, e)
    del packed


def test_gemv_empty_input_gives_zero():
    d_out = 40
    s = to_dev(np.ones(d_out, dtype=np.float16))
    y = torch.full((2, d_out), 7.0, dtype=torch.float16, device=dev())
    aqd.aqd_gemv(torch.empty(0, dtype=torch.uint8, device=dev()), torch.empty(0, dtype=torch.float16, device=dev()),
                 s, 1, torch.empty((2, 0), dtype=torch.float16, device=dev()), d_out, 0, 2, out=y)
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("d_out,d_in,M", [(256, 256, 2), (100, 1000, 4)])
def test_gemv_dyadic_bit_exact(orc, d_out, d_in, M):
    codes, cb, s, x = wl.dyadic_case(wl.rng(31, extra=d_out), d_out, d_in, M, batch=8)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    for k in range(1, M + 1):
        ref = orc.linear(codes, cb, s, k, x)
        assert np.max(np.abs(ref)) < 512          # every value and partial sum is exact in fp16/fp32
        for B in (1, 2, 3, 4, 8):
            y = aqd.aqd_gemv(packed, cbdev, sdev, k, to_dev(x[:B]), d_out, d_in, M).cpu().numpy()
            assert np.array_equal(y.astype(np.float64), ref[:B]), (k, B)


def test_gemv_prefix_property(orc):
    """Keeping k codebooks equals keeping all four with codebooks k.. zeroed."""
    lin = wl.config(2)[0]
    codes, cb, s, x = wl.layer_inputs(2, lin)
    cdev, sdev = to_dev(codes), to_dev(s)
    packed = aqd.aqd_pack_codes(cdev)
    xr = to_dev(wl.gen_x(wl.rng(41), 1, lin.d_in, "f16"))
    for k in (1, 2, 3):
        cbz = cb.copy()
        cbz[k:] = 0
        yk = aqd.aqd_gemv(packed, to_dev(cb), sdev, k, xr, lin.d_out, lin.d_in, 4).cpu().numpy().astype(np.float64)
        yz = aqd.aqd_gemv(packed, to_dev(cbz), sdev, 4, xr, lin.d_out, lin.d_in, 4).cpu().numpy().astype(np.float64)
        assert normwise(yz, yk) <= 1e-3, k


def test_gemv_rejects_bad_k_on_device():
    lin = wl.config(1)[0]
    codes, cb, s, x = wl.layer_inputs(1, lin)
    with pytest.raises(aqd.AqdError) as ei:
        aqd.aqd_gemv(aqd.aqd_pack_codes(to_dev(codes)), to_dev(cb), to_dev(s), 3, to_dev(x), 256, 256, 2)
    assert ei.value.status == 3


# ---------------------------------------------------------------------------
# small batch on the matrix cores
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["gate14336x4096_sb", "down4096x14336_sb"])
def test_small_batch_config(orc, name):
    lin = [l for l in wl.config(5) if l.name == name][0]
    codes, cb, s, x = wl.layer_inputs(5, lin, batch=64)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    xd = to_dev(x, bf16_bits=True)
    xr = aqd.aqd_hadamard_rotate(xd, lin.block, aqd.AQD_BF16X2)
    xr16 = aqd.aqd_hadamard_rotate(xd, lin.block, aqd.AQD_F16)
    for k in lin.ks:
        ref = orc.forward(codes, cb, s, k, x, lin.block, "bf16")
        for B in lin.batches:
            xb = xr[:, :B].contiguous()
            y = aqd.aqd_gemm_small_batch(packed, cbdev, sdev, k, xb, lin.d_out, lin.d_in, 4, aqd.AQD_BF16X2)
            e = normwise(y.cpu().numpy(), ref[:B])
            record(test="small_batch", mode="bf16x2", layer=name, k=k, batch=B, err=e,
                   rms=rms_rel(y.cpu().numpy(), ref[:B]))
            assert e <= TOL, (k, B, e)
            yf = aqd.aqd_gemm_small_batch(packed, cbdev, sdev, k, xr16[:B].contiguous(), lin.d_out, lin.d_in, 4,
                                          aqd.AQD_F16)
            ef = normwise(yf.cpu().numpy(), ref[:B])
            record(test="small_batch", mode="f16", layer=name, k=k, batch=B, err=ef,
                   rms=rms_rel(yf.cpu().numpy(), ref[:B]))
            assert ef <= TOL, (k, B, ef)


@pytest.mark.parametrize("d_out,d_in,M,batches", [(1000, 1000, 3, (1, 17, 64)), (16, 64, 1, (16,))])
def test_small_batch_edge_shapes(orc, d_out, d_in, M, batches):
    g = wl.rng(51, extra=d_out + d_in)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    x = g.standard_normal((max(batches), d_in)).astype(np.float32)
    xt = torch.from_numpy(x).to(dev())
    hi = xt.to(torch.bfloat16)
    lo = (xt - hi.float()).to(torch.bfloat16)
    xx = torch.stack([hi, lo])                       # AQD_BF16X2 operand of an already rotated activation
    x_exact = hi.double().cpu().numpy() + lo.double().cpu().numpy()
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    for k in range(1, M + 1):
        ref = orc.linear(codes, cb, s, k, x_exact)
        for B in batches:
            y = aqd.aqd_gemm_small_batch(packed, cbdev, sdev, k, xx[:, :B].contiguous(), d_out, d_in, M,
                                         aqd.AQD_BF16X2).cpu().numpy()
            e = normwise(y, ref[:B])
            record(test="small_batch_edge", shape=[d_out, d_in, M], k=k, batch=B, err=e)
            assert e <= TOL, (k, B, e)
            y1 = aqd.aqd_gemm_small_batch(packed, cbdev, sdev, k, hi[:B].contiguous(), d_out, d_in, M,
                                          aqd.AQD_BF16).cpu().numpy()
            r1 = orc.linear(codes, cb, s, k, hi[:B].double().cpu().numpy())
            assert normwise(y1, r1) <= TOL, (k, B)


def test_small_batch_dyadic_bit_exact(orc):
    d_out, d_in, M = 200, 512, 2
    codes, cb, s, x = wl.dyadic_case(wl.rng(61), d_out, d_in, M, batch=32)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    xb = torch.from_numpy(x.astype(np.float32)).to(dev()).to(torch.bfloat16).contiguous()
    xh = torch.from_numpy(x).to(dev()).contiguous()
    for k in (1, 2):
        ref = orc.linear(codes, cb, s, k, x)
        y = aqd.aqd_gemm_small_batch(packed, cbdev, sdev, k, xb, d_out, d_in, M, aqd.AQD_BF16).cpu().numpy()
        assert np.array_equal(y.astype(np.float64), ref), k
        yh = aqd.aqd_gemm_small_batch(packed, cbdev, sdev, k, xh, d_out, d_in, M, aqd.AQD_F16).cpu().numpy()
        assert np.array_equal(yh.astype(np.float64), ref), k


def test_quantized_linear_forward(orc):
    """The resident-layer helper: rotate + product, both batch regimes."""
    lin = wl.config(2)[0]
    codes, cb, s, _ = wl.layer_inputs(2, lin)
    q = aqd.QuantizedLinear(to_dev(codes), to_dev(cb), to_dev(s), lin.block)
    for B in (1, 4, 16):
        x = wl.gen_x(wl.rng(71, extra=B), B, lin.d_in, "f16")
        y = q.forward(to_dev(x), 3).float().cpu().numpy()
        ref = orc.forward(codes, cb, s, 3, x, lin.block)
        assert normwise(y, ref) <= TOL, B


def test_gemv_workspace_reusable_and_deterministic(orc):
    """The batch-1 path keeps partials and counters in the workspace: its counters must be zero again after
    every call (so one buffer serves the next call), and repeated calls must give the same bits."""
    lin = wl.config(2)[0]
    codes, cb, s, x = wl.layer_inputs(2, lin)
    packed = aqd.aqd_pack_codes(to_dev(codes))
    need = aqd.aqd_gemv_workspace_bytes(lin.d_out, lin.d_in, lin.M, 1)
    ws = torch.zeros(need, dtype=torch.uint8, device=dev())
    xr = aqd.aqd_hadamard_rotate(to_dev(x), lin.block, aqd.AQD_F16)
    outs = []
    for k in (4, 1, 4, 2):
        outs.append(aqd.aqd_gemv(packed, to_dev(cb), to_dev(s), k, xr, lin.d_out, lin.d_in, 4, workspace=ws))
        torch.cuda.synchronize()
        assert torch.count_nonzero(ws).item() == 0, k
    assert torch.equal(outs[0], outs[2])       # same inputs, same bits
    ref = orc.forward(codes, cb, s, 2, x, lin.block)
    assert normwise(outs[3].cpu().numpy(), ref) <= TOL
    # one buffer sized for batch 8 serves batch 8 (matrix-core route, partial sums after the batch-1
    # region) and then batch 1: the batch-1 region is still zero and batch 1 gives the same bits
    need8 = aqd.aqd_gemv_workspace_bytes(lin.d_out, lin.d_in, lin.M, 8)
    assert need8 > need
    ws8 = torch.zeros(need8, dtype=torch.uint8, device=dev())
    x8 = aqd.aqd_hadamard_rotate(to_dev(wl.gen_x(wl.rng(42), 8, lin.d_in, "f16")), lin.block, aqd.AQD_F16)
    y8 = aqd.aqd_gemv(packed, to_dev(cb), to_dev(s), 4, x8, lin.d_out, lin.d_in, 4, workspace=ws8)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws8[:need]).item() == 0
    y1 = aqd.aqd_gemv(packed, to_dev(cb), to_dev(s), 4, xr, lin.d_out, lin.d_in, 4, workspace=ws8)
    assert torch.equal(y1, outs[0])
    assert torch.equal(aqd.aqd_gemv(packed, to_dev(cb), to_dev(s), 4, x8, lin.d_out, lin.d_in, 4, workspace=ws8), y8)
    # batch 2 (lookup tables of two columns) shares the zeroed region: it leaves it zero, repeats its bits,
    # and batch 1 after it is unchanged
    y2 = [aqd.aqd_gemv(packed, to_dev(cb), to_dev(s), k, x8[:2].contiguous(), lin.d_out, lin.d_in, 4, workspace=ws8)
          for k in (3, 3)]
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws8[:need]).item() == 0
    assert torch.equal(y2[0], y2[1])
    ref2 = orc.linear(codes, cb, s, 3, x8[:2].cpu().numpy())
    assert normwise(y2[0].cpu().numpy(), ref2) <= TOL
    assert torch.equal(aqd.aqd_gemv(packed, to_dev(cb), to_dev(s), 4, xr, lin.d_out, lin.d_in, 4, workspace=ws8),
                       outs[0])


def test_graph_replay_matches_eager(orc):
    """Rotation, batch-1 GEMV and small-batch product captured in one HIP graph: every replay, with eager
    work on the same workspaces in between, gives the eager result bit for bit."""
    lin = wl.config(2)[0]
    codes, cb, s, x = wl.layer_inputs(2, lin)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    xd = to_dev(x)
    xs = to_dev(wl.gen_x(wl.rng(81), 32, lin.d_in, "f16"))
    ws1 = torch.zeros(max(aqd.aqd_gemv_workspace_bytes(lin.d_out, lin.d_in, lin.M, 1), 16), dtype=torch.uint8,
                      device=dev())
    ws2 = torch.zeros(max(aqd.aqd_gemm_small_batch_workspace_bytes(lin.d_out, lin.d_in, lin.M, 32), 16),
                      dtype=torch.uint8, device=dev())
    xr = torch.empty_like(xd)
    xsr = torch.empty_like(xs)
    y1 = torch.empty((1, lin.d_out), dtype=torch.float16, device=dev())
    y2 = torch.empty((32, lin.d_out), dtype=torch.float32, device=dev())

    def work():
        aqd.aqd_hadamard_rotate(xd, lin.block, aqd.AQD_F16, out=xr)
        aqd.aqd_gemv(packed, cbdev, sdev, 3, xr, lin.d_out, lin.d_in, lin.M, out=y1, workspace=ws1)
        aqd.aqd_hadamard_rotate(xs, lin.block, aqd.AQD_F16, out=xsr)
        aqd.aqd_gemm_small_batch(packed, cbdev, sdev, 2, xsr, lin.d_out, lin.d_in, lin.M, aqd.AQD_F16, out=y2,
                                 workspace=ws2)

    work()
    torch.cuda.synchronize()
    e1, e2 = y1.clone(), y2.clone()
    stream = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            work()
    stream.wait_stream(side)
    for rep in range(3):
        y1.zero_()
        y2.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y1, e1), rep
        assert torch.equal(y2, e2), rep
        # eager calls on the same workspaces between replays
        aqd.aqd_gemv(packed, cbdev, sdev, 1, xr, lin.d_out, lin.d_in, lin.M, workspace=ws1)
        aqd.aqd_gemm_small_batch(packed, cbdev, sdev, 4, xsr, lin.d_out, lin.d_in, lin.M, aqd.AQD_F16,
                                 workspace=ws2)
        torch.cuda.synchronize()
    ref = orc.forward(codes, cb, s, 3, x, lin.block)
    assert normwise(e1.float().cpu().numpy(), ref) <= TOL


@pytest.mark.parametrize("shapes,d_in,k", [
    ([4096, 1024, 1024], 4096, 3),           # q, k, v of the 8B-shaped stack
    ([14336, 14336], 4096, 2),               # gate, up
    ([14336, 14336], 4096, 4),               # gate, up with four row tiles per wave (one round of workgroups)
    ([1000, 0, 33, 16], 1000, 2),            # ragged rows and groups, an empty linear, four linears
    ([14336, 1024, 4096], 4096, 3),          # members that take 4 and 2 table slots: one launch per slot count
])
def test_grouped_gemv_matches_separate_calls(orc, shapes, d_in, k):
    """One launch over several linears sharing the input gives, per linear, the bits of its own aqd_gemv
    call, and the oracle's result within tolerance."""
    g = wl.rng(91, extra=d_in + sum(shapes))
    M = 4
    x = wl.gen_x(g, 1, d_in, "f16")
    xr = to_dev(x)                                # treated as already rotated
    lins, refs = [], []
    for d_out in shapes:
        codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
        cdev, cbdev, sdev = _layer_dev(codes, cb, s)
        packed = aqd.aqd_pack_codes(cdev)
        lins.append((packed, cbdev, sdev, d_out, M))
        refs.append((codes, cb, s))
    outs = aqd.aqd_gemv_grouped(lins, k, xr, d_in)
    for (packed, cbdev, sdev, d_out, _), y, (codes, cb, s) in zip(lins, outs, refs):
        if d_out == 0:
            continue
        single = aqd.aqd_gemv(packed, cbdev, sdev, k, xr, d_out, d_in, M)
        assert torch.equal(y, single), d_out
        ref = orc.linear(codes, cb, s, k, x)
        e = normwise(y.float().cpu().numpy(), ref)
        record(test="gemv_grouped", d_out=d_out, d_in=d_in, k=k, err=e)
        assert e <= TOL, (d_out, e)


@pytest.mark.parametrize("shapes,d_in,block,k", [
    ([4096, 1024, 1024], 4096, 128, 3),     # q, k, v with their rotation
    ([4096], 14336, 256, 4),                 # down projection
    ([14336, 14336], 4096, 128, 3),          # gate, up with four row tiles per wave
    ([300, 17], 576, 64, 2),                 # ragged rows, a partial group tile, block 64
    ([64], 256, 256, 1),
])
def test_rotate_gemv_grouped_matches_rotate_then_gemv(orc, shapes, d_in, block, k):
    """The launch that rotates its own input gives the bits of the standalone rotation followed by the
    grouped GEMV, and the oracle's rotate-then-multiply within tolerance."""
    g = wl.rng(97, extra=d_in + block + sum(shapes))
    M = 4
    x = wl.gen_x(g, 1, d_in, "f16")
    xd = to_dev(x)
    lins, refs = [], []
    for d_out in shapes:
        codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
        cdev, cbdev, sdev = _layer_dev(codes, cb, s)
        lins.append((aqd.aqd_pack_codes(cdev), cbdev, sdev, d_out, M))
        refs.append((codes, cb, s))
    fused = aqd.aqd_rotate_gemv_grouped(lins, k, xd, d_in, block)
    xr = aqd.aqd_hadamard_rotate(xd, block, aqd.AQD_F16)
    split = aqd.aqd_gemv_grouped(lins, k, xr, d_in)
    for y, y2, (codes, cb, s), d_out in zip(fused, split, refs, shapes):
        assert torch.equal(y, y2), d_out
        ref = orc.forward(codes, cb, s, k, x, block)
        e = normwise(y.float().cpu().numpy(), ref)
        record(test="rotate_gemv_grouped", d_out=d_out, d_in=d_in, block=block, k=k, err=e)
        assert e <= TOL, (d_out, e)


@pytest.mark.parametrize("shapes,d_in,block,k", [
    ([4096, 1024, 1024], 4096, 128, 4),     # q, k, v
    ([4096], 14336, 256, 2),                 # down projection
    ([300, 17], 576, 64, 3),                 # ragged rows, a partial group tile
    ([14336, 14336], 4096, 128, 4),          # gate, up: four slots on one group tile, rotated in registers
    ([4096], 14336, 256, 4),                 # down, rotated in registers
    ([8200], 4224, 128, 4),                  # in registers with ragged rows and a half-empty last group tile
])
def test_rotate_gemv_grouped_signed(orc, shapes, d_in, block, k):
    """Randomized rotation inside the launch: the bits of the signed standalone rotation followed by the
    grouped GEMV, and the oracle's signed rotation then product within tolerance."""
    g = wl.rng(98, extra=d_in + block + sum(shapes))
    M = 4
    x = wl.gen_x(g, 1, d_in, "f16")
    signs = wl.gen_signs(g, d_in)
    xd, sd = to_dev(x), to_dev(signs)
    lins, refs = [], []
    for d_out in shapes:
        codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
        cdev, cbdev, sdev = _layer_dev(codes, cb, s)
        lins.append((aqd.aqd_pack_codes(cdev), cbdev, sdev, d_out, M))
        refs.append((codes, cb, s))
    fused = aqd.aqd_rotate_gemv_grouped_signed(lins, k, xd, d_in, block, sd)
    xr = aqd.aqd_hadamard_rotate_signed(xd, block, sd, aqd.AQD_F16)
    split = aqd.aqd_gemv_grouped(lins, k, xr, d_in)
    xrot = orc.rotate_signed(x, signs, block)
    for y, y2, (codes, cb, s), d_out in zip(fused, split, refs, shapes):
        assert torch.equal(y, y2), d_out
        ref = orc.linear(codes, cb, s, k, xrot)
        e = normwise(y.float().cpu().numpy(), ref)
        record(test="rotate_gemv_grouped_signed", d_out=d_out, d_in=d_in, block=block, k=k, err=e)
        assert e <= TOL, (d_out, e)


def test_quantized_linear_signed(orc):
    """A layer with a sign mask: batch 1 (one launch), 4 (GEMV), 16 (small batch) and 130 (prefill)."""
    g = wl.rng(99)
    d_out, d_in, M, block, k = 512, 1024, 4, 128, 3
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    signs = wl.gen_signs(g, d_in)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    ql = aqd.QuantizedLinear(cdev, cbdev, sdev, block, signs=to_dev(signs))
    for batch in (1, 4, 16, 130):
        x = wl.gen_x(g, batch, d_in, "f16")
        y = ql.forward(to_dev(x), k).float().cpu().numpy()
        ref = orc.linear(codes, cb, s, k, orc.rotate_signed(x, signs, block))
        e = normwise(y, ref)
        record(test="quantized_linear_signed", batch=batch, err=e)
        assert e <= TOL, (batch, e)


@pytest.mark.parametrize("name,ks", [
    ("down4096x14336_sb", [4] * 4 + [3] * 4 + [2] * 4 + [1] * 4),          # tiers sorted by descending k
    ("gate14336x4096_sb", [2, 4, 1, 3] * 8),                               # unsorted, 32 columns
])
def test_small_batch_tiered(orc, name, ks):
    """One launch where column n uses the first ks[n] codebooks: every column matches the oracle at its own k,
    and the single-k product of its tier within tolerance."""
    lin = [l for l in wl.config(5) if l.name == name][0]
    B = len(ks)
    codes, cb, s, _ = wl.layer_inputs(5, lin, batch=64)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    x = wl.gen_x(wl.rng(101, extra=B), B, lin.d_in, "f16")
    xd = to_dev(x)                                 # treated as already rotated
    y = aqd.aqd_gemm_small_batch_tiered(packed, cbdev, sdev, ks, xd, lin.d_out, lin.d_in, lin.M).cpu().numpy()
    for k in sorted(set(ks)):
        cols = [n for n in range(B) if ks[n] == k]
        ref = orc.linear(codes, cb, s, k, x[cols])
        e = normwise(y[cols], ref)
        record(test="small_batch_tiered", layer=name, k=k, columns=len(cols), err=e)
        assert e <= TOL, (k, e)
        single = aqd.aqd_gemm_small_batch(packed, cbdev, sdev, k, xd[cols].contiguous(), lin.d_out, lin.d_in,
                                          lin.M, aqd.AQD_F16).cpu().numpy()
        assert normwise(y[cols], single.astype(np.float64)) <= TOL, k


def test_small_batch_tiered_edge(orc):
    d_out, d_in, M = 1000, 1000, 3
    g = wl.rng(103)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    ks = [3, 1, 2, 3, 1]
    x = wl.gen_x(g, len(ks), d_in, "f16")
    y = aqd.aqd_gemm_small_batch_tiered(packed, cbdev, sdev, ks, to_dev(x), d_out, d_in, M).cpu().numpy()
    for n, k in enumerate(ks):
        ref = orc.linear(codes, cb, s, k, x[n:n + 1])
        assert normwise(y[n:n + 1], ref) <= TOL, (n, k)
    # dyadic inputs: exact in any summation order, so the tiered product is bit-exact against the oracle
    codes, cb, s, xq = wl.dyadic_case(wl.rng(105), 200, 512, 2, batch=8)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    ks = [2, 1, 1, 2, 2, 1, 2, 1]
    y = aqd.aqd_gemm_small_batch_tiered(packed, cbdev, sdev, ks, to_dev(xq), 200, 512, 2).cpu().numpy()
    for n, k in enumerate(ks):
        assert np.array_equal(y[n].astype(np.float64), orc.linear(codes, cb, s, k, xq[n:n + 1])[0]), n


# ---------------------------------------------------------------------------
# prefill / large batch on the matrix cores
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_out,d_in,M,batches", [
    (1000, 1000, 3, (1, 130, 200)),   # ragged rows, a ragged 64-input chunk, columns past one 128-column tile
    (17, 64, 2, (1, 5, 129)),         # one chunk, rows inside one fragment
    (512, 960, 4, (128,)),            # 15 chunks split one per workgroup: odd chunk counts per split
    (33, 8, 8, (3,)),                 # one group, M = 8, every k
    (600, 8192, 4, (520,)),           # 256-column tiles (batch >= 512, long inputs): ragged rows and columns
    (1000, 1000, 3, (300,)),          # 256-column tiles from batch 256 on short inputs
    (40, 600, 3, (1030,)),            # k = 3: fp16 weights staged once (batch >= 1024): ragged rows, groups,
                                      # chunks, columns; one-chunk splits with the zero padding chunk
    (33, 8, 8, (512,)),               # k >= 5 staged from 512 columns: one group (the rest of its tile
                                      # zeroed), M = 8
    (1000, 1000, 3, (1100,)),         # k = 3 staged: several row blocks, a ragged last 256-column tile
])
def test_prefill_edge_shapes(orc, d_out, d_in, M, batches):
    g = wl.rng(51, extra=d_out * 7 + d_in + M)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    xr = wl.gen_x(g, max(batches), d_in, "f16")          # stands for an already rotated activation
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    for k in range(1, M + 1):
        ref = orc.linear(codes, cb, s, k, xr)
        for B in batches:
            y = aqd.aqd_gemm_prefill(packed, cbdev, sdev, k, to_dev(xr[:B]), d_out, d_in, M).cpu().numpy()
            e = normwise(y, ref[:B])
            record(test="prefill_edge", shape=[d_out, d_in, M], k=k, batch=B, err=e)
            assert e <= TOL, (k, B, e)


def test_prefill_dyadic_bit_exact(orc):
    """Exact arithmetic: every split, chunk and column of the tiled product gives the oracle's bits, with
    the weights rebuilt per workgroup (160 and 600 columns: 128- and 256-column tiles) and, at k = 4,
    staged once as fp16 (1040 columns)."""
    d_out, d_in, M = 300, 2048, 4
    codes, cb, s, x = wl.dyadic_case(wl.rng(52), d_out, d_in, M, batch=1040)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    for k in (1, 4):
        ref = orc.linear(codes, cb, s, k, x)
        for B in (160, 600, 1040):
            y = aqd.aqd_gemm_prefill(packed, cbdev, sdev, k, to_dev(x[:B]), d_out, d_in, M).cpu().numpy()
            assert np.array_equal(y.astype(np.float64), ref[:B]), (k, B)


@pytest.mark.parametrize("d_out,d_in,batch,k", [
    (4096, 14336, 512, 4),      # down projection, 512 prompt tokens
    (4096, 14336, 512, 2),
    (14336, 4096, 1024, 4),     # gate / up projection, 1024 prompt tokens
    (4096, 14336, 2048, 4),     # down projection, 2048 prompt tokens (fp16 weights staged once, split inputs)
    (4096, 14336, 2048, 2),     # rebuilt per workgroup, 256-column tiles, split inputs
    (4096, 14336, 128, 4),      # rebuilt per workgroup, 128-column tiles, split inputs
    (14336, 4096, 128, 2),
    (14336, 4096, 512, 4),      # rebuilt per workgroup, 256-column tiles, two splits
    (14336, 4096, 2048, 2),     # rebuilt per workgroup, 256-column tiles, two rounds of workgroups
    (14336, 4096, 2048, 4),     # staged weights, two rounds of workgroups
])
def test_prefill_full_size_sampled(orc, d_out, d_in, batch, k):
    """Full 8B-shape layers in the launch configuration the benchmark times; eight sampled columns
    against the oracle, and a repeated call gives the same bits."""
    M = 4
    g = wl.rng(53, extra=d_out + batch + k)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    x = wl.gen_x(g, batch, d_in, "f16")
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    xd = to_dev(x)
    y = aqd.aqd_gemm_prefill(packed, cbdev, sdev, k, xd, d_out, d_in, M)
    y2 = aqd.aqd_gemm_prefill(packed, cbdev, sdev, k, xd, d_out, d_in, M)
    assert torch.equal(y, y2)
    cols = np.sort(np.random.Generator(np.random.PCG64(54)).choice(batch, size=8, replace=False))
    ref = orc.linear(codes, cb, s, k, x[cols])
    e = normwise(y.cpu().numpy()[cols], ref)
    record(test="prefill_full", shape=[d_out, d_in], batch=batch, k=k, err=e)
    assert e <= TOL, e


def test_prefill_maximum_batch(orc):
    """The largest batch the ABI accepts (AQD_PREFILL_MAX_BATCH columns) on a small layer: columns at the
    ends of 128- and 256-column tiles and the last column against the oracle, and a bit-identical repeat."""
    B, d_out, d_in, M, k = aqd.AQD_PREFILL_MAX_BATCH, 272, 1024, 3, 3   # k = 3: staged weights
    g = wl.rng(57)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    x = wl.gen_x(g, B, d_in, "f16")
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    xd = to_dev(x)
    y = aqd.aqd_gemm_prefill(packed, cbdev, sdev, k, xd, d_out, d_in, M)
    assert torch.equal(y, aqd.aqd_gemm_prefill(packed, cbdev, sdev, k, xd, d_out, d_in, M))
    extra = np.random.Generator(np.random.PCG64(58)).choice(B, size=6, replace=False)
    cols = np.unique(np.concatenate([[0, 127, 128, 255, 256, B // 2, B - 257, B - 256, B - 1], extra]))
    ref = orc.linear(codes, cb, s, k, x[cols])
    e = normwise(y.cpu().numpy()[cols], ref)
    record(test="prefill_max_batch", shape=[d_out, d_in], batch=B, k=k, err=e)
    assert e <= TOL, e


def test_prefill_empty_input_gives_zero():
    d_out = 40
    s = to_dev(np.ones(d_out, dtype=np.float16))
    y = torch.full((130, d_out), 7.0, dtype=torch.float32, device=dev())
    aqd.aqd_gemm_prefill(torch.empty(0, dtype=torch.uint8, device=dev()),
                         torch.empty(0, dtype=torch.float16, device=dev()), s, 1,
                         torch.empty((130, 0), dtype=torch.float16, device=dev()), d_out, 0, 2, out=y)
    assert torch.count_nonzero(y).item() == 0


# ---------------------------------------------------------------------------
# encode side: greedy residual code assignment
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d_out,d_in,M", [(300, 1000, 4), (17, 64, 8), (1, 8, 1), (1000, 512, 2)])
def test_encode_bit_exact(orc, d_out, d_in, M):
    """Codes are index work: the GPU encoder returns exactly the oracle's codes (same float32 decision)."""
    g = wl.rng(61, extra=d_out + d_in + M)
    cb = wl.gen_codebooks(g, M)
    _, _, target = wl.gen_encode_targets(g, d_out, d_in, M)
    got = aqd.aqd_encode_greedy(to_dev(target), to_dev(cb)).cpu().numpy()
    want = orc.encode_greedy(target, cb)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:5].tolist()}"


def test_encode_planted_codes():
    """Sign-pattern codebooks at scales 1, 1/8, 1/64, 1/512: the planted codes come back exactly."""
    g = wl.rng(62)
    M, d_out, G = 4, 64, 40
    bits = (np.arange(256)[:, None] >> np.arange(8)[None, :]) & 1
    cb = np.stack([np.where(bits == 1, 1.0, -1.0) * 8.0 ** -m for m in range(M)]).astype(np.float16)
    planted = g.integers(0, 256, size=(d_out, G, M))
    target = np.zeros((d_out, G, 8))
    for m in range(M):
        target += cb[m].astype(np.float64)[planted[:, :, m]]
    got = aqd.aqd_encode_greedy(to_dev(target.reshape(d_out, G * 8).astype(np.float32)), to_dev(cb)).cpu().numpy()
    assert np.array_equal(got, planted.astype(np.uint8))


def test_encode_full_size_sampled_and_decoded(orc):
    """The 4096x14336 layer (M = 4): sampled rows equal the oracle's codes; the encoded layer, packed and
    run through the GEMV, reproduces the oracle's output for those codes, and the weight error falls with k."""
    d_out, d_in, M = 4096, 14336, 4
    g = wl.rng(63)
    cb = wl.gen_codebooks(g, M)
    w, s, target = wl.gen_encode_targets(g, d_out, d_in, M)
    codes = aqd.aqd_encode_greedy(to_dev(target), to_dev(cb))
    rows = np.sort(np.random.Generator(np.random.PCG64(64)).choice(d_out, size=48, replace=False))
    want = orc.encode_greedy(target[rows], cb)
    assert np.array_equal(codes.cpu().numpy()[rows], want)
    # decode side on the sampled rows: the GEMV of the GPU-encoded layer against the oracle's output for
    # the oracle's own codes of those rows
    x = wl.gen_x(g, 1, d_in, "f16")
    y = aqd.aqd_gemv(aqd.aqd_pack_codes(codes), to_dev(cb), to_dev(s), M, to_dev(x), d_out, d_in, M)
    ref = orc.linear(want, cb, s[rows], M, x)
    e = normwise(y.float().cpu().numpy()[:, rows], ref)
    assert e <= TOL, e
    # weight error of the encoded rows against the rotated weights, per k: falls with every codebook
    errs = []
    for k in range(1, M + 1):
        wk = orc.reconstruct(want, cb, s[rows], k)
        errs.append(np.linalg.norm(wk - w[rows].astype(np.float64)) / np.linalg.norm(w[rows]))
    record(test="encode_error_curve", rel_err=errs)
    assert all(a > b for a, b in zip(errs, errs[1:])), errs


# ---------------------------------------------------------------------------
# seeded random shapes across the entry points
# ---------------------------------------------------------------------------

def _random_case(seed: int, block_multiple: int = 8):
    g = np.random.Generator(np.random.PCG64(0xF00D + seed))
    d_out = int(g.integers(1, 700))
    d_in = int(g.integers(1, 1600 // block_multiple)) * block_multiple
    M = int(g.integers(1, 9))
    k = int(g.integers(1, M + 1))
    gg = wl.rng(81, extra=seed)
    return g, d_out, d_in, M, k, wl.gen_codes(gg, d_out, d_in, M), wl.gen_codebooks(gg, M), wl.gen_scales(gg, d_out)


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes_gemv_small_batch_prefill(orc, seed):
    """Random d_out (1..699), d_in (8..1592), M (1..8), k and batch: the GEMV (batch 1..8), the small batch
    (1..64) and the prefill (1..300) against the oracle on the same inputs."""
    g, d_out, d_in, M, k, codes, cb, s = _random_case(seed)
    cdev, cbdev, sdev = _layer_dev(codes, cb, s)
    packed = aqd.aqd_pack_codes(cdev)
    bg, bs, bp = int(g.integers(1, 9)), int(g.integers(1, 65)), int(g.integers(1, 301))
    x = wl.gen_x(wl.rng(82, extra=seed), max(bg, bs, bp), d_in, "f16")
    ref = orc.linear(codes, cb, s, k, x)
    cases = (
        ("gemv", bg, lambda: aqd.aqd_gemv(packed, cbdev, sdev, k, to_dev(x[:bg]), d_out, d_in, M)),
        ("small_batch", bs, lambda: aqd.aqd_gemm_small_batch(packed, cbdev, sdev, k, to_dev(x[:bs]), d_out, d_in, M,
                                                             aqd.AQD_F16)),
        ("prefill", bp, lambda: aqd.aqd_gemm_prefill(packed, cbdev, sdev, k, to_dev(x[:bp]), d_out, d_in, M)),
    )
    for name, B, fn in cases:
        y = fn().float().cpu().numpy()
        e = normwise(y, ref[:B])
        record(test="random_" + name, shape=[d_out, d_in, M], k=k, batch=B, err=e)
        assert e <= TOL, (name, d_out, d_in, M, k, B, e)


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_rotating_grouped(orc, seed):
    """Random groups of 1..4 linears sharing an input of random width (a multiple of the block), plain or
    with a sign mask: the launch that rotates its own input against the oracle's rotation and product."""
    g = np.random.Generator(np.random.PCG64(0xBEEF + seed))
    block = int(g.choice([64, 128, 256]))
    d_in = int(g.integers(1, 2048 // block + 1)) * block
    n = int(g.integers(1, 5))
    M = int(g.integers(1, 9))
    k = int(g.integers(1, M + 1))
    signed = bool(seed % 2)
    gg = wl.rng(83, extra=seed)
    x = wl.gen_x(gg, 1, d_in, "f16")
    signs = wl.gen_signs(gg, d_in)
    xrot = orc.rotate_signed(x, signs, block) if signed else orc.rotate(x, block)
    lins, refs = [], []
    for _ in range(n):
        d_out = int(g.integers(1, 900))
        codes, cb, s = wl.gen_codes(gg, d_out, d_in, M), wl.gen_codebooks(gg, M), wl.gen_scales(gg, d_out)
        cdev, cbdev, sdev = _layer_dev(codes, cb, s)
        lins.append((aqd.aqd_pack_codes(cdev), cbdev, sdev, d_out, M))
        refs.append(orc.linear(codes, cb, s, k, xrot))
    if signed:
        ys = aqd.aqd_rotate_gemv_grouped_signed(lins, k, to_dev(x), d_in, block, to_dev(signs))
    else:
        ys = aqd.aqd_rotate_gemv_grouped(lins, k, to_dev(x), d_in, block)
    for y, ref, lin in zip(ys, refs, lins):
        e = normwise(y.float().cpu().numpy(), ref)
        record(test="random_rotating_grouped", d_out=lin[3], d_in=d_in, M=M, k=k, block=block, signed=signed, err=e)
        assert e <= TOL, (lin[3], d_in, M, k, block, signed, e)
