"""Parity of launch routes and call sequences that the layer-level tests do not reach (needs an MI355X).

- QuantizedLinear across its batch regimes in an order where a small-batch
  call (split partial sums in its workspace) comes before batch-1 and batch-2
  calls (counted row sums that must start at zero);
- the batch-1 and batch-2 GEMV on inputs too long for the lookup tables (the
  codeword-gather kernel);
- the 32-layer stack exactly as the benchmark issues it: one launch per
  q/k/v group, o, gate/up group and down, each rotating its own input, every
  layer at its seeded k, checked per linear against the oracle on sampled rows;
- the rotating grouped launch on every stack shape at k = 2, 3 and 4, and on a group whose
  members choose different table slots per workgroup;
- the table paths (batch 1 and 2) over a sweep of activation and codebook
  magnitudes, since their fp16 table entries and fixed-point row sums have an
  absolute error floor.
- the small-batch kernel in its 7-wave form on a layer whose row tiles do not
  fill the last workgroup (14320 rows: 895 tiles in 128 workgroups of 7), as
  the small-batch call and as the matrix-core route of the batch-8 GEMV.
- the small-batch kernel in its 16-wave form (bf16 hi + lo operands, k = 4,
  49..64 columns: the LDS holds one workgroup per CU) on ragged rows.

Every comparison is against the fp64 oracle (Drop-by-Drop, section 3.2: the
group sums of the first k codebooks; section 5: the block rotation applied to
the activation online), within the 2e-3 normwise bound.
"""
import numpy as np
import pytest
import torch

import additive_codebook_gemv_amd as aqd
import oracle
import workloads as wl
from tests.gpu_util import TOL, dev, normwise, record, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    o = oracle.load()
    o.set_threads(16)
    return o


def _upload(codes, cb, s):
    return aqd.aqd_pack_codes(to_dev(codes)), to_dev(cb), to_dev(s)


def test_quantized_linear_batch_sequence(orc):
    """Small batch, then batch 1..4, then small batch and batch 1 again on one resident layer: every
    output matches the oracle, and the GEMV workspace's counters are zero after every batch-1..4 call."""
    lin = wl.config(2)[0]                                  # 4096 x 4096, M = 4, block 128
    codes, cb, s, _ = wl.layer_inputs(2, lin)
    q = aqd.QuantizedLinear(to_dev(codes), to_dev(cb), to_dev(s), lin.block)
    n1 = aqd.aqd_gemv_workspace_bytes(lin.d_out, lin.d_in, lin.M, 1)
    for step, (B, k) in enumerate(((16, 3), (1, 3), (2, 4), (4, 1), (16, 2), (3, 2), (1, 1), (64, 4), (4, 2),
                                    (2, 2), (1, 4))):
        x = wl.gen_x(wl.rng(601, extra=step), B, lin.d_in, "f16")
        y = q.forward(to_dev(x), k)
        torch.cuda.synchronize()
        ref = orc.forward(codes, cb, s, k, x, lin.block)
        e = normwise(y.float().cpu().numpy(), ref)
        record(test="quantized_linear_sequence", step=step, batch=B, k=k, err=e)
        assert e <= TOL, (step, B, k, e)
        if B <= 4:
            assert torch.count_nonzero(q.workspace[:n1]).item() == 0, (step, B)


def test_small_batch_seven_wave_ragged(orc):
    """14320 x 4096 plans 7-wave workgroups (4 input splits: 112 eight-wave row blocks would leave 64 CUs
    with one workgroup and the rest with two); the last workgroup holds 6 row tiles and one idle wave."""
    d_out, d_in, M = 14320, 4096, 4
    g = wl.rng(621)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    xr = wl.gen_x(g, 40, d_in, "f16")                    # stands for an already rotated activation
    packed, cbd, sd = _upload(codes, cb, s)
    for k in (2, 4):
        ref = orc.linear(codes, cb, s, k, xr)
        for B in (16, 40):
            y = aqd.aqd_gemm_small_batch(packed, cbd, sd, k, to_dev(xr[:B]), d_out, d_in, M, aqd.AQD_F16)
            e = normwise(y.cpu().numpy(), ref[:B])
            record(test="small_batch_seven_wave", k=k, batch=B, err=e)
            assert e <= TOL, (k, B, e)
        y8 = aqd.aqd_gemv(packed, cbd, sd, k, to_dev(xr[:8]), d_out, d_in, M).float().cpu().numpy()
        e8 = normwise(y8, ref[:8])
        record(test="gemv_batch8_seven_wave", k=k, err=e8)
        assert e8 <= TOL, (k, e8)


def test_small_batch_sixteen_wave_ragged(orc):
    """1000 x 4096 with bf16 hi + lo activations at 49 and 64 columns, k = 4: 63 row tiles in workgroups
    of 16 waves, the last one with 15 tiles and an idle wave."""
    d_out, d_in, M = 1000, 4096, 4
    g = wl.rng(631)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    x = g.standard_normal((64, d_in)).astype(np.float32)   # stands for an already rotated activation
    hi = torch.from_numpy(x).bfloat16()
    lo = (torch.from_numpy(x) - hi.float()).bfloat16()
    xd = torch.stack([hi, lo]).to(dev())
    xr = (hi.float() + lo.float()).numpy().astype(np.float64)
    packed, cbd, sd = _upload(codes, cb, s)
    for k in (3, 4):
        ref = orc.linear(codes, cb, s, k, xr)
        for B in (49, 64):
            y = aqd.aqd_gemm_small_batch(packed, cbd, sd, k, xd[:, :B].contiguous(), d_out, d_in, M,
                                         aqd.AQD_BF16X2)
            e = normwise(y.cpu().numpy(), ref[:B])
            record(test="small_batch_sixteen_wave", k=k, batch=B, err=e)
            assert e <= TOL, (k, B, e)


@pytest.mark.parametrize("d_out,d_in,M,batches", [
    (16, 524288, 1, (1, 2)),      # 1024 group tiles: k = 1 already needs 256 table slices (at most 255)
    (16, 65536, 8, (1,)),         # k = 8 needs 8 * 128 slots = 256 slices; k = 7 still fits the tables
])
def test_gemv_direct_route_long_inputs(orc, d_out, d_in, M, batches):
    g = wl.rng(611, extra=d_in + M)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    xr = wl.gen_x(g, max(batches), d_in, "f16")          # stands for an already rotated activation
    packed, cbd, sd = _upload(codes, cb, s)
    for k in range(1, M + 1):
        ref = orc.linear(codes, cb, s, k, xr)
        for B in batches:
            y = aqd.aqd_gemv(packed, cbd, sd, k, to_dev(xr[:B]), d_out, d_in, M).cpu().numpy()
            e = normwise(y, ref[:B])
            record(test="gemv_direct_long", shape=[d_out, d_in, M], k=k, batch=B, err=e)
            assert e <= TOL, (k, B, e)


def test_stack_fused_schedule_sampled(orc):
    """The 32-layer stack as the benchmark's token issues it: per layer aqd_rotate_gemv_grouped over
    (q, k, v), (o), (gate, up) and (down), each from its raw fp16 activation, at the layer's seeded k.
    Every linear of every layer is checked against the oracle's rotate-then-multiply on 64 sampled rows."""
    lins = wl.config(4)
    ks = wl.stack_ks()
    assert {2, 3, 4} <= set(ks)                            # every k instantiation is reached
    groups = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))
    ws = torch.zeros(max(aqd.aqd_gemv_grouped_workspace_bytes([14336, 14336], 4096, [4, 4]),
                         aqd.aqd_gemv_grouped_workspace_bytes([4096, 1024, 1024], 4096, [4, 4, 4]),
                         aqd.aqd_gemv_grouped_workspace_bytes([4096], 14336, [4])),
                     dtype=torch.uint8, device=dev())
    sel = np.random.Generator(np.random.PCG64(612))
    worst = 0.0
    for layer in range(32):
        by_proj = {l.proj: l for l in lins if l.layer == layer}
        for gi, names in enumerate(groups):
            d_in = by_proj[names[0]].d_in
            block = wl.block_for(d_in)
            k = ks[layer]
            x = wl.gen_x(wl.rng(613, layer=layer, extra=gi), 1, d_in, "f16")
            parts, host = [], []
            for p in names:
                lin = by_proj[p]
                codes, cb, s, _ = wl.layer_inputs(4, lin)
                packed, cbd, sd = _upload(codes, cb, s)
                parts.append((packed, cbd, sd, lin.d_out, lin.M))
                rows = np.sort(sel.choice(lin.d_out, size=64, replace=False))
                host.append((codes[rows], cb, s[rows], rows))
            outs = aqd.aqd_rotate_gemv_grouped(parts, k, to_dev(x), d_in, block, workspace=ws)
            for p, y, (c_r, cb, s_r, rows) in zip(names, outs, host):
                got = y.float().cpu().numpy()[:, rows]
                ref = orc.forward(c_r, cb, s_r, k, x, block)
                e = normwise(got, ref)
                worst = max(worst, e)
                assert e <= TOL, (layer, p, k, e)
            del parts, outs
        assert torch.count_nonzero(ws).item() == 0, layer
    record(test="stack_fused_schedule", layers=32, ks=ks, worst_err=worst)


@pytest.mark.parametrize("k", [2, 3, 4])
@pytest.mark.parametrize("shapes,d_in,block", [
    ([4096, 1024, 1024], 4096, 128),       # q, k, v: three linears, rotation in the launch
    ([4096], 4096, 128),                   # o: one linear that rotates its own input
    ([14336, 14336], 4096, 128),           # gate, up
    ([4096], 14336, 256),                  # down
    ([14336, 1024], 4096, 128),            # members that take 4 and 2 table slots at k = 3, 4: two launches
    ([8200], 4224, 128),                   # ragged rows, last group tile half past the input (k = 4: in registers)
])
def test_rotating_launch_every_stack_shape_and_k(orc, shapes, d_in, block, k):
    g = wl.rng(621, extra=d_in + block + sum(shapes) + k)
    M = 4
    x = wl.gen_x(g, 1, d_in, "f16")
    xd = to_dev(x)
    parts, host = [], []
    for d_out in shapes:
        codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
        parts.append((*_upload(codes, cb, s), d_out, M))
        host.append((codes, cb, s))
    fused = aqd.aqd_rotate_gemv_grouped(parts, k, xd, d_in, block)
    split = aqd.aqd_gemv_grouped(parts, k, aqd.aqd_hadamard_rotate(xd, block, aqd.AQD_F16), d_in)
    for y, y2, (codes, cb, s), d_out in zip(fused, split, host, shapes):
        assert torch.equal(y, y2), d_out
        ref = orc.forward(codes, cb, s, k, x, block)
        e = normwise(y.float().cpu().numpy(), ref)
        record(test="rotating_launch_shapes", d_out=d_out, d_in=d_in, block=block, k=k, err=e)
        assert e <= TOL, (d_out, k, e)


# Exponent pairs (activation 2^j, codebooks 2^c).  Outputs must stay inside fp16 (|y| reaches about
# 32 * 2^(j + c) here), so j + c <= 8.  The bound is asserted where the table entries
# <C_m[c], x> (RMS about 0.14 * 2^(j + c)) stay at or above about 2^-15; below that they fall into the
# fp16 subnormals and the fixed-point quantum, whose absolute floor is recorded but not asserted.
_MAG = [(j, c) for c in (-4, 0, 4) for j in range(-14, 7) if j + c <= 8]


def test_table_paths_magnitude_sweep(orc):
    d_out, d_in, M = 1024, 4096, 4
    g = wl.rng(631)
    codes, cb0, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    x0 = wl.gen_x(g, 2, d_in, "f16")
    packed = aqd.aqd_pack_codes(to_dev(codes))
    sd = to_dev(s)
    ws = torch.zeros(aqd.aqd_gemv_workspace_bytes(d_out, d_in, M, 2), dtype=torch.uint8, device=dev())
    failures = []
    for j, c in _MAG:
        # scaling by a power of two is exact unless a value leaves the fp16 normal range; both sides get
        # the same rounded inputs either way
        xs = (x0.astype(np.float64) * 2.0 ** j).astype(np.float16)
        cbs = (cb0.astype(np.float64) * 2.0 ** c).astype(np.float16)
        cbd, xd = to_dev(cbs), to_dev(xs)
        for k in (1, 4):
            ref = orc.linear(codes, cbs, s, k, xs)
            for B in (1, 2):
                y = aqd.aqd_gemv(packed, cbd, sd, k, xd[:B].contiguous(), d_out, d_in, M, workspace=ws)
                e = normwise(y.float().cpu().numpy(), ref[:B])
                record(test="table_magnitude", j=j, c=c, k=k, batch=B, err=e)
                if j + c >= -12 and not e <= TOL:
                    failures.append((j, c, k, B, e))
    assert not failures, failures
