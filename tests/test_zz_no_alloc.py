"""aqd_gemv_noalloc, the GEMV entry point that allocates nothing (needs an MI355X).

It must give aqd_gemv's bits on the same inputs, call after call on the shared
scratch array, the second call with a smaller input, on every route (batch 1
and 2 through the lookup tables, batch 4 at k = 2 through the four-column
tables, batch 8 on the matrix cores, the codeword-gather kernel for inputs too
long for the tables), and stay within the
oracle's tolerance (Drop-by-Drop, sections 3.2 and 5).  Runs alone in a fresh
process or after the other tests.
"""
import numpy as np
import pytest
import torch

import additive_codebook_gemv_amd as aqd
import oracle
import workloads as wl
from tests.gpu_util import TOL, dev, normwise, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def orc():
    o = oracle.load()
    o.set_threads(16)
    return o


def _layer(seed, d_out, d_in, M):
    g = wl.rng(seed, extra=d_out + d_in + M)
    codes, cb, s = wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out)
    x = wl.gen_x(g, 8, d_in, "f16")                     # stands for an already rotated activation
    return codes, cb, s, x


@pytest.mark.parametrize("first,second", [
    ((4096, 14336, 4, 4, 1), (1024, 4096, 4, 2, 1)),    # batch 1 (tables), then a smaller layer
    ((4096, 4096, 4, 3, 2), (300, 1000, 3, 3, 2)),      # batch 2 (two-column tables), ragged second
    ((14336, 4096, 4, 4, 8), (4096, 4096, 4, 2, 4)),    # batch 8 on the matrix cores, then batch 4 (4-column tables)
    ((16, 65536, 8, 8, 1), (16, 8192, 8, 8, 1)),        # codeword gathers (too long for the tables), then tables
])
def test_noalloc_matches_gemv_twice(orc, first, second):
    for call, (d_out, d_in, M, k, B) in enumerate((first, second)):
        codes, cb, s, x = _layer(700 + call, d_out, d_in, M)
        packed, cbd, sd = aqd.aqd_pack_codes(to_dev(codes)), to_dev(cb), to_dev(s)
        xd = to_dev(x[:B])
        y0 = torch.full((B, d_out), float("nan"), dtype=torch.float16, device=dev())
        aqd.aqd_gemv_noalloc(packed, cbd, sd, k, xd, d_out, d_in, M, out=y0)
        ref_gpu = aqd.aqd_gemv(packed, cbd, sd, k, xd, d_out, d_in, M)
        torch.cuda.synchronize()
        assert torch.equal(y0, ref_gpu), (call, d_out, d_in, k, B)
        e = normwise(y0.float().cpu().numpy(), orc.linear(codes, cb, s, k, x[:B]))
        assert e <= TOL, (call, e)


def test_noalloc_repeat_and_rejects_oversize(orc):
    d_out, d_in, M = 1024, 4096, 4
    codes, cb, s, x = _layer(710, d_out, d_in, M)
    packed, cbd, sd = aqd.aqd_pack_codes(to_dev(codes)), to_dev(cb), to_dev(s)
    xd = to_dev(x[:1])
    ys = [aqd.aqd_gemv_noalloc(packed, cbd, sd, 3, xd, d_out, d_in, M) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], y) for y in ys[1:])
    # a layer whose workspace exceeds the fixed array is refused before anything is enqueued
    big = 1 << 22
    assert aqd.aqd_gemv_workspace_bytes(big, 4096, 4, 8) > aqd.AQD_NOALLOC_SCRATCH_BYTES
    y = torch.empty((8, 16), dtype=torch.float16, device=dev())
    with pytest.raises(aqd.AqdError) as ei:
        aqd.aqd_gemv_noalloc(packed, cbd, sd, 1, to_dev(x), big, 4096, 4, out=y)
    assert ei.value.status == 8
