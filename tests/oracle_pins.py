"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each ``pin_*`` function takes a loaded oracle and raises AssertionError when
the oracle disagrees with something the pages or the mathematics fix:
library routines for number formats and the Sylvester Hadamard matrix,
closed forms (orthogonality, involution, Parseval), invariants (rotation
invariance, codebook-prefix property, linearity, thread determinism),
an independent numpy brute force on tiny shapes, a hand-derived case, and the
storage worked example printed in the paper's appendix "Estimating Model
Size".  The pins are chosen so that a plausible slip anywhere in the oracle
(a dropped term, a wrong sign or index, a transposed operand, a wrong
rounding) makes at least one of them fail; the mutant test checks exactly
that by compiling altered copies of the oracle.

Run as a script (``python tests/oracle_pins.py LIB``) it loads the oracle at
LIB, runs every pin and exits with the number of failures.
"""
from __future__ import annotations

import json
import os
import sys
import traceback

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

GOLDEN = os.path.join(ROOT, "tests", "golden")


def _rng(tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(0x0AC1E000 + tag))


def _sylvester(b: int) -> np.ndarray:
    import scipy.linalg
    return scipy.linalg.hadamard(b).astype(np.int64)


def _np_blockdiag_rotate(x: np.ndarray, b: int) -> np.ndarray:
    """Independent rotation: reshape into blocks and multiply by scipy's Hadamard / sqrt(b)."""
    H = _sylvester(b).astype(np.float64) / np.sqrt(b)
    B, d = x.shape
    return (x.reshape(B, d // b, b) @ H.T).reshape(B, d)


def _np_weights(codes: np.ndarray, cb: np.ndarray, s: np.ndarray, k: int) -> np.ndarray:
    """Independent reconstruction by fancy indexing: W[i, 8j+t] = s_i * sum_m cb[m, codes[i,j,m], t]."""
    d_out, G, M = codes.shape
    cbd = cb.astype(np.float64)
    acc = np.zeros((d_out, G, 8))
    for m in range(k):
        acc = acc + cbd[m][codes[:, :, m]]
    return s.astype(np.float64)[:, None] * acc.reshape(d_out, G * 8)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def pin_f16_decode_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = orc.decode(bits, "f16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_f16_encode_matches_numpy(orc):
    g = _rng(1)
    v = np.concatenate([
        g.standard_normal(20000) * 10.0 ** g.uniform(-9, 5, 20000),      # wide range incl. subnormal, overflow
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 6.0e-8]),
    ])
    # exact midpoints between neighbouring fp16 values: ties go to the even significand
    h = np.arange(0x0001, 0x7BFF, 97, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    v = np.concatenate([v, (lo + hi) / 2, -(lo + hi) / 2])
    ref = v.astype(np.float16).view(np.uint16)
    got = orc.encode(v, "f16")
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {v[bad[:5]]} got {got[bad[:5]]} ref {ref[bad[:5]]}"


def pin_bf16_decode_all_patterns(orc):
    import torch
    bits = np.arange(65536, dtype=np.int32).astype(np.int16)
    ref = torch.from_numpy(bits).view(torch.bfloat16).to(torch.float64).numpy()
    got = orc.decode(bits.view(np.uint16), "bf16")
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def pin_bf16_encode_matches_torch(orc):
    import torch
    g = _rng(2)
    # float32-representable inputs, so torch's float32 -> bfloat16 rounding is a single rounding
    v32 = (g.standard_normal(20000) * 10.0 ** g.uniform(-40, 38, 20000)).astype(np.float32)
    v32 = v32[np.isfinite(v32)]
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.encode(v32.astype(np.float64), "bf16")
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first {v32[bad[:5]]}"
    # ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    assert orc.encode(np.array([1 + 2.0 ** -8]), "bf16")[0] == 0x3F80
    assert orc.encode(np.array([1 + 3 * 2.0 ** -8]), "bf16")[0] == 0x3F82


def pin_formats_roundtrip(orc):
    for dt in ("f16", "bf16"):
        bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        v = orc.decode(bits, dt)
        fin = np.isfinite(v)
        back = orc.encode(v[fin], dt)
        assert np.array_equal(back, bits[fin]), dt


# ---------------------------------------------------------------------------
# Hadamard rotation
# ---------------------------------------------------------------------------

def pin_hadamard_orthogonal(orc):
    for b in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        H = orc.hadamard(b).astype(np.int64)
        assert np.array_equal(H @ H.T, b * np.eye(b, dtype=np.int64)), b


def pin_hadamard_is_sylvester(orc):
    for b in (2, 8, 64, 128, 256):
        assert np.array_equal(orc.hadamard(b).astype(np.int64), _sylvester(b)), b
    for b in (32, 64, 128):
        H = orc.hadamard(b).astype(np.int64)
        H2 = orc.hadamard(2 * b).astype(np.int64)
        assert np.array_equal(H2, np.block([[H, H], [H, -H]])), b


def pin_rotation_closed_forms(orc):
    g = _rng(3)
    for b in (64, 128, 256):
        d = 2 * b
        x = g.standard_normal((3, d))
        y = orc.rotate(x, b)
        # orthonormal: Parseval per block and involution (H/sqrt(b) is symmetric, squares to I)
        assert np.allclose(np.linalg.norm(y.reshape(3, 2, b), axis=2), np.linalg.norm(x.reshape(3, 2, b), axis=2), rtol=1e-13)
        assert np.allclose(orc.rotate(y, b), x, rtol=0, atol=1e-12)
        # unit vectors map to Hadamard columns / sqrt(b); the all-ones block maps to sqrt(b) e_0
        H = _sylvester(b).astype(np.float64)
        for c in (0, 1, b // 2 + 3, b - 1):
            e = np.zeros((1, d))
            e[0, b + c] = 1.0
            col = orc.rotate(e, b)
            assert np.allclose(col[0, :b], 0.0, atol=0)
            assert np.allclose(col[0, b:], H[:, c] / np.sqrt(b), rtol=0, atol=1e-15)
        ones = np.ones((1, d))
        r = orc.rotate(ones, b)
        target = np.zeros(d)
        target[0] = target[b] = np.sqrt(b)
        assert np.allclose(r[0], target, rtol=0, atol=1e-12)
        # blocks are independent: changing block 0 leaves block 1 untouched
        x2 = x.copy()
        x2[:, :b] += 1.0
        assert np.array_equal(orc.rotate(x2, b)[:, b:], y[:, b:])


def pin_rotation_matches_numpy(orc):
    g = _rng(4)
    for b, d in ((64, 256), (128, 512), (256, 1024)):
        x = g.standard_normal((2, d))
        assert np.allclose(orc.rotate(x, b), _np_blockdiag_rotate(x, b), rtol=0, atol=1e-12)


def pin_rotation_invariance(orc):
    """W x = (W Q^T)(Q x) for a dense random W: the weight-side rotation cancels the activation-side one."""
    g = _rng(5)
    for b in (64, 256):
        d_in = 2 * b
        W = g.standard_normal((7, d_in))
        x = g.standard_normal((1, d_in))
        WQt = orc.rotate(W, b)          # rows of W rotated = W Q^T (Q symmetric)
        Qx = orc.rotate(x, b)
        assert np.allclose(WQt @ Qx[0], W @ x[0], rtol=1e-12, atol=1e-12)


def _np_eps(signs: np.ndarray, d_in: int) -> np.ndarray:
    """Independent sign expansion with numpy's little-endian bit unpacking: bit c % 8 of byte c // 8."""
    bits = np.unpackbits(np.asarray(signs, dtype=np.uint8), bitorder="little")[:d_in]
    return 1.0 - 2.0 * bits.astype(np.float64)


def pin_sign_mask_layout(orc):
    """Worked by hand: bytes 0x05, 0x80 flip inputs 0, 2 and 15; every other input keeps its sign."""
    eps = orc.sign_vector(np.array([0x05, 0x80, 0x00], dtype=np.uint8), 24)
    want = np.ones(24)
    want[[0, 2, 15]] = -1.0
    assert np.array_equal(eps, want), eps


def pin_signed_rotation_special_cases(orc):
    """No bits set is the unsigned rotation; every bit set negates it; one bit negates one input."""
    g = _rng(6)
    for b in (64, 128, 256):
        d = 2 * b
        x = g.standard_normal((2, d))
        zero = np.zeros(d // 8, dtype=np.uint8)
        full = np.full(d // 8, 0xFF, dtype=np.uint8)
        assert np.array_equal(orc.rotate_signed(x, zero, b), orc.rotate(x, b))
        assert np.array_equal(orc.rotate_signed(x, full, b), -orc.rotate(x, b))
        for c in (0, 7, b + 9, d - 1):
            one = zero.copy()
            one[c // 8] = 1 << (c % 8)
            xf = x.copy()
            xf[:, c] = -xf[:, c]
            assert np.allclose(orc.rotate_signed(x, one, b), _np_blockdiag_rotate(xf, b), rtol=0, atol=1e-12), c


def pin_signed_rotation_closed_forms(orc):
    """R = H diag(eps)/sqrt(b): R e_c = eps_c H[:, c]/sqrt(b); R^T R = I; Q (R x) = eps * x."""
    g = _rng(7)
    for b in (64, 128, 256):
        d = 2 * b
        signs = g.integers(0, 256, d // 8, dtype=np.uint8)
        eps = _np_eps(signs, d)
        H = _sylvester(b).astype(np.float64)
        R = orc.rotate_signed(np.eye(d), signs, b).T          # column c = R e_c
        for c in range(d):
            blk, cc = divmod(c, b)
            want = np.zeros(d)
            want[blk * b:(blk + 1) * b] = eps[c] * H[:, cc] / np.sqrt(b)
            assert np.allclose(R[:, c], want, rtol=0, atol=1e-15), (b, c)
        assert np.allclose(R.T @ R, np.eye(d), rtol=0, atol=1e-13)
        x = g.standard_normal((3, d))
        assert np.allclose(orc.rotate(orc.rotate_signed(x, signs, b), b), x * eps, rtol=0, atol=1e-12)
        assert np.allclose(orc.rotate_signed(x, signs, b), _np_blockdiag_rotate(x * eps, b), rtol=0, atol=1e-12)


def pin_signed_rotation_invariance(orc):
    """W x = (W R^T)(R x): rotating the weight rows by R cancels the randomized activation rotation."""
    g = _rng(8)
    for b in (64, 256):
        d_in = 2 * b
        signs = g.integers(0, 256, d_in // 8, dtype=np.uint8)
        W = g.standard_normal((7, d_in))
        x = g.standard_normal((1, d_in))
        WRt = orc.rotate_signed(W, signs, b)   # row i of W R^T is R w_i
        Rx = orc.rotate_signed(x, signs, b)
        assert np.allclose(WRt @ Rx[0], W @ x[0], rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# reconstruction and product
# ---------------------------------------------------------------------------

def _tiny(tag: int, d_out: int, d_in: int, M: int, batch: int = 1):
    g = _rng(tag)
    return (wl.gen_codes(g, d_out, d_in, M), wl.gen_codebooks(g, M), wl.gen_scales(g, d_out),
            wl.gen_x(g, batch, d_in, "f16"))


def pin_reconstruct_matches_numpy(orc):
    codes, cb, s, _ = _tiny(6, 5, 128, 3)
    for k in (1, 2, 3):
        W = orc.reconstruct(codes, cb, s, k)
        assert np.allclose(W, _np_weights(codes, cb, s, k), rtol=1e-15, atol=0), k


def pin_bruteforce_tiny(orc):
    """d_out in {1,2,3}, d_in = 64, M = 2, b = 64, every k, batch 1 and 2, against numpy."""
    for d_out in (1, 2, 3):
        for batch in (1, 2):
            codes, cb, s, x = _tiny(10 + d_out + 7 * batch, d_out, 64, 2, batch)
            xd = x.astype(np.float64)
            for k in (1, 2):
                W = _np_weights(codes, cb, s, k)
                ref = _np_blockdiag_rotate(xd, 64) @ W.T
                got = orc.forward(codes, cb, s, k, x, 64)
                assert got.shape == (batch, d_out)
                assert np.allclose(got, ref, rtol=1e-12, atol=1e-14), (d_out, batch, k)


def pin_hand_case(orc):
    """A case worked by hand.

    d_out = 2, d_in = 64 (8 groups), M = 2, b = 64, s = (1, 2).
    C_0[3][t] = (t+1)/8, C_1[5][t] = -1/2, every other codeword 0.
    Row 0 uses codes (3, 5) in every group; row 1 uses (3, 0) in group 0 and (0, 0) elsewhere.
    x = e_0: rotated x is the all-ones vector / 8, so y_i = s_i/8 * (sum of row i of W):
      k=1: row 0 sums 8 * 36/8 = 36 -> 4.5 ; row 1 sums 36/8 = 4.5 -> 2 * 4.5/8 = 1.125
      k=2: row 0 adds 8 * 8 * (-1/2) = -32 -> (36 - 32)/8 = 0.5 ; row 1 unchanged (C_1[0] = 0).
    x = e_1: rotated x alternates +1/8, -1/8 (column 1 of H), so each group contributes
      sum_t w_t (-1)^t / 8 ; for C_0[3]: (1-2+3-4+5-6+7-8)/8/8 = -1/16, for C_1[5]: 0.
      row 0: 8 * (-1/16) = -0.5 for k = 1 and 2 ; row 1: 2 * (-1/16) = -0.125.
    """
    codes = np.zeros((2, 8, 2), dtype=np.uint8)
    codes[0, :, 0], codes[0, :, 1] = 3, 5
    codes[1, 0, 0] = 3
    cb = np.zeros((2, 256, 8), dtype=np.float16)
    cb[0, 3, :] = (np.arange(8) + 1) / 8.0
    cb[1, 5, :] = -0.5
    s = np.array([1.0, 2.0], dtype=np.float16)
    e0 = np.zeros((1, 64), dtype=np.float16)
    e0[0, 0] = 1
    e1 = np.zeros((1, 64), dtype=np.float16)
    e1[0, 1] = 1
    assert np.array_equal(orc.forward(codes, cb, s, 1, e0, 64)[0], [4.5, 1.125])
    assert np.array_equal(orc.forward(codes, cb, s, 2, e0, 64)[0], [0.5, 1.125])
    assert np.array_equal(orc.forward(codes, cb, s, 1, e1, 64)[0], [-0.5, -0.125])
    assert np.array_equal(orc.forward(codes, cb, s, 2, e1, 64)[0], [-0.5, -0.125])


def pin_prefix_property(orc):
    """Keeping k codebooks equals keeping all M with codebooks k..M-1 set to zero;
    the step from k-1 to k is the contribution of codebook k-1 alone."""
    codes, cb, s, x = _tiny(20, 6, 128, 4)
    xr = orc.rotate(x, 128)
    for k in (1, 2, 3, 4):
        cbz = cb.copy()
        cbz[k:] = 0
        assert np.array_equal(orc.linear(codes, cbz, s, 4, xr), orc.linear(codes, cb, s, k, xr)), k
    for k in (2, 3, 4):
        only = np.zeros_like(cb)
        only[k - 1] = cb[k - 1]
        step = orc.linear(codes, cb, s, k, xr) - orc.linear(codes, cb, s, k - 1, xr)
        alone = orc.linear(codes, only, s, k, xr)
        assert np.allclose(step, alone, rtol=1e-12, atol=1e-13), k


def pin_linearity(orc):
    codes, cb, s, _ = _tiny(30, 4, 256, 2)
    g = _rng(31)
    x1, x2 = g.standard_normal((1, 256)), g.standard_normal((1, 256))
    f = lambda x, sc=s: orc.forward(codes, cb, sc, 2, x, 64)  # noqa: E731
    assert np.allclose(f(x1 + x2), f(x1) + f(x2), rtol=1e-12, atol=1e-13)
    assert np.array_equal(f(4.0 * x1), 4.0 * f(x1))              # power-of-two scaling is exact
    s2 = (2 * s.astype(np.float64)).astype(np.float16)            # exact doubling in fp16
    assert np.array_equal(f(x1, s2), 2.0 * f(x1))


def pin_forward_is_rotate_then_linear(orc):
    codes, cb, s, x = _tiny(40, 3, 256, 2, 2)
    for k in (1, 2):
        assert np.array_equal(orc.forward(codes, cb, s, k, x, 128), orc.linear(codes, cb, s, k, orc.rotate(x, 128)))


def pin_thread_determinism(orc):
    codes, cb, s, x = _tiny(50, 64, 512, 3, 2)
    prev = orc.set_threads(1)
    a = orc.forward(codes, cb, s, 3, x, 128)
    orc.set_threads(4)
    b = orc.forward(codes, cb, s, 3, x, 128)
    orc.set_threads(prev)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# packed layout and storage
# ---------------------------------------------------------------------------

def _byte_compare(a: np.ndarray, b: np.ndarray, what: str):
    """Byte comparison that reports the failing positions; comparing nothing is a failure."""
    assert a.size > 0 and a.size == b.size, f"{what}: nothing to compare or size mismatch"
    bad = np.nonzero(a.reshape(-1) != b.reshape(-1))[0]
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at {bad[:8].tolist()}"


def _np_tiles(codes: np.ndarray) -> np.ndarray:
    """Independent construction of the packed tiles with numpy reshapes:
    pad to whole 16-row x 64-group tiles, then order [m][group tile][row tile][group][row]."""
    d_out, G, M = codes.shape
    R, T = -(-d_out // 16), -(-G // 64)
    pad = np.zeros((R * 16, T * 64, M), dtype=np.uint8)
    pad[:d_out, :G, :] = codes
    t = pad.reshape(R, 16, T, 64, M)          # [it][r][jt][l][m]
    return np.ascontiguousarray(t.transpose(4, 2, 0, 3, 1)).reshape(-1)


def pin_pack_roundtrip_and_prefix(orc):
    g = _rng(60)
    for d_out, G, M in ((3, 5, 4), (16, 64, 2), (37, 130, 3), (1, 1, 1)):
        codes = g.integers(0, 256, size=(d_out, G, M), dtype=np.uint8)
        packed = orc.pack(codes)
        _byte_compare(packed, _np_tiles(codes), "pack vs numpy tiles")
        _byte_compare(orc.unpack(packed, d_out, G, M), codes, "unpack(pack)")
        plane = packed.size // M
        for k in range(1, M + 1):
            _byte_compare(packed[: k * plane], orc.pack(codes[:, :, :k]), f"prefix k={k}")
        # a hand-located byte: plane m, row i, group j
        m, i, j = M - 1, d_out - 1, G - 1
        R = -(-d_out // 16)
        assert packed[m * plane + ((j // 64) * R + i // 16) * 1024 + (j % 64) * 16 + i % 16] == codes[i, j, m]


def pin_storage_worked_example(orc):
    with open(os.path.join(GOLDEN, "storage_worked_example.json")) as f:
        ex = json.load(f)
    v = orc.bits_per_param(ex["d_out"], ex["d_in"], ex["group"], ex["codebooks"], ex["code_bits"])
    assert round(v, ex["printed_decimals"]) == ex["bits_per_parameter_printed"], v
    # smallest layer worked by hand: one row of 8 inputs, one 1-bit codebook:
    # codebook 8*1*2*16 = 256 bits, codes 1*1*1*1 = 1 bit, scale 16 bits
    assert orc.storage_bits(1, 8, 8, 1, 1) == 273.0
    # codes dominate: M codebooks of 8-bit codes over groups of 8 give M bits per weight plus overhead
    for M in (1, 2, 3, 4):
        assert M < orc.bits_per_param(4096, 14336, 8, M, 8) < M + 0.01


# ---------------------------------------------------------------------------
# encode side: greedy residual code assignment
# ---------------------------------------------------------------------------

def _sign_codebooks(M: int) -> np.ndarray:
    """Codebook m holds every +-8^-m sign pattern: codeword c has +8^-m at element t where bit t of c is
    set, -8^-m elsewhere (fp16-exact)."""
    bits = (np.arange(256)[:, None] >> np.arange(8)[None, :]) & 1
    pat = np.where(bits == 1, 1.0, -1.0)
    return np.stack([pat * 8.0 ** -m for m in range(M)]).astype(np.float16)


def pin_encode_planted_codes(orc):
    """Targets that are exact sums of one +-1, one +-1/8, one +-1/64 and one +-1/512 sign pattern: at each
    stage the remaining scales add up to less than the gap to a wrong sign, so the greedy search must
    return exactly the planted codes, plane by plane."""
    g = _rng(20)
    M, d_out, G = 4, 5, 12
    cb = _sign_codebooks(M)
    planted = g.integers(0, 256, size=(d_out, G, M))
    target = np.zeros((d_out, G, 8))
    for m in range(M):
        target += cb[m].astype(np.float64)[planted[:, :, m]]
    codes = orc.encode_greedy(target.reshape(d_out, G * 8).astype(np.float32), cb)
    assert np.array_equal(codes, planted.astype(np.uint8))
    # a prefix of the planes only: the first two planes come out the same
    assert np.array_equal(orc.encode_greedy(target.reshape(d_out, G * 8).astype(np.float32), cb[:2]),
                          planted[:, :, :2].astype(np.uint8))


def pin_encode_is_stagewise_nearest(orc):
    """Gaussian targets, N(0, 0.05) codebooks: every stage picks a nearest codeword to the residual left by
    the earlier stages (checked in float64 against all 256; float32 rounding may only break near-ties)."""
    g = _rng(21)
    M, d_out, d_in = 3, 7, 96
    cb = wl.gen_codebooks(g, M)
    target = (g.standard_normal((d_out, d_in)) * 0.1).astype(np.float32)
    codes = orc.encode_greedy(target, cb)
    C = cb.astype(np.float64)
    r = target.astype(np.float64).reshape(d_out, d_in // 8, 8)
    for m in range(M):
        d = ((r[:, :, None, :] - C[m][None, None, :, :]) ** 2).sum(-1)        # [d_out][G][256]
        chosen = np.take_along_axis(d, codes[:, :, m][:, :, None].astype(np.int64), axis=2)[..., 0]
        assert np.all(chosen <= d.min(axis=2) * (1 + 1e-5) + 1e-12), m
        r = r - C[m][codes[:, :, m]]


def pin_encode_ties_go_to_lower_index(orc):
    """Equal codewords: the lower index wins.  A target equal to a codeword leaves a zero residual, after
    which the next plane picks its shortest codeword (the first one among equals)."""
    g = _rng(22)
    cb = (g.standard_normal((2, 256, 8)) * 0.05).astype(np.float16)
    cb[0, 9] = cb[0, 5]
    cb[0, 200] = cb[0, 5]
    cb[1, 77] = 0.0
    cb[1, 140] = 0.0
    target = cb[0, 5].astype(np.float32)[None, :]
    codes = orc.encode_greedy(target, cb)
    assert codes[0, 0, 0] == 5 and codes[0, 0, 1] == 77, codes


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]


def run_all(lib_path: str) -> int:
    import oracle
    orc = oracle.Oracle(lib_path)
    failures = 0
    for pin in PINS:
        try:
            pin(orc)
        except Exception:  # noqa: BLE001
            failures += 1
            print(f"FAIL {pin.__name__}: {traceback.format_exc().strip().splitlines()[-1]}")
    return failures


if __name__ == "__main__":
    n = run_all(sys.argv[1])
    print(f"{n} pin failures")
    sys.exit(min(n, 100))
