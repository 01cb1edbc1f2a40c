"""The C ABI library on the host (no GPU needed).

- libaqd.so loads and exports every function the headers under include/ declare;
- argument validation rejects bad calls with the documented status before
  anything is enqueued (every call here fails validation, so no kernel is
  ever launched on a machine without a GPU);
- the product library does not link or load the oracle.
"""
import ctypes
import os
import re
import subprocess

import pytest

import additive_codebook_gemv_amd as aqd
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))

OK, E_NULL, E_SHAPE, E_K, E_BLOCK, E_DTYPE, E_ALIGN, E_UNSUP, E_WS, E_HIP = range(10)
F16, BF16, F32, BF16X2 = 0, 1, 2, 3
FAKE = 0x10000      # 16-byte aligned, never dereferenced: each call below fails validation first
FAKE_ODD = 0x10008  # 8-byte aligned only


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(aqd_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    return aqd.lib()


def lay(d_out=64, d_in=256, M=2, group=8, bits=8):
    return ctypes.byref(aqd.aqd_layer(d_out, d_in, M, group, bits))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 11, names
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert set(names) == set(aqd._SIGNATURES), "binding and header disagree"


def test_dynamic_symbol_table_matches_header():
    out = subprocess.run(["nm", "-D", "--defined-only", aqd.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (aqd_[a-z0-9_]+)$", out, flags=re.M))
    assert set(declared_functions()) <= exported


def test_status_strings_and_version(L):
    assert L.aqd_abi_version() == 1
    for st in range(10):
        assert L.aqd_status_string(st)
    assert L.aqd_status_string(99) == b"unknown status"


def test_packed_bytes_matches_oracle_layout(L):
    orc = oracle.load()
    for d_out, d_in, M in ((256, 256, 2), (4096, 14336, 4), (1000, 1000, 3), (1, 8, 1), (0, 128, 2)):
        got = L.aqd_packed_codes_bytes(lay(d_out, d_in, M))
        assert got == orc.packed_bytes(d_out, d_in // 8, M), (d_out, d_in, M)
    assert L.aqd_packed_codes_bytes(lay(64, 100, 2)) == 0      # d_in not a multiple of 8
    assert L.aqd_packed_codes_bytes(lay(64, 256, 2, group=4)) == 0


def _gemv(L, k=1, batch=1, layer=None, packed=FAKE, cb=FAKE, s=FAKE, x=FAKE, y=FAKE, ws=None, ws_bytes=0):
    return L.aqd_gemv(packed, cb, s, k, x, y, batch, layer if layer is not None else lay(), ws, ws_bytes, None)


def test_gemv_rejects_bad_arguments(L):
    assert _gemv(L, k=0) == E_K
    assert _gemv(L, k=3) == E_K                       # M = 2
    assert _gemv(L, batch=0) == E_SHAPE
    assert _gemv(L, batch=9) == E_SHAPE
    assert _gemv(L, layer=lay(d_in=100)) == E_SHAPE
    assert _gemv(L, layer=lay(M=0)) == E_SHAPE
    assert _gemv(L, layer=lay(M=9)) == E_SHAPE
    assert _gemv(L, layer=lay(d_out=-1)) == E_SHAPE
    assert _gemv(L, layer=lay(group=4)) == E_UNSUP
    assert _gemv(L, layer=lay(bits=4)) == E_UNSUP
    assert L.aqd_gemv(FAKE, FAKE, FAKE, 1, FAKE, FAKE, 1, None, None, 0, None) == E_NULL
    assert _gemv(L, packed=None) == E_NULL
    assert _gemv(L, cb=None) == E_NULL
    assert _gemv(L, x=None) == E_NULL
    assert _gemv(L, y=None) == E_NULL
    assert _gemv(L, s=None) == E_NULL
    assert _gemv(L, packed=FAKE_ODD) == E_ALIGN
    assert _gemv(L, x=FAKE_ODD) == E_ALIGN
    assert _gemv(L, cb=FAKE_ODD) == E_ALIGN
    assert _gemv(L, y=FAKE + 1) == E_ALIGN
    assert b"k must be" in (L.aqd_last_error() if _gemv(L, k=0) else b"")


def test_empty_layer_is_a_no_op(L):
    # d_out = 0: nothing to compute, every pointer may be NULL
    assert L.aqd_gemv(None, None, None, 1, None, None, 1, lay(d_out=0), None, 0, None) == OK
    assert L.aqd_gemm_small_batch(None, None, None, 1, None, BF16, None, 16, lay(d_out=0), None, 0, None) == OK
    assert L.aqd_hadamard_rotate(None, None, F16, F16, 0, 256, 64, None) == OK
    assert L.aqd_pack_codes(None, None, lay(d_out=0, d_in=0), None) == OK


def test_small_batch_rejects_bad_arguments(L):
    def sb(k=1, batch=16, x_dt=BF16X2, layer=None, y=FAKE, x=FAKE, ws=FAKE, ws_bytes=1 << 30):
        return L.aqd_gemm_small_batch(FAKE, FAKE, FAKE, k, x, x_dt, y, batch, layer if layer is not None else lay(),
                                      ws, ws_bytes, None)
    assert sb(batch=0) == E_SHAPE
    assert sb(batch=65) == E_SHAPE
    assert sb(k=0) == E_K
    assert sb(x_dt=F32) == E_DTYPE
    assert sb(y=FAKE + 2) == E_ALIGN
    assert sb(x=None) == E_NULL
    ks = (ctypes.c_int32 * 16)(*([2] * 8 + [1] * 8))
    tier = lambda ks_, batch=16: L.aqd_gemm_small_batch_tiered(FAKE, FAKE, FAKE, ks_, FAKE, FAKE, batch, lay(),
                                                                FAKE, 1 << 30, None)
    assert tier(None) == E_NULL
    assert tier((ctypes.c_int32 * 16)(*([3] + [1] * 15))) == E_K        # M = 2
    assert tier((ctypes.c_int32 * 16)(*([0] + [1] * 15))) == E_K
    assert tier(ks, batch=65) == E_SHAPE
    big = lay(4096, 14336, 4)
    need = L.aqd_gemm_small_batch_workspace_bytes(big, 16)
    assert need > 0                                   # the input dimension is split over workgroups
    assert sb(layer=big, ws=None, ws_bytes=0) == E_WS
    assert sb(layer=big, ws_bytes=need - 1) == E_WS


def test_hadamard_rejects_bad_arguments(L):
    def rot(x=FAKE, y=FAKE + 4096, i=F16, o=F16, batch=1, d_in=256, b=64):
        return L.aqd_hadamard_rotate(x, y, i, o, batch, d_in, b, None)
    assert rot(b=32) == E_BLOCK
    assert rot(b=512) == E_BLOCK
    assert rot(b=128, d_in=192) == E_BLOCK
    assert rot(i=BF16X2) == E_DTYPE
    assert rot(i=7) == E_DTYPE
    assert rot(o=9) == E_DTYPE
    assert rot(batch=-1) == E_SHAPE
    assert rot(x=None) == E_NULL
    assert rot(y=FAKE_ODD) == E_ALIGN
    assert rot(y=FAKE, i=F16, o=F32) == E_DTYPE          # in place with different dtypes
    assert rot(y=FAKE, i=F16, o=BF16X2) == E_DTYPE


def test_signed_hadamard_rejects_bad_arguments(L):
    def rot(x=FAKE, y=FAKE + 4096, i=F16, o=F16, batch=1, d_in=256, b=64, signs=FAKE + 8192):
        return L.aqd_hadamard_rotate_signed(x, y, i, o, batch, d_in, b, signs, None)
    assert rot(signs=None) == E_NULL
    assert rot(signs=FAKE + 8192 + 4) == E_ALIGN          # the mask is read as 64-bit words
    assert rot(b=32) == E_BLOCK
    assert rot(b=128, d_in=192) == E_BLOCK
    assert rot(i=BF16X2) == E_DTYPE
    assert rot(x=None) == E_NULL
    assert rot(y=FAKE_ODD) == E_ALIGN
    assert rot(y=FAKE, i=F16, o=F32) == E_DTYPE
    assert rot(batch=0, signs=None) == OK                 # nothing to rotate


def test_pack_rejects_bad_arguments(L):
    assert L.aqd_pack_codes(FAKE, None, lay(), None) == E_NULL
    assert L.aqd_pack_codes(FAKE, FAKE_ODD, lay(), None) == E_ALIGN
    assert L.aqd_unpack_codes(FAKE_ODD, FAKE, lay(), None) == E_ALIGN
    assert L.aqd_pack_codes(FAKE, FAKE, lay(group=16), None) == E_UNSUP


def test_product_does_not_link_or_load_the_oracle():
    deps = subprocess.run(["readelf", "-d", aqd.LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "oracle" not in deps
    pkg = os.path.join(ROOT, "additive_codebook_gemv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src and "liboracle" not in src, f


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(aqd, "_lib", None)
    monkeypatch.setattr(aqd, "LIB_PATH", str(tmp_path / "libaqd.so"))
    with pytest.raises(RuntimeError, match="missing"):
        aqd.lib()


def test_gemv_workspace_required(L):
    need = L.aqd_gemv_workspace_bytes(lay(4096, 14336, 4), 1)
    assert need >= 4 * 4096
    assert _gemv(L, layer=lay(4096, 14336, 4), ws=None, ws_bytes=0) == E_WS
    assert _gemv(L, layer=lay(4096, 14336, 4), ws=FAKE, ws_bytes=need - 1) == E_WS
    assert _gemv(L, layer=lay(4096, 14336, 4), ws=FAKE_ODD, ws_bytes=need) == E_ALIGN


def test_grouped_gemv_rejects_bad_arguments(L):
    def lins(n, d_out=64, M=2):
        arr = (aqd.aqd_linear * max(n, 1))()
        for i in range(n):
            arr[i] = aqd.aqd_linear(FAKE, FAKE, FAKE, FAKE, d_out, M)
        return arr
    big = lins(3, 4096, 4)
    need = L.aqd_gemv_grouped_workspace_bytes(big, 3, 4096)
    assert need >= 3 * 4096 * 8
    assert L.aqd_gemv_grouped(lins(0), 0, 1, FAKE, 256, FAKE, 1 << 20, None) == E_SHAPE
    assert L.aqd_gemv_grouped(lins(5), 5, 1, FAKE, 256, FAKE, 1 << 20, None) == E_SHAPE
    assert L.aqd_gemv_grouped(None, 2, 1, FAKE, 256, FAKE, 1 << 20, None) == E_NULL
    assert L.aqd_gemv_grouped(lins(2), 2, 3, FAKE, 256, FAKE, 1 << 20, None) == E_K          # M = 2
    assert L.aqd_gemv_grouped(lins(2), 2, 1, FAKE, 100, FAKE, 1 << 20, None) == E_SHAPE      # d_in % 8
    assert L.aqd_gemv_grouped(big, 3, 2, FAKE, 4096, None, 0, None) == E_WS
    assert L.aqd_gemv_grouped(big, 3, 2, FAKE, 4096, FAKE, need - 1, None) == E_WS
    assert L.aqd_gemv_grouped(lins(2), 2, 1, FAKE_ODD, 256, FAKE, 1 << 20, None) == E_ALIGN
    assert L.aqd_gemv_grouped_workspace_bytes(lins(5), 5, 256) == 0
    # the limit of one launch's lookup tables, refused before anything is enqueued: more than 1020
    # slots (k * ceil(d_in / 512))
    assert L.aqd_gemv_grouped(lins(2, 64, 4), 2, 4, FAKE, 131072, FAKE, 1 << 20, None) == E_UNSUP
    # the fused rotation: block must be 64/128/256 and divide d_in
    assert L.aqd_rotate_gemv_grouped(lins(2), 2, 1, FAKE, 256, 32, FAKE, 1 << 20, None) == E_BLOCK
    assert L.aqd_rotate_gemv_grouped(lins(2), 2, 1, FAKE, 192, 128, FAKE, 1 << 20, None) == E_BLOCK
    assert L.aqd_rotate_gemv_grouped(lins(5), 5, 1, FAKE, 256, 64, FAKE, 1 << 20, None) == E_SHAPE
    assert L.aqd_rotate_gemv_grouped(big, 3, 2, FAKE, 4096, 128, None, 0, None) == E_WS
    # the randomized rotation adds a sign mask: required, 8-byte aligned
    sg = FAKE + 8192
    assert L.aqd_rotate_gemv_grouped_signed(lins(2), 2, 1, FAKE, 256, 64, None, FAKE, 1 << 20, None) == E_NULL
    assert L.aqd_rotate_gemv_grouped_signed(lins(2), 2, 1, FAKE, 256, 64, sg + 2, FAKE, 1 << 20, None) == E_ALIGN
    assert L.aqd_rotate_gemv_grouped_signed(lins(2), 2, 1, FAKE, 256, 32, sg, FAKE, 1 << 20, None) == E_BLOCK
    assert L.aqd_rotate_gemv_grouped_signed(lins(5), 5, 1, FAKE, 256, 64, sg, FAKE, 1 << 20, None) == E_SHAPE
    assert L.aqd_rotate_gemv_grouped_signed(big, 3, 2, FAKE, 4096, 128, sg, None, 0, None) == E_WS
    assert L.aqd_rotate_gemv_grouped_signed(lins(2), 2, 3, FAKE, 256, 64, sg, FAKE, 1 << 20, None) == E_K


def test_prefill_workspace_follows_the_plan(L):
    """The prefill workspace is the staged fp16 weight (2 bytes per weight, tile padding included) plus,
    when the inputs are split, one float4 per (split, column, row quad); the plan charges the reduce
    of the partials, so tall layers split at most in two.  Host logic only: nothing is launched."""
    def pf(d_out, d_in, batch):
        return L.aqd_gemm_prefill_workspace_bytes(lay(d_out=d_out, d_in=d_in, M=4), batch)

    def partials(d_out, batch, splits):
        return splits * batch * ((d_out + 3) // 4) * 16
    w = 4096 * 14336 * 2                        # the staged weight of either 8B MLP shape
    # 4096x14336: 16 row blocks x 8 column blocks fill half the chip; two splits, staged at k = 3, 4
    assert pf(4096, 14336, 2048) == partials(4096, 2048, 2) + w
    # 14336x4096 at 512 columns, rebuilt per workgroup in 256-column tiles: 112 tiles, two splits
    # (sixteen would read 470 MB of partials back)
    assert pf(14336, 4096, 512) == partials(14336, 512, 2)
    # 14336x4096 at 1024 and 2048 columns: staged at k = 3, 4; the tiles cover the chip, no split
    assert pf(14336, 4096, 1024) == w
    assert pf(14336, 4096, 2048) == w
    # below 1024 columns nothing is staged at k <= 4; 511 columns of 14336x4096 take 256-column tiles
    # (short inputs), 112 of them, split in two
    assert pf(14336, 4096, 511) == partials(14336, 511, 2)
    # 255 columns: 128-column tiles, 112 of them, split in two
    assert pf(14336, 4096, 255) == partials(14336, 255, 2)
    # a layer of more than 2 GiB of fp16 weight is never staged: partials only, or nothing
    big = pf(65536, 32768, 4096)
    assert big < 65536 * 32768 * 2 and big % 16 == 0


def test_prefill_rejects_bad_arguments(L):
    def pf(packed=FAKE, cb=FAKE, s=FAKE, k=1, x=FAKE, y=FAKE, batch=256, layer=None, ws=FAKE, nws=1 << 30):
        return L.aqd_gemm_prefill(packed, cb, s, k, x, y, batch, layer if layer is not None else lay(), ws, nws,
                                  None)
    assert pf(batch=0) == E_SHAPE
    assert pf(batch=aqd.AQD_PREFILL_MAX_BATCH + 1) == E_SHAPE
    assert pf(k=3) == E_K                         # M = 2
    assert pf(k=0) == E_K
    assert pf(x=None) == E_NULL
    assert pf(y=FAKE + 2) == E_ALIGN               # fp32 output
    assert pf(x=FAKE_ODD) == E_ALIGN
    assert pf(layer=lay(d_in=100)) == E_SHAPE
    assert pf(layer=lay(d_out=0), y=None) == OK   # nothing to compute
    big = lay(d_out=4096, d_in=14336, M=4)
    need = L.aqd_gemm_prefill_workspace_bytes(big, 512)
    assert need > 0                                # 16 row blocks x 4 column blocks: the inputs are split
    assert L.aqd_gemm_prefill(FAKE, FAKE, FAKE, 2, FAKE, FAKE, 512, big, None, 0, None) == E_WS
    assert L.aqd_gemm_prefill(FAKE, FAKE, FAKE, 2, FAKE, FAKE, 512, big, FAKE, need - 1, None) == E_WS
    tall = lay(d_out=14336, d_in=4096, M=4)
    assert L.aqd_gemm_prefill_workspace_bytes(lay(d_out=14336, d_in=4096, M=2), 1024) == 0   # fused, no split
    assert L.aqd_gemm_prefill_workspace_bytes(tall, 4096) == 14336 * 4096 * 2   # staged fp16 weights, no split
    assert L.aqd_gemm_prefill_workspace_bytes(big, 0) == 0


def test_encode_rejects_bad_arguments(L):
    def enc(t=FAKE, cb=FAKE, M=2, d_out=64, d_in=256, codes=FAKE):
        return L.aqd_encode_greedy(t, cb, M, d_out, d_in, codes, None)
    assert enc(M=0) == E_SHAPE
    assert enc(M=9) == E_SHAPE
    assert enc(d_in=100) == E_SHAPE
    assert enc(d_out=-1) == E_SHAPE
    assert enc(t=None) == E_NULL
    assert enc(codes=None) == E_NULL
    assert enc(t=FAKE_ODD) == E_ALIGN              # float4 loads
    assert enc(cb=FAKE + 1) == E_ALIGN
    assert enc(d_out=0, t=None) == OK              # nothing to encode


def test_read_probe_rejects_bad_arguments(L):
    probe = L.aqd_read_probe
    assert probe(FAKE, 0, FAKE, 256, 8, 4, 0, None) == OK                   # nothing to read
    assert probe(None, 1024, FAKE, 256, 8, 4, 0, None) == E_NULL
    assert probe(FAKE, 1024, None, 256, 8, 4, 0, None) == E_NULL
    assert probe(FAKE_ODD, 1024, FAKE, 256, 8, 4, 0, None) == E_ALIGN
    assert probe(FAKE, 1000, FAKE, 256, 8, 4, 0, None) == E_SHAPE           # not a multiple of 16
    assert probe(FAKE, 1024, FAKE, 0, 8, 4, 0, None) == E_SHAPE
    assert probe(FAKE, 1024, FAKE, 65537, 8, 4, 0, None) == E_SHAPE
    assert probe(FAKE, 1024, FAKE, 256, 17, 4, 0, None) == E_SHAPE
    assert probe(FAKE, 1024, FAKE, 256, 8, 3, 0, None) == E_SHAPE
    assert probe(FAKE, 1024, FAKE, 256, 8, 4, 2, None) == E_SHAPE


def test_gemv_noalloc_rejects_before_touching_the_device(L):
    """Every check of aqd_gemv_noalloc runs before the scratch array is looked up or anything is enqueued,
    so on a machine without a GPU each of these returns its status."""
    def call(k=1, batch=1, layer=None, y=FAKE, x=FAKE):
        return L.aqd_gemv_noalloc(FAKE, FAKE, FAKE, k, x, y, batch, layer or lay(64, 256, 2), None)
    assert call(batch=0) == E_SHAPE
    assert call(batch=9) == E_SHAPE
    assert call(k=3) == E_K
    assert call(y=None) == E_NULL
    assert call(x=FAKE_ODD) == E_ALIGN
    assert call(layer=lay(64, 256, 2, group=16)) == E_UNSUP
    big = lay(1 << 22, 4096, 4)          # workspace above AQD_NOALLOC_SCRATCH_BYTES at batch 8
    assert L.aqd_gemv_workspace_bytes(big, 8) > aqd.AQD_NOALLOC_SCRATCH_BYTES
    assert call(batch=8, layer=big) == E_WS
