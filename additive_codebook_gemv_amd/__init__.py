"""Python binding of libaqd, the MI355X additive-codebook decode kernels.

Argument marshalling only: every computation runs in the HIP kernels behind
the C ABI declared in ``include/aqd.h``.  PyTorch provides device memory and
the current stream.  The functions keep the C names; each takes torch CUDA
tensors and returns the output tensor (allocated here unless ``out=`` is
given).  If the library is not built, or a call fails, an exception is raised:
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libaqd.so")

AQD_F16, AQD_BF16, AQD_F32, AQD_BF16X2 = 0, 1, 2, 3
_TORCH_DT = {torch.float16: AQD_F16, torch.bfloat16: AQD_BF16, torch.float32: AQD_F32}


class AqdError(RuntimeError):
    """A libaqd call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class aqd_layer(ctypes.Structure):
    _fields_ = [("d_out", ctypes.c_int64), ("d_in", ctypes.c_int64), ("M", ctypes.c_int32),
                ("group", ctypes.c_int32), ("code_bits", ctypes.c_int32)]


class aqd_linear(ctypes.Structure):
    _fields_ = [("packed_codes", ctypes.c_void_p), ("codebooks", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("d_out", ctypes.c_int64), ("M", ctypes.c_int32)]


AQD_MAX_GROUP = 4

_lib: Optional[ctypes.CDLL] = None

_VP, _SZ, _I32, _I64, _INT = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_int
_LP = ctypes.POINTER(aqd_layer)
_SIGNATURES = {
    "aqd_abi_version": (_INT, []),
    "aqd_status_string": (ctypes.c_char_p, [_INT]),
    "aqd_last_error": (ctypes.c_char_p, []),
    "aqd_packed_codes_bytes": (_SZ, [_LP]),
    "aqd_pack_codes": (_INT, [_VP, _VP, _LP, _VP]),
    "aqd_unpack_codes": (_INT, [_VP, _VP, _LP, _VP]),
    "aqd_hadamard_rotate": (_INT, [_VP, _VP, _INT, _INT, _I64, _I64, _I32, _VP]),
    "aqd_hadamard_rotate_signed": (_INT, [_VP, _VP, _INT, _INT, _I64, _I64, _I32, _VP, _VP]),
    "aqd_gemv_workspace_bytes": (_SZ, [_LP, _I32]),
    "aqd_gemv": (_INT, [_VP, _VP, _VP, _I32, _VP, _VP, _I32, _LP, _VP, _SZ, _VP]),
    "aqd_gemv_grouped_workspace_bytes": (_SZ, [ctypes.POINTER(aqd_linear), _I32, _I64]),
    "aqd_gemv_grouped": (_INT, [ctypes.POINTER(aqd_linear), _I32, _I32, _VP, _I64, _VP, _SZ, _VP]),
    "aqd_rotate_gemv_grouped": (_INT, [ctypes.POINTER(aqd_linear), _I32, _I32, _VP, _I64, _I32, _VP, _SZ, _VP]),
    "aqd_gemm_prefill_workspace_bytes": (_SZ, [ctypes.POINTER(aqd_layer), _I32]),
    "aqd_gemm_prefill": (_INT, [_VP, _VP, _VP, _I32, _VP, _VP, _I32, ctypes.POINTER(aqd_layer), _VP, _SZ, _VP]),
    "aqd_encode_greedy": (_INT, [_VP, _VP, _I32, _I64, _I64, _VP, _VP]),
    "aqd_rotate_gemv_grouped_signed": (_INT, [ctypes.POINTER(aqd_linear), _I32, _I32, _VP, _I64, _I32, _VP, _VP,
                                              _SZ, _VP]),
    "aqd_gemm_small_batch_workspace_bytes": (_SZ, [_LP, _I32]),
    "aqd_gemm_small_batch": (_INT, [_VP, _VP, _VP, _I32, _VP, _INT, _VP, _I32, _LP, _VP, _SZ, _VP]),
    "aqd_gemm_small_batch_tiered": (_INT, [_VP, _VP, _VP, ctypes.POINTER(_I32), _VP, _VP, _I32, _LP, _VP, _SZ, _VP]),
    "aqd_read_probe": (_INT, [_VP, _SZ, _VP, _I32, _I32, _I32, _I32, _VP]),
    "aqd_gemv_noalloc": (_INT, [_VP, _VP, _VP, _I32, _VP, _VP, _I32, _LP, _VP]),
}


def lib() -> ctypes.CDLL:
    """The loaded libaqd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m additive_codebook_gemv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def layer(d_out: int, d_in: int, M: int) -> aqd_layer:
    return aqd_layer(d_out, d_in, M, 8, 8)


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise AqdError(status, f"{L.aqd_status_string(status).decode()}: {L.aqd_last_error().decode()}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libaqd must be contiguous")
    return t.data_ptr() or None


def aqd_packed_codes_bytes(d_out: int, d_in: int, M: int) -> int:
    return int(lib().aqd_packed_codes_bytes(ctypes.byref(layer(d_out, d_in, M))))


def aqd_pack_codes(codes: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """codes: uint8 [d_out][d_in/8][M] on the GPU -> packed uint8 tiles."""
    d_out, G, M = codes.shape
    L = layer(d_out, G * 8, M)
    n = int(lib().aqd_packed_codes_bytes(ctypes.byref(L)))
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=codes.device)
    _check(lib().aqd_pack_codes(_ptr(codes), _ptr(out), ctypes.byref(L), _stream()))
    return out


def aqd_unpack_codes(packed: torch.Tensor, d_out: int, d_in: int, M: int,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty((d_out, d_in // 8, M), dtype=torch.uint8, device=packed.device)
    L = layer(d_out, d_in, M)
    _check(lib().aqd_unpack_codes(_ptr(packed), _ptr(out), ctypes.byref(L), _stream()))
    return out


def _rotation_out(x2: torch.Tensor, out_dtype: int) -> torch.Tensor:
    batch, d_in = x2.shape
    if out_dtype == AQD_BF16X2:
        return torch.empty((2, batch, d_in), dtype=torch.bfloat16, device=x2.device)
    tdt = {AQD_F16: torch.float16, AQD_BF16: torch.bfloat16, AQD_F32: torch.float32}[out_dtype]
    return torch.empty((batch, d_in), dtype=tdt, device=x2.device)


def aqd_hadamard_rotate(x: torch.Tensor, block: int, out_dtype: int = AQD_F16,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """x: [batch][d_in] fp16/bf16/fp32 -> rotated [batch][d_in] (or [2][batch][d_in] for AQD_BF16X2)."""
    x2 = x.reshape(-1, x.shape[-1])
    batch, d_in = x2.shape
    if out is None:
        out = _rotation_out(x2, out_dtype)
    _check(lib().aqd_hadamard_rotate(_ptr(x2), _ptr(out), _TORCH_DT[x.dtype], out_dtype, batch, d_in, block,
                                     _stream()))
    return out


def aqd_hadamard_rotate_signed(x: torch.Tensor, block: int, signs: torch.Tensor, out_dtype: int = AQD_F16,
                               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Randomized rotation H diag(eps) / sqrt(b) per block; signs: uint8 [d_in / 8] device bit mask
    (bit c % 8 of byte c // 8 set -> input c negated)."""
    x2 = x.reshape(-1, x.shape[-1])
    batch, d_in = x2.shape
    if out is None:
        out = _rotation_out(x2, out_dtype)
    _check(lib().aqd_hadamard_rotate_signed(_ptr(x2), _ptr(out), _TORCH_DT[x.dtype], out_dtype, batch, d_in,
                                            block, _ptr(signs), _stream()))
    return out


def aqd_gemv_workspace_bytes(d_out: int, d_in: int, M: int, batch: int) -> int:
    return int(lib().aqd_gemv_workspace_bytes(ctypes.byref(layer(d_out, d_in, M)), batch))


def aqd_gemv(packed: torch.Tensor, codebooks: torch.Tensor, scales: torch.Tensor, k: int, x_rot: torch.Tensor,
             d_out: int, d_in: int, M: int, out: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[batch][d_out] fp16 = s * (W_k @ x_rot) for fp16 x_rot [batch][d_in], batch 1..8."""
    x2 = x_rot if x_rot.dim() == 2 else x_rot.reshape(1, -1)
    batch = x2.shape[0]
    L = layer(d_out, d_in, M)
    if out is None:
        out = torch.empty((batch, d_out), dtype=torch.float16, device=x_rot.device)
    # only a missing workspace is sized here; the library checks the size of a given one
    need = int(lib().aqd_gemv_workspace_bytes(ctypes.byref(L), batch)) if workspace is None else 0
    if need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=x_rot.device)
    _check(lib().aqd_gemv(_ptr(packed), _ptr(codebooks), _ptr(scales), k, _ptr(x2), _ptr(out), batch,
                          ctypes.byref(L), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                          _stream()))
    return out


AQD_NOALLOC_SCRATCH_BYTES = 16 << 20


def aqd_gemv_noalloc(packed: torch.Tensor, codebooks: torch.Tensor, scales: torch.Tensor, k: int,
                     x_rot: torch.Tensor, d_out: int, d_in: int, M: int,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """aqd_gemv with the library's fixed scratch array as workspace (the call itself allocates no device
    memory; give `out` to allocate nothing here either)."""
    x2 = x_rot if x_rot.dim() == 2 else x_rot.reshape(1, -1)
    batch = x2.shape[0]
    if out is None:
        out = torch.empty((batch, d_out), dtype=torch.float16, device=x_rot.device)
    _check(lib().aqd_gemv_noalloc(_ptr(packed), _ptr(codebooks), _ptr(scales), k, _ptr(x2), _ptr(out), batch,
                                  ctypes.byref(layer(d_out, d_in, M)), _stream()))
    return out


def _linears(parts):
    arr = (aqd_linear * len(parts))()
    for i, (packed, codebooks, scales, y, d_out, M) in enumerate(parts):
        arr[i] = aqd_linear(_ptr(packed), _ptr(codebooks), _ptr(scales), _ptr(y), d_out, M)
    return arr


def aqd_gemv_grouped_workspace_bytes(d_outs, d_in: int, Ms) -> int:
    arr = (aqd_linear * len(d_outs))()
    for i, (d_out, M) in enumerate(zip(d_outs, Ms)):
        arr[i] = aqd_linear(None, None, None, None, d_out, M)
    return int(lib().aqd_gemv_grouped_workspace_bytes(arr, len(d_outs), d_in))


def aqd_gemv_grouped(linears, k: int, x_rot: torch.Tensor, d_in: int,
                     workspace: Optional[torch.Tensor] = None, block: int = 0,
                     signs: Optional[torch.Tensor] = None):
    """Batch-1 GEMV of several linears sharing x_rot (fp16 [d_in] or [1][d_in]) in one launch (one per
    table-slot choice when the linears' sizes call for different ones; each output has its own call's bits).

    linears: sequence of (packed, codebooks, scales, d_out, M) or (packed, codebooks, scales, d_out, M, out);
    returns the fp16 outputs [1][d_out], one per linear.  With block (64/128/256) the input is the raw
    activation and the launch applies the block rotation itself (aqd_rotate_gemv_grouped), with the sign
    mask of the randomized rotation when signs is given (aqd_rotate_gemv_grouped_signed).
    """
    outs, parts = [], []
    for lin in linears:
        packed, codebooks, scales, d_out, M = lin[:5]
        y = lin[5] if len(lin) > 5 else torch.empty((1, d_out), dtype=torch.float16, device=x_rot.device)
        outs.append(y)
        parts.append((packed, codebooks, scales, y, d_out, M))
    arr = _linears(parts)
    # only a missing workspace is sized here; the library checks the size of a given one
    need = int(lib().aqd_gemv_grouped_workspace_bytes(arr, len(parts), d_in)) if workspace is None else 0
    if need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=x_rot.device)
    nws = workspace.numel() if workspace is not None else 0
    if signs is not None:
        if not block:
            raise ValueError("signs apply to the rotating launch only (give block)")
        _check(lib().aqd_rotate_gemv_grouped_signed(arr, len(parts), k, _ptr(x_rot.reshape(-1)), d_in, block,
                                                    _ptr(signs), _ptr(workspace), nws, _stream()))
    elif block:
        _check(lib().aqd_rotate_gemv_grouped(arr, len(parts), k, _ptr(x_rot.reshape(-1)), d_in, block,
                                             _ptr(workspace), nws, _stream()))
    else:
        _check(lib().aqd_gemv_grouped(arr, len(parts), k, _ptr(x_rot.reshape(-1)), d_in, _ptr(workspace), nws,
                                      _stream()))
    return outs


def aqd_rotate_gemv_grouped(linears, k: int, x: torch.Tensor, d_in: int, block: int,
                            workspace: Optional[torch.Tensor] = None):
    """Rotation (block 64/128/256) of the raw fp16 activation x and the grouped batch-1 GEMV, one launch."""
    return aqd_gemv_grouped(linears, k, x, d_in, workspace=workspace, block=block)


def aqd_rotate_gemv_grouped_signed(linears, k: int, x: torch.Tensor, d_in: int, block: int, signs: torch.Tensor,
                                   workspace: Optional[torch.Tensor] = None):
    """As aqd_rotate_gemv_grouped with the randomized rotation H diag(eps) / sqrt(b) (uint8 sign mask)."""
    return aqd_gemv_grouped(linears, k, x, d_in, workspace=workspace, block=block, signs=signs)


def aqd_gemm_small_batch_workspace_bytes(d_out: int, d_in: int, M: int, batch: int) -> int:
    return int(lib().aqd_gemm_small_batch_workspace_bytes(ctypes.byref(layer(d_out, d_in, M)), batch))


def aqd_gemm_small_batch(packed: torch.Tensor, codebooks: torch.Tensor, scales: torch.Tensor, k: int,
                         x_rot: torch.Tensor, d_out: int, d_in: int, M: int, x_dtype: int = AQD_BF16X2,
                         out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[batch][d_out] fp32 for x_rot bf16 [batch][d_in] (AQD_BF16), [2][batch][d_in] (AQD_BF16X2) or
    fp16 [batch][d_in] (AQD_F16)."""
    batch = x_rot.shape[-2]
    L = layer(d_out, d_in, M)
    if out is None:
        out = torch.empty((batch, d_out), dtype=torch.float32, device=x_rot.device)
    # only a missing workspace is sized here; the library checks the size of a given one
    need = int(lib().aqd_gemm_small_batch_workspace_bytes(ctypes.byref(L), batch)) if workspace is None else 0
    if need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=x_rot.device)
    _check(lib().aqd_gemm_small_batch(_ptr(packed), _ptr(codebooks), _ptr(scales), k, _ptr(x_rot), x_dtype,
                                      _ptr(out), batch, ctypes.byref(L), _ptr(workspace),
                                      workspace.numel() if workspace is not None else 0, _stream()))
    return out


def aqd_encode_greedy(target: torch.Tensor, codebooks: torch.Tensor, M: Optional[int] = None,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Greedy residual codes uint8 [d_out][d_in/8][M] for float32 targets [d_out][d_in] (rotated weights
    divided by their row scale) and fp16 codebooks [M][256][8]."""
    d_out, d_in = target.shape
    M = codebooks.shape[0] if M is None else M
    if out is None:
        out = torch.empty((d_out, d_in // 8, M), dtype=torch.uint8, device=target.device)
    _check(lib().aqd_encode_greedy(_ptr(target), _ptr(codebooks), M, d_out, d_in, _ptr(out), _stream()))
    return out


AQD_PREFILL_MAX_BATCH = 32768


def aqd_gemm_prefill_workspace_bytes(d_out: int, d_in: int, M: int, batch: int) -> int:
    return int(lib().aqd_gemm_prefill_workspace_bytes(ctypes.byref(layer(d_out, d_in, M)), batch))


def aqd_gemm_prefill(packed: torch.Tensor, codebooks: torch.Tensor, scales: torch.Tensor, k: int,
                     x_rot: torch.Tensor, d_out: int, d_in: int, M: int, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[batch][d_out] fp32 = s * (W_k @ x_rot) for fp16 x_rot [batch][d_in], batch 1..32768 (meant for >= 128)."""
    batch = x_rot.shape[0]
    L = layer(d_out, d_in, M)
    if out is None:
        out = torch.empty((batch, d_out), dtype=torch.float32, device=x_rot.device)
    need = int(lib().aqd_gemm_prefill_workspace_bytes(ctypes.byref(L), batch))
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=x_rot.device)
    _check(lib().aqd_gemm_prefill(_ptr(packed), _ptr(codebooks), _ptr(scales), k, _ptr(x_rot), _ptr(out), batch,
                                  ctypes.byref(L), _ptr(workspace), workspace.numel() if workspace is not None else 0,
                                  _stream()))
    return out


def aqd_gemm_small_batch_tiered(packed: torch.Tensor, codebooks: torch.Tensor, scales: torch.Tensor, ks,
                                x_rot: torch.Tensor, d_out: int, d_in: int, M: int,
                                out: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[batch][d_out] fp32 where column n uses the first ks[n] codebooks; x_rot fp16 [batch][d_in]."""
    batch = x_rot.shape[0]
    if len(ks) != batch:
        raise ValueError("one k per column")
    L = layer(d_out, d_in, M)
    if out is None:
        out = torch.empty((batch, d_out), dtype=torch.float32, device=x_rot.device)
    # only a missing workspace is sized here; the library checks the size of a given one
    need = int(lib().aqd_gemm_small_batch_workspace_bytes(ctypes.byref(L), batch)) if workspace is None else 0
    if need:
        workspace = torch.zeros(need, dtype=torch.uint8, device=x_rot.device)
    karr = (ctypes.c_int32 * batch)(*[int(k) for k in ks])
    _check(lib().aqd_gemm_small_batch_tiered(_ptr(packed), _ptr(codebooks), _ptr(scales), karr, _ptr(x_rot),
                                             _ptr(out), batch, ctypes.byref(L), _ptr(workspace),
                                             workspace.numel() if workspace is not None else 0, _stream()))
    return out


class QuantizedLinear:
    """One additive-codebook linear resident on the GPU: packed codes, codebooks, scales.

    ``forward(x, k)`` rotates the activation online and applies the k-codebook
    product: batch 1 (fp16) in one launch that rotates its own input, batch
    1..8 through the rotation and the GEMV (fp16 output), batch 9..64 through
    the fp16 matrix-core path (fp32 output), larger batches (prefill) through
    the fused dequantize + matrix-core GEMM (fp32 output).  With ``signs`` the rotation is
    the randomized H diag(eps) / sqrt(b), and the codes must be those of W R^T.
    """

    def __init__(self, codes: torch.Tensor, codebooks: torch.Tensor, scales: torch.Tensor, block: int,
                 signs: Optional[torch.Tensor] = None):
        d_out, G, M = codes.shape
        self.d_out, self.d_in, self.M, self.block = d_out, G * 8, M, block
        # randomized rotation H diag(eps) when a sign mask (uint8 [d_in / 8]) is given
        self.signs = None if signs is None else signs.contiguous()
        if self.signs is not None and (self.signs.dtype != torch.uint8 or self.signs.numel() * 8 != self.d_in):
            raise ValueError("signs must be uint8 [d_in / 8]")
        self.packed = aqd_pack_codes(codes)
        self.codebooks = codebooks.contiguous()
        self.scales = scales.contiguous()
        # Two buffers, never shared: the GEMV workspace (batch 1..8 and the launch that rotates its own
        # input) holds counted row sums that must be zero when a call starts and that every call leaves
        # zero; the small-batch workspace holds split partial sums that every call overwrites.  Handing
        # the second to a GEMV would leave partial sums where the counters must be zero.
        n = max([aqd_gemv_workspace_bytes(d_out, self.d_in, M, b) for b in range(1, 9)] +
                [aqd_gemv_grouped_workspace_bytes([d_out], self.d_in, [M])])
        self.workspace = torch.zeros(n, dtype=torch.uint8, device=codes.device) if n else None
        n = max(aqd_gemm_small_batch_workspace_bytes(d_out, self.d_in, M, b) for b in range(9, 65))
        self.sb_workspace = torch.empty(n, dtype=torch.uint8, device=codes.device) if n else None

    def rotate(self, x2: torch.Tensor) -> torch.Tensor:
        """fp16 rotated activation (with the sign mask when the layer has one)."""
        if self.signs is not None:
            return aqd_hadamard_rotate_signed(x2, self.block, self.signs, AQD_F16)
        return aqd_hadamard_rotate(x2, self.block, AQD_F16)

    def forward(self, x: torch.Tensor, k: int) -> torch.Tensor:
        x2 = x.reshape(-1, self.d_in)
        if x2.shape[0] == 1 and x2.dtype == torch.float16 and self.d_in > 0:
            # one launch: the GEMV rotates its own input
            return aqd_gemv_grouped([(self.packed, self.codebooks, self.scales, self.d_out, self.M)], k,
                                    x2.contiguous(), self.d_in, workspace=self.workspace, block=self.block,
                                    signs=self.signs)[0]
        xr = self.rotate(x2)
        if x2.shape[0] <= 8:
            return aqd_gemv(self.packed, self.codebooks, self.scales, k, xr, self.d_out, self.d_in, self.M,
                            workspace=self.workspace)
        if x2.shape[0] <= 64:
            return aqd_gemm_small_batch(self.packed, self.codebooks, self.scales, k, xr, self.d_out, self.d_in,
                                        self.M, AQD_F16, workspace=self.sb_workspace)
        return aqd_gemm_prefill(self.packed, self.codebooks, self.scales, k, xr, self.d_out, self.d_in, self.M)


def aqd_read_probe(buf: torch.Tensor, nbytes: int, sink: torch.Tensor, workgroups: int, waves: int, unroll: int,
                   contiguous: bool) -> None:
    """Measurement reference (include/aqd_probe.h): read the first nbytes of buf once with 16-byte loads in
    one launch of the given shape; sink is int32/uint32 [>= workgroups] and is in practice not written."""
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    if sink.numel() < workgroups:
        raise ValueError("sink needs one word per workgroup")
    _check(lib().aqd_read_probe(_ptr(buf), nbytes, _ptr(sink), workgroups, waves, unroll, int(contiguous),
                                _stream()))
