"""ctypes front end of the CPU oracle (test infrastructure).

Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg import this package.  The product library never loads
it, and it never loads the product library.

The arithmetic is in ``aqd_oracle.c`` (plain C, double precision); this file
only builds it with gcc, marshals numpy arrays and decodes fp16/bf16 inputs
through the oracle's own decoder.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "aqd_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F16, BF16, F32 = 0, 1, 2
_DT = {"f16": F16, "bf16": BF16, "f32": F32}

_c_dp = ctypes.POINTER(ctypes.c_double)
_c_u8p = ctypes.POINTER(ctypes.c_uint8)
_c_u16p = ctypes.POINTER(ctypes.c_uint16)
_c_i32p = ctypes.POINTER(ctypes.c_int32)
_i64, _i32 = ctypes.c_int64, ctypes.c_int32


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", *extra_flags, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctype)


class Oracle:
    """The oracle library loaded from `path`."""

    def __init__(self, path: str = LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        self.lib = lib
        lib.oracle_f16_to_f64.restype = ctypes.c_double
        lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_f64.restype = ctypes.c_double
        lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.oracle_f64_to_f16.restype = ctypes.c_uint16
        lib.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
        lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_decode.argtypes = [ctypes.c_void_p, ctypes.c_int, _i64, _c_dp]
        lib.oracle_encode.argtypes = [_c_dp, ctypes.c_int, _i64, _c_u16p]
        lib.oracle_hadamard.argtypes = [_i32, _c_i32p]
        lib.oracle_rotate.argtypes = [_c_dp, _i64, _i64, _i32, _c_dp]
        lib.oracle_sign_vector.argtypes = [_c_u8p, _i64, _c_dp]
        lib.oracle_rotate_signed.argtypes = [_c_dp, _c_u8p, _i64, _i64, _i32, _c_dp]
        lib.oracle_reconstruct.argtypes = [_c_u8p, _c_dp, _c_dp, _i64, _i64, _i32, _i32, _c_dp]
        lib.oracle_linear.argtypes = [_c_u8p, _c_dp, _c_dp, _i64, _i64, _i32, _i32, _c_dp, _i64, _c_dp]
        lib.oracle_forward.argtypes = [_c_u8p, _c_dp, _c_dp, _i64, _i64, _i32, _i32, _c_dp, _i64, _i32, _c_dp]
        lib.oracle_packed_bytes.restype = _i64
        lib.oracle_packed_bytes.argtypes = [_i64, _i64, _i32]
        lib.oracle_pack_codes.argtypes = [_c_u8p, _i64, _i64, _i32, _c_u8p]
        lib.oracle_unpack_codes.argtypes = [_c_u8p, _i64, _i64, _i32, _c_u8p]
        lib.oracle_storage_bits.restype = ctypes.c_double
        lib.oracle_storage_bits.argtypes = [_i64, _i64, _i32, _i32, _i32]
        lib.oracle_bits_per_param.restype = ctypes.c_double
        lib.oracle_bits_per_param.argtypes = [_i64, _i64, _i32, _i32, _i32]
        lib.oracle_set_threads.argtypes = [ctypes.c_int]
        lib.oracle_encode_greedy.argtypes = [ctypes.POINTER(ctypes.c_float), _c_u16p, _i64, _i64, _i32, _c_u8p]

    # -- number formats --------------------------------------------------
    def decode(self, a: np.ndarray, dtype: str = "f16") -> np.ndarray:
        """fp16 array / uint16 bit patterns (f16, bf16) or float32 array -> float64."""
        if dtype == "f32":
            src = np.ascontiguousarray(a, dtype=np.float32)
        else:
            src = np.ascontiguousarray(a).view(np.uint16)
        out = np.empty(src.shape, dtype=np.float64)
        rc = self.lib.oracle_decode(src.ctypes.data_as(ctypes.c_void_p), _DT[dtype], src.size, _ptr(out, _c_dp))
        assert rc == 0
        return out

    def encode(self, v: np.ndarray, dtype: str = "f16") -> np.ndarray:
        """float64 -> uint16 bit patterns, round to nearest even."""
        v = np.ascontiguousarray(v, dtype=np.float64)
        out = np.empty(v.shape, dtype=np.uint16)
        rc = self.lib.oracle_encode(_ptr(v, _c_dp), _DT[dtype], v.size, _ptr(out, _c_u16p))
        assert rc == 0
        return out

    def _f64(self, a: Optional[np.ndarray], dtype: str = "f16") -> Optional[np.ndarray]:
        if a is None:
            return None
        if a.dtype == np.float64:
            return np.ascontiguousarray(a)
        if a.dtype == np.float16 or a.dtype == np.uint16:
            return self.decode(a, dtype)
        if a.dtype == np.float32:
            return self.decode(a, "f32")
        raise TypeError(a.dtype)

    # -- method ----------------------------------------------------------
    def hadamard(self, b: int) -> np.ndarray:
        H = np.empty((b, b), dtype=np.int32)
        assert self.lib.oracle_hadamard(b, _ptr(H, _c_i32p)) == 0
        return H

    def rotate(self, x: np.ndarray, b: int, dtype: str = "f16") -> np.ndarray:
        """Rotated activation (float64) from x [B][d_in] (float64, fp16 or bf16 bits)."""
        xd = self._f64(x, dtype)
        xd = np.ascontiguousarray(np.atleast_2d(xd))
        out = np.empty_like(xd)
        rc = self.lib.oracle_rotate(_ptr(xd, _c_dp), xd.shape[0], xd.shape[1], b, _ptr(out, _c_dp))
        if rc != 0:
            raise ValueError(f"oracle_rotate rc={rc}")
        return out

    def sign_vector(self, signs: np.ndarray, d_in: int) -> np.ndarray:
        """+-1.0 per input from the sign bit mask (bit c % 8 of byte c // 8 set -> -1)."""
        signs = np.ascontiguousarray(signs, dtype=np.uint8)
        assert signs.size * 8 >= d_in
        eps = np.empty(d_in, dtype=np.float64)
        assert self.lib.oracle_sign_vector(_ptr(signs, _c_u8p), d_in, _ptr(eps, _c_dp)) == 0
        return eps

    def rotate_signed(self, x: np.ndarray, signs: np.ndarray, b: int, dtype: str = "f16") -> np.ndarray:
        """Randomized rotation H_b diag(eps) / sqrt(b) per block of x [B][d_in] (float64 result)."""
        xd = np.ascontiguousarray(np.atleast_2d(self._f64(x, dtype)))
        signs = np.ascontiguousarray(signs, dtype=np.uint8)
        assert signs.size * 8 >= xd.shape[1]
        out = np.empty_like(xd)
        rc = self.lib.oracle_rotate_signed(_ptr(xd, _c_dp), _ptr(signs, _c_u8p), xd.shape[0], xd.shape[1], b,
                                           _ptr(out, _c_dp))
        if rc != 0:
            raise ValueError(f"oracle_rotate_signed rc={rc}")
        return out

    def reconstruct(self, codes: np.ndarray, codebooks: np.ndarray, scales: Optional[np.ndarray], k: int) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        d_out, G, M = codes.shape
        cb = self._f64(codebooks)
        s = self._f64(scales)
        W = np.empty((d_out, G * 8), dtype=np.float64)
        rc = self.lib.oracle_reconstruct(_ptr(codes, _c_u8p), _ptr(cb, _c_dp),
                                         _ptr(s, _c_dp) if s is not None else None,
                                         d_out, G * 8, M, k, _ptr(W, _c_dp))
        if rc != 0:
            raise ValueError(f"oracle_reconstruct rc={rc}")
        return W

    def linear(self, codes: np.ndarray, codebooks: np.ndarray, scales: Optional[np.ndarray], k: int,
               xrot: np.ndarray, x_dtype: str = "f16") -> np.ndarray:
        """y [B][d_out] (float64) from an already rotated activation."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        d_out, G, M = codes.shape
        cb = self._f64(codebooks)
        s = self._f64(scales)
        xr = np.ascontiguousarray(np.atleast_2d(self._f64(xrot, x_dtype)))
        assert xr.shape[1] == G * 8
        y = np.empty((xr.shape[0], d_out), dtype=np.float64)
        rc = self.lib.oracle_linear(_ptr(codes, _c_u8p), _ptr(cb, _c_dp),
                                    _ptr(s, _c_dp) if s is not None else None,
                                    d_out, G * 8, M, k, _ptr(xr, _c_dp), xr.shape[0], _ptr(y, _c_dp))
        if rc != 0:
            raise ValueError(f"oracle_linear rc={rc}")
        return y

    def forward(self, codes: np.ndarray, codebooks: np.ndarray, scales: Optional[np.ndarray], k: int,
                x: np.ndarray, b: int, x_dtype: str = "f16") -> np.ndarray:
        """y [B][d_out] (float64) from the raw activation: rotate, then multiply."""
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        d_out, G, M = codes.shape
        cb = self._f64(codebooks)
        s = self._f64(scales)
        xd = np.ascontiguousarray(np.atleast_2d(self._f64(x, x_dtype)))
        y = np.empty((xd.shape[0], d_out), dtype=np.float64)
        rc = self.lib.oracle_forward(_ptr(codes, _c_u8p), _ptr(cb, _c_dp),
                                     _ptr(s, _c_dp) if s is not None else None,
                                     d_out, G * 8, M, k, _ptr(xd, _c_dp), xd.shape[0], b, _ptr(y, _c_dp))
        if rc != 0:
            raise ValueError(f"oracle_forward rc={rc}")
        return y

    # -- layout ----------------------------------------------------------
    def packed_bytes(self, d_out: int, G: int, M: int) -> int:
        return int(self.lib.oracle_packed_bytes(d_out, G, M))

    def pack(self, codes: np.ndarray) -> np.ndarray:
        codes = np.ascontiguousarray(codes, dtype=np.uint8)
        d_out, G, M = codes.shape
        out = np.empty(self.packed_bytes(d_out, G, M), dtype=np.uint8)
        assert self.lib.oracle_pack_codes(_ptr(codes, _c_u8p), d_out, G, M, _ptr(out, _c_u8p)) == 0
        return out

    def unpack(self, packed: np.ndarray, d_out: int, G: int, M: int) -> np.ndarray:
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        assert packed.size == self.packed_bytes(d_out, G, M)
        out = np.empty((d_out, G, M), dtype=np.uint8)
        assert self.lib.oracle_unpack_codes(_ptr(packed, _c_u8p), d_out, G, M, _ptr(out, _c_u8p)) == 0
        return out

    # -- encode ----------------------------------------------------------
    def encode_greedy(self, target: np.ndarray, codebooks: np.ndarray, M: Optional[int] = None) -> np.ndarray:
        """Greedy residual codes [d_out][G][M] (uint8) for float32 targets [d_out][d_in] (rotated weights
        divided by their row scale) and fp16 codebooks [M][256][8]."""
        t = np.ascontiguousarray(target, dtype=np.float32)
        cb = np.ascontiguousarray(codebooks).view(np.uint16)
        M = cb.shape[0] if M is None else M
        d_out, d_in = t.shape
        codes = np.empty((d_out, d_in // 8, M), dtype=np.uint8)
        rc = self.lib.oracle_encode_greedy(t.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), _ptr(cb, _c_u16p),
                                           d_out, d_in, M, _ptr(codes, _c_u8p))
        if rc != 0:
            raise ValueError(f"oracle_encode_greedy rc={rc}")
        return codes

    # -- storage ---------------------------------------------------------
    def storage_bits(self, d_out: int, d_in: int, g: int, M: int, B: int) -> float:
        return self.lib.oracle_storage_bits(d_out, d_in, g, M, B)

    def bits_per_param(self, d_out: int, d_in: int, g: int, M: int, B: int) -> float:
        return self.lib.oracle_bits_per_param(d_out, d_in, g, M, B)

    def set_threads(self, n: int) -> int:
        return self.lib.oracle_set_threads(n)


_default: Optional[Oracle] = None


def load(path: str = LIB) -> Oracle:
    """The oracle at `path`, built first when the default library is missing."""
    global _default
    if path == LIB:
        if _default is None:
            if not os.path.exists(LIB):
                build()
            _default = Oracle(LIB)
        return _default
    return Oracle(path)
