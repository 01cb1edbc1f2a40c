"""Seeded synthetic workloads for the additive-codebook decode linear.

This module only draws random numbers and lays them out: it holds none of
the method's arithmetic (no rotation, no codeword sums, no products), so
both the CPU oracle and the HIP path can consume what it produces without
sharing any computation.

Shapes and distributions follow the decode workloads of the Drop-by-Drop
paper ("Multi-Bitwidth Quantization for LLMs Using Additive Codebooks",
section 6 "Experimental Setup" and "Method Definitions": groups of g=8,
8-bit codebooks, M in {3,4,5}; evaluated models include Meta-Llama-3-8B,
whose projection shapes the layer configs below copy).  Trained
checkpoints are not available, so codes are uniform random bytes (the
byte stream and access pattern a decoder sees are the same), codebooks
are N(0, 0.05) in fp16 and per-row scales U(0.5, 1.5) in fp16.

Every tensor has its own PCG64 stream derived from (config seed, layer,
projection, tensor kind), so any tensor can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence, Tuple

import numpy as np

GROUP = 8          # g: inputs per codeword
CODEWORDS = 256    # 2^B with B = 8 bit codes
BASE_SEED = 0xA0D00000

_KIND = {"codes": 1, "codebooks": 2, "scales": 3, "x": 4, "k": 5, "misc": 6}
_PROJ = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "single": 7}


def rng(seed: int, layer: int = 0, proj: str = "single", kind: str = "misc", extra: int = 0) -> np.random.Generator:
    """Independent generator for one tensor of one layer of one workload."""
    ss = np.random.SeedSequence([seed & 0xFFFFFFFF, layer, _PROJ[proj], _KIND[kind], extra])
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16, returned as uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    nan = np.isnan(a)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def gen_codes(g: np.random.Generator, d_out: int, d_in: int, M: int) -> np.ndarray:
    """uint8 codes in logical order [d_out][d_in/8][M], uniform over 0..255."""
    assert d_in % GROUP == 0
    return g.integers(0, CODEWORDS, size=(d_out, d_in // GROUP, M), dtype=np.uint8)


def gen_codebooks(g: np.random.Generator, M: int, sigma: float = 0.05) -> np.ndarray:
    """fp16 codebooks [M][256][8], entries N(0, sigma) rounded to nearest fp16."""
    return (g.standard_normal((M, CODEWORDS, GROUP)) * sigma).astype(np.float16)


def gen_scales(g: np.random.Generator, d_out: int, lo: float = 0.5, hi: float = 1.5) -> np.ndarray:
    """fp16 per-output-row scales, U(lo, hi) rounded to nearest fp16."""
    return g.uniform(lo, hi, size=d_out).astype(np.float16)


def gen_signs(g: np.random.Generator, d_in: int) -> np.ndarray:
    """Sign bit mask of a randomized rotation: d_in / 8 uniformly random bytes (each bit a fair coin)."""
    return g.integers(0, 256, size=d_in // 8, dtype=np.uint8)


def gen_encode_targets(g: np.random.Generator, d_out: int, d_in: int, M: int, sigma_c: float = 0.05):
    """Synthetic encoder input: rotated Gaussian weights and their row scales.

    W Q^T of an i.i.d. Gaussian W under an orthonormal Q is again i.i.d.
    Gaussian, so the rotated weights are drawn directly as N(0, 1) float32.
    The row scale is chosen so the scaled row has the RMS of a sum of M
    codewords with N(0, sigma_c) entries: s_i = fp16(rms_i / (sigma_c sqrt(M))).
    Returns (w_rot float32 [d_out][d_in], scales fp16 [d_out],
    target float32 [d_out][d_in] = w_rot / s_i).
    """
    w = g.standard_normal((d_out, d_in)).astype(np.float32)
    rms = np.sqrt(np.mean(w.astype(np.float64) ** 2, axis=1)) if d_in else np.ones(d_out)
    s = (rms / (sigma_c * np.sqrt(M))).astype(np.float16)
    target = (w.astype(np.float64) / s.astype(np.float64)[:, None]).astype(np.float32)
    return w, s, target


def gen_x(g: np.random.Generator, batch: int, d_in: int, dtype: str = "f16") -> np.ndarray:
    """Activations N(0,1): fp16 array for 'f16', uint16 bf16 bit patterns for 'bf16'."""
    v = g.standard_normal((batch, d_in))
    if dtype == "f16":
        return v.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(v.astype(np.float32))
    raise ValueError(dtype)


def dyadic_case(g: np.random.Generator, d_out: int, d_in: int, M: int, batch: int = 1):
    """Inputs whose products and sums are exact in fp32 and fp16.

    Codeword entries are in {-2,-1,0,1,2}/4, scales are 1 and the (already
    rotated) activations are in {-1,0,1}; every partial sum is a multiple of
    1/4 bounded by 2*M*d_in/4, so any summation order gives the same bits.
    """
    codes = gen_codes(g, d_out, d_in, M)
    cb = (g.integers(-2, 3, size=(M, CODEWORDS, GROUP)) / 4.0).astype(np.float16)
    s = np.ones(d_out, dtype=np.float16)
    x = g.integers(-1, 2, size=(batch, d_in)).astype(np.float16)
    return codes, cb, s, x


@dataclasses.dataclass(frozen=True)
class Linear:
    """One decode linear: y[B][d_out] = s * (W_k @ H_b x)."""
    name: str
    d_out: int
    d_in: int
    M: int
    ks: Tuple[int, ...]
    batches: Tuple[int, ...]
    block: int          # Hadamard block size b
    x_dtype: str = "f16"
    layer: int = 0
    proj: str = "single"


def block_for(d_in: int) -> int:
    """Hadamard block used for an input width: 256 for the 14336-wide down input, else 128."""
    return 256 if d_in % 256 == 0 and d_in > 8192 else 128


LLAMA8B = {  # (d_out, d_in) per projection of a Llama-3-8B decoder layer
    "q": (4096, 4096), "k": (1024, 4096), "v": (1024, 4096), "o": (4096, 4096),
    "gate": (14336, 4096), "up": (14336, 4096), "down": (4096, 14336),
}


def config(cid: int) -> List[Linear]:
    """The five workload configurations (1-based ids)."""
    if cid == 1:
        return [Linear("single256", 256, 256, 2, (1, 2), (1,), 64)]
    if cid == 2:
        return [Linear("q_proj4096", 4096, 4096, 4, (1, 2, 3, 4), (1,), 128, proj="q")]
    if cid == 3:
        return [Linear("gate14336x4096", 14336, 4096, 4, (1, 2, 3, 4), (1, 2, 4, 8), 128, proj="gate"),
                Linear("up14336x4096", 14336, 4096, 4, (1, 2, 3, 4), (1, 2, 4, 8), 128, proj="up"),
                Linear("down4096x14336", 4096, 14336, 4, (1, 2, 3, 4), (1, 2, 4, 8), 256, proj="down")]
    if cid == 4:
        ks = stack_ks()
        out = []
        for layer in range(32):
            for p in ("q", "k", "v", "o", "gate", "up", "down"):
                d_out, d_in = LLAMA8B[p]
                out.append(Linear(f"L{layer}.{p}", d_out, d_in, 4, (ks[layer],), (1,), block_for(d_in),
                                  layer=layer, proj=p))
        return out
    if cid == 5:
        return [Linear("gate14336x4096_sb", 14336, 4096, 4, (4, 2), (16, 32, 64), 128, "bf16", proj="gate"),
                Linear("down4096x14336_sb", 4096, 14336, 4, (4, 2), (16, 32, 64), 256, "bf16", proj="down")]
    raise ValueError(cid)


def stack_ks(n_layers: int = 32) -> List[int]:
    """Per-layer number of codebooks kept for the 32-layer stack, drawn from {2,3,4}."""
    g = rng(BASE_SEED + 4, kind="k")
    return [int(v) for v in g.integers(2, 5, size=n_layers)]


def layer_inputs(cid: int, lin: Linear, batch: int = 1, x_extra: int = 0):
    """codes [d_out][G][M] u8, codebooks [M][256][8] f16, scales [d_out] f16, x [B][d_in]."""
    seed = BASE_SEED + cid
    codes = gen_codes(rng(seed, lin.layer, lin.proj, "codes"), lin.d_out, lin.d_in, lin.M)
    cb = gen_codebooks(rng(seed, lin.layer, lin.proj, "codebooks"), lin.M)
    s = gen_scales(rng(seed, lin.layer, lin.proj, "scales"), lin.d_out)
    x = gen_x(rng(seed, lin.layer, lin.proj, "x", extra=1000 * batch + x_extra), batch, lin.d_in, lin.x_dtype)
    return codes, cb, s, x
