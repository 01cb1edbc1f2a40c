"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of the oracle source with one plausible slip (a wrong
sign or index, a dropped term, a transposed operand, a wrong rounding); it is
compiled into a temporary library and the full pin set is run against it in a
child process.  A mutant that passes every pin would mean the pins leave that
part of the oracle unchecked.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "oracle_pins.py")

MUTANTS = {
    "hadamard_or_instead_of_and": ("popcount32((uint32_t)(r & c))", "popcount32((uint32_t)(r | c))"),
    "hadamard_negated": ("& 1) ? -1 : 1;", "& 1) ? 1 : -1;"),
    "rotation_no_normalisation": ("ob[r] = acc * inv;", "ob[r] = acc;"),
    "rotation_wrong_input_index": ("H[(int64_t)r * b + c] * xb[c];", "H[(int64_t)r * b + c] * xb[r];"),
    "rotation_block_offset_dropped": ("const double *xb = x + n * d_in + beta * b;", "const double *xb = x + n * d_in;"),
    "signed_eps_ignored": ("acc += (double)H[(int64_t)r * b + c] * (es[c] * xs[c]);",
                           "acc += (double)H[(int64_t)r * b + c] * (xs[c]);"),
    "sign_bits_msb_first": ("eps[c] = ((signs[c / 8] >> (c % 8)) & 1u)", "eps[c] = ((signs[c / 8] >> (7 - c % 8)) & 1u)"),
    "sign_block_offset_dropped": ("const double *es = eps + beta * b;", "const double *es = eps;"),
    "signed_no_normalisation": ("os[r] = acc * inv;", "os[r] = acc;"),
    "encode_residual_not_updated": ("r[t] = r[t] - cm[best * ORACLE_GROUP + t];", "r[t] = r[t];"),
    "encode_ties_to_higher_index": ("if (c == 0 || d < best_d) {", "if (c == 0 || d <= best_d) {"),
    "encode_one_plane_for_all": ("const float *cm = cbf + (int64_t)m * ORACLE_CODEWORDS * ORACLE_GROUP;",
                                 "const float *cm = cbf;"),
    "encode_elements_reversed": ("const float e = r[t] - cm[c * ORACLE_GROUP + t];",
                                 "const float e = r[t] - cm[c * ORACLE_GROUP + (ORACLE_GROUP - 1 - t)];"),
    "encode_planes_stored_reversed": ("codes[q * M + m] = (uint8_t)best;", "codes[q * M + (M - 1 - m)] = (uint8_t)best;"),
    "first_codebook_dropped": ("for (int32_t m = 0; m < k; ++m) {", "for (int32_t m = 1; m < k; ++m) {"),
    "prefix_ignored": ("for (int32_t m = 0; m < k; ++m) {", "for (int32_t m = 0; m < M; ++m) {"),
    "planes_reversed": ("const uint8_t c = codes[(i * G + j) * M + m];", "const uint8_t c = codes[(i * G + j) * M + (M - 1 - m)];"),
    "codeword_elements_reversed": ("g += codebooks[((int64_t)m * ORACLE_CODEWORDS + c) * ORACLE_GROUP + t];",
                                   "g += codebooks[((int64_t)m * ORACLE_CODEWORDS + c) * ORACLE_GROUP + (ORACLE_GROUP - 1 - t)];"),
    "scale_dropped": ("const double s = scales ? scales[i] : 1.0;", "const double s = 1.0;"),
    "groups_transposed": ("w[j * ORACLE_GROUP + t] = s * g;", "w[t * G + j] = s * g;"),
    "matvec_index_reversed": ("acc += w[c] * xr[c];", "acc += w[c] * xr[d_in - 1 - c];"),
    "batch_row_ignored": ("const double *xr = xrot + n * d_in;", "const double *xr = xrot;"),
    "f16_decode_exponent": ("ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    "f16_decode_subnormal": ("ldexp((double)f, -24)", "ldexp((double)f, -25)"),
    "bf16_decode_exponent": ("ldexp((double)(128 + f), e - 134)", "ldexp((double)(128 + f), e - 133)"),
    "encode_truncates": ("q = nearbyint(ldexp(a, mant - ex));", "q = floor(ldexp(a, mant - ex));"),
    "encode_overflow_bound": ("if (ex + bias >= emax_field)", "if (ex + bias > emax_field)"),
    "bf16_encode_width": ("encode_mag(fabs(v), 7, 127, 255)", "encode_mag(fabs(v), 8, 127, 255)"),
    "pack_tile_transposed": ("+ l * ORACLE_TILE_ROWS + r;", "+ r * ORACLE_TILE_GROUPS + l;"),
    "pack_tiles_row_major": ("(jt * R + it)", "(it * tiles_g(P) + jt)"),
    "pack_planes_interleaved": ("packed[packed_offset(i, j, m, R, P)] = codes[(i * G + j) * M + m];",
                                "packed[packed_offset(i, j, 0, R, P) * M + m] = codes[(i * G + j) * M + m];"),
    "unpack_planes_reversed": ("codes[(i * G + j) * M + m] = packed[packed_offset(i, j, m, R, P)];",
                               "codes[(i * G + j) * M + m] = packed[packed_offset(i, j, M - 1 - m, R, P)];"),
    "storage_scale_bits": ("(double)d_out * 16.0;", "(double)d_out * 8.0;"),
    "storage_codebook_bits": ("ldexp(1.0, B) * 16.0", "ldexp(1.0, B) * 8.0"),
}


def _run_pins(lib):
    return subprocess.run([sys.executable, PINS, lib], capture_output=True, text=True, timeout=300)


def test_unmodified_oracle_passes_in_child(tmp_path):
    lib = oracle.build(oracle.SRC, str(tmp_path / "liboracle_ref.so"))
    r = _run_pins(lib)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    before, after = MUTANTS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(before) == 1, f"mutation site for {name} not unique in the oracle source"
    mutant = tmp_path / f"{name}.c"
    mutant.write_text(src.replace(before, after))
    lib = oracle.build(str(mutant), str(tmp_path / f"lib{name}.so"))
    r = _run_pins(lib)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}"
