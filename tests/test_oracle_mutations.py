"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins in ``test_oracle_pins.py`` catch every one of them.

Each mutation is a textual edit of ``oracle/lora_oracle.c`` compiled into a
temporary library; the real oracle is untouched.  Mutations are chosen so
that every access stays in bounds.
"""
from __future__ import annotations

import os

import pytest

import oracle
from test_oracle_pins import PINS

MUTATIONS = [
    ("drop_scale", "li[c] = s * acc;", "li[c] = acc;"),
    ("sign_flip", "y[i * d_out + c] = bi[c] + li[c];", "y[i * d_out + c] = bi[c] - li[c];"),
    ("drop_lora_term", "y[i * d_out + c] = bi[c] + li[c];", "y[i * d_out + c] = bi[c];"),
    ("drop_base_term", "y[i * d_out + c] = bi[c] + li[c];", "y[i * d_out + c] = li[c];"),
    ("A_transposed", "Aa[k * r + j]", "Aa[(int64_t)j * d_in + k]"),
    ("B_transposed", "Ba[(int64_t)j * d_out + c]", "Ba[c * r + j]"),
    ("W_transposed", "bi[c] += xk * Wk[c];", "bi[c] += xk * W[c * d_in + k];"),
    ("rank_off_by_one", "for (int32_t j = 0; j < r; ++j) {\n                const double* Aa",
     "for (int32_t j = 0; j + 1 < r; ++j) {\n                const double* Aa"),
    ("expand_wrong_t_index", "acc += ti[j] * Ba", "acc += ti[0] * Ba"),
    ("t_not_cleared", "for (int32_t j = 0; j < r_max; ++j) ti[j] = 0.0;", ""),
    ("base_skips_first_k", "for (int64_t k = 0; k < d_in; ++k) {\n                        double xk",
     "for (int64_t k = 1; k < d_in; ++k) {\n                        double xk"),
    ("minus_one_counted_bad", "if (a != -1 && !valid) ++bad;", "if (!valid) ++bad;"),
    ("segments_unstable", "for (int64_t i = 0; i < n_rows; ++i) {\n            int32_t key",
     "for (int64_t i = n_rows - 1; i >= 0; --i) {\n            int32_t key"),
    ("segments_offset_shift", "seg_off[s] = (int32_t)start;", "seg_off[s] = (int32_t)start + (s > 0);"),
    ("segments_descending", "for (int32_t v = -1; v < n_adapters; ++v) {",
     "for (int32_t v = n_adapters - 1; v >= -1; --v) {"),
    ("segments_invalid_dropped", "int32_t key = id_valid(ids[i], n_adapters) ? ids[i] : -1;",
     "int32_t key = ids[i];"),
    ("shrink_uses_scale", "ti[j] = acc;\n", "ti[j] = scales[a] * acc;\n"),
    ("merge_drop_scale", "W[k * d_out + c] += s * acc;", "W[k * d_out + c] += acc;"),
    ("merge_overwrites", "W[k * d_out + c] += s * acc;", "W[k * d_out + c] = s * acc;"),
    ("merge_sign_ignored", "const double s = sign * scales[adapter];", "const double s = scales[adapter];"),
    ("merge_A_transposed", "acc += Ak[j] *", "acc += Aa[(int64_t)j * d_in + k] *"),
    ("merge_B_transposed", "Ba[c + (int64_t)j * d_out]", "Ba[c * r + j]"),
    ("q4_nibbles_swapped", "const int nib = (k % 2 == 0) ? (byte & 15) : (byte >> 4);",
     "const int nib = (k % 2 == 0) ? (byte >> 4) : (byte & 15);"),
    ("q4_unsigned", "const int v = nib >= 8 ? nib - 16 : nib;", "const int v = nib;"),
    ("q4_group_from_byte_index", "(double)v * scale[n * lds + k / group]",
     "(double)v * scale[n * lds + (k / 2) / group]"),
    ("q4_transposed_out", "W[k * d_out + n] = (double)v", "W[n * d_in + k] = (double)v"),
    ("merge_rank_off_by_one", "for (int32_t j = 0; j < r; ++j) acc += Ak[j]",
     "for (int32_t j = 0; j + 1 < r; ++j) acc += Ak[j]"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, old, new, tmp_path):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    mutated = src.replace(old, new)
    path = tmp_path / "mut.c"
    path.write_text(mutated)
    so = str(tmp_path / f"libmut_{name}.so")
    oracle.build(str(path), so)
    lib = oracle.load(so)
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except Exception as e:  # noqa: BLE001 - any failure of a pin counts
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"mutation {name} passed every pin"
    os.remove(so)
