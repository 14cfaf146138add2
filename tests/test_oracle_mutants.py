"""The oracle's pins must be sensitive: each planted mistake below (a wrong
sign or index, a swapped operand, a dropped term) is compiled into a private
copy of the oracle on the CPU, and at least one pin must reject it.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "na3d_oracle.c")

# (name, exact source text, replacement)
MUTANTS = [
    ("no_high_clamp", "if (s > L - K) s = L - K;", ""),
    ("no_low_clamp", "if (s < 0) s = 0;", ""),
    ("even_window_other_side", "int s = i - K / 2;", "int s = i - (K - 1) / 2;"),
    ("off_by_one_centre", "int s = i - K / 2;", "int s = i - K / 2 + 1;"),
    ("left_aligned_window", "int s = i - K / 2;", "int s = i;"),
    # index mistakes that stay inside the buffers
    ("window_t_ignored", "(st + dt)) * H + (sh + dh)) * W", "(t + 0 * dt)) * H + (sh + dh)) * W"),
    ("w_offset_from_h", "* W + (sw + dw)) *", "* W + (sw + dh % KW)) *"),
    ("q_k_swapped", "bf16_to_double(q[qoff + d]) * bf16_to_double(k[koff + d])",
     "bf16_to_double(q[koff + d]) * bf16_to_double(k[qoff + d])"),
    ("v_read_from_k", "o[d] += e[j] * bf16_to_double(v[voff + d]);",
     "o[d] += e[j] * bf16_to_double(k[voff + d]);"),
    ("no_normalisation", "for (int d = 0; d < HD; ++d) o[d] /= l;", ""),
    ("head_stride_dropped", "tok_stride +\n            n * head_stride;\n        double acc",
     "tok_stride;\n        double acc"),
    ("last_dim_dropped", "for (int d = 0; d < HD; ++d)\n          acc +=",
     "for (int d = 0; d < HD - 1; ++d)\n          acc +="),
    ("exp_sign", "e[j] = exp(s[j] - m);", "e[j] = exp(m - s[j]);"),
    ("max_not_subtracted", "e[j] = exp(s[j] - m);", "e[j] = exp(s[j]);"),
    ("weights_reversed", "wts[j] = e[j] / l;", "wts[K - 1 - j] = e[j] / l;"),
    ("weights_unnormalised", "wts[j] = e[j] / l;", "wts[j] = e[j];"),
]

CHECKS = [
    lambda o: pins.test_golden_window_starts(o),
    lambda o: pins.test_window_start_matches_interval_search(o),
    lambda o: pins.test_oracle_vs_dense_masked(o, (4, 6, 8), (3, 3, 5), 8),
    lambda o: pins.test_oracle_vs_dense_masked(o, (5, 4, 3), (5, 3, 1), 32),
    lambda o: pins.test_oracle_vs_dense_masked_tiny_workload(o),
    lambda o: pins.test_unit_window_returns_v_exactly(o),
    lambda o: pins.test_zero_query_gives_window_mean(o),
    lambda o: pins.test_dominant_key_is_selected(o),
    lambda o: pins.test_window_equal_to_grid_is_dense_attention(o),
    lambda o: pins.test_weights_match_dense_masked_in_window_order(o),
    lambda o: pins.test_extreme_scores_stay_finite(o),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(tmp_path, source, name, old, new):
    assert source.count(old) >= 1, "mutation site vanished: " + name
    src = tmp_path / ("mutant_%s.c" % name)
    src.write_text(source.replace(old, new))
    so = tmp_path / ("libmutant_%s.so" % name)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(src),
                    "-o", str(so), "-lm"], check=True)
    real = oracle._load()
    mut = ctypes.CDLL(str(so))
    for fn in ("na3d_oracle_window_start", "na3d_oracle_max_threads", "na3d_oracle_fwd",
               "na3d_oracle_fwd_points", "na3d_oracle_weights"):
        getattr(mut, fn).argtypes = getattr(real, fn).argtypes
        getattr(mut, fn).restype = getattr(real, fn).restype
    caught = []
    try:
        oracle._lib = mut
        for i, check in enumerate(CHECKS):
            try:
                check(oracle)
            except (AssertionError, ValueError):
                caught.append(i)
    finally:
        oracle._lib = real
    assert caught, "no pin rejected mutant " + name
