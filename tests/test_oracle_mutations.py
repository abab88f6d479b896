"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a flipped sign,
a dropped term, a transposed operand, a wrong tie rule, ...), builds it into a
scratch library, and checks that at least one pin fails against it.  The real
oracle source is never modified.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_alloc as PA
import test_oracle_attention as PT
import test_oracle_factors as PF
import test_oracle_policies as PP
import test_oracle_svd as PS

SRC = os.path.join(os.path.dirname(oracle.__file__), "milo_oracle.c")


def _block():
    from synthetic import planted_blocks
    X = planted_blocks(1, 256, 128, (4.0, 32.0), 31, out_dtype="f64").numpy()[0]
    sigma, V, _ = oracle.svd_blocks(X[None])
    return X, sigma[0], V[0]


MUTATIONS = [
    ("rotation sign", "wp[t] = c * a - s * b;", "wp[t] = c * a + s * b;",
     lambda: PS.test_planted_spectrum_recovered(oracle, 256)),
    ("right vectors not rotated", "vp[j] = c * a - s * b;", "vp[j] = a;",
     lambda: PS.test_full_rank_reconstruction(oracle)),
    ("singular values sorted ascending", "norms[order[j]] < norms[key]",
     "norms[order[j]] > norms[key]", lambda: PS.test_planted_spectrum_recovered(oracle, 256)),
    ("greedy tie goes to the last block", "gain > best_gain", "gain >= best_gain",
     lambda: PA.test_equal_spectra_round_robin(oracle)),
    ("gain uses sigma instead of sigma^2", "double gain = log1p(s * s / eps2);",
     "double gain = log1p(s / eps2);",
     lambda: PA.test_greedy_is_optimal_by_enumeration(oracle, 3, 4)),
    ("projection uses V transposed", "X[(size_t)t * d + j] * V[(size_t)j * d + i]",
     "X[(size_t)t * d + j] * V[(size_t)i * d + j]",
     lambda: PF.test_eckart_young(oracle, _block(), 40)),
    ("reconstruction drops the last rank", "for (int i = 0; i < r; ++i)\n                acc += A",
     "for (int i = 0; i + 1 < r; ++i)\n                acc += A",
     lambda: PF.test_identity_at_full_rank(oracle, _block())),
    ("bf16 ties away from zero", "double r = nearbyint(x / quantum) * quantum;",
     "double r = round(x / quantum) * quantum;", lambda: PF.test_round_bf16_hand_values(oracle)),
    ("int8 truncates", "float v = nearbyintf((float)row[c] / s);",
     "float v = truncf((float)row[c] / s);", lambda: PF.test_int8_hand_values(oracle)),
    ("int4 scale over 8 levels", "float s = m / 7.0f;", "float s = m / 8.0f;",
     lambda: PF.test_int4_hand_values(oracle)),
    ("int4 groups overlap", "const double *x = M + (size_t)r * cols + (size_t)g * group;",
     "const double *x = M + (size_t)r * cols + (size_t)g;",
     lambda: PF.test_int4_hand_values(oracle)),
    ("int2 scale over 4 levels", "float s = m / 3.0f;", "float s = m / 4.0f;",
     lambda: PF.test_int2_hand_values(oracle)),
    ("int2 ties toward zero", "q = v <= -2.0f ? 0 : 1;", "q = v < -2.0f ? 0 : 1;",
     lambda: PF.test_int2_hand_values(oracle)),
    ("int2 groups overlap", "const double *run = M + (size_t)r * cols + (size_t)g * group;",
     "const double *run = M + (size_t)r * cols + (size_t)g;",
     lambda: PF.test_int2_hand_values(oracle)),
    ("int2 zero on the negative level", "q = v >= 2.0f ? 3 : 2;", "q = v >= 2.0f ? 3 : (v > 0.0f ? 2 : 1);",
     lambda: PF.test_int2_hand_values(oracle)),
    ("rope second component sign", "x[j + h] = a * s + b * c;", "x[j + h] = a * s - b * c;",
     lambda: PT.test_rope_matches_complex_form(oracle)),
    ("rope frequency exponent", "pow(base, -2.0 * j / (double)d)", "pow(base, -1.0 * j / (double)d)",
     lambda: PT.test_rope_matches_complex_form(oracle)),
    ("softmax without max subtraction", "double p = exp(logit[t] - m);", "double p = exp(logit[t]);",
     lambda: PT.test_attention_closed_forms(oracle)),
    ("attention output not normalised", "out[j] /= den;", "out[j] /= 1.0;",
     lambda: PT.test_attention_matches_torch_sdpa(oracle)),
    ("key rotated at the query position", "oracle_rope(kr, d, (double)pos[t], base);",
     "oracle_rope(kr, d, (double)q_pos, base);", lambda: PT.test_attention_matches_torch_sdpa(oracle)),
    ("splitmix64 first shift", "z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;",
     "z = (z ^ (z >> 31)) * 0xBF58476D1CE4E5B9ull;", lambda: PP.test_splitmix64_reference_output()),
    ("uniform remainder to the last blocks", "rank[j] = (int32_t)(Rp / n + (j < Rp % n ? 1 : 0));",
     "rank[j] = (int32_t)(Rp / n + (j >= n - Rp % n ? 1 : 0));",
     lambda: PP.test_uniform_is_the_greedy_on_identical_spectra(5, 8, 17)),
]


@pytest.mark.parametrize("name,old,new,pin", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pin_catches_mutation(tmp_path, name, old, new, pin):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                    "-o", str(so), str(mutated), "-lm"], check=True)
    saved = oracle.lib()
    oracle._lib = oracle.load(str(so))
    try:
        with np.errstate(all="ignore"):
            with pytest.raises(AssertionError):
                pin()
    finally:
        oracle._lib = saved


def test_unmutated_pins_pass():
    """The same pin calls pass on the real oracle (so the failures above are the mutations')."""
    for _, _, _, pin in MUTATIONS:
        pin()


# Mistakes planted in the oracle's Python layer (the loops over pools, sequences,
# KV heads and query heads), each against the pin that must catch it.
PY_SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")
PY_MUTATIONS = [
    ("query heads interleaved over KV heads", "hq = h * G + g", "hq = g * n_kv_heads + h",
     lambda m: PT.test_decode_batches_kv_heads_and_groups(m)),
    ("block id with heads outermost", "fid = (s * n_kv_heads + h) * blocks_per_seq + b",
     "fid = (h * batch + s) * blocks_per_seq + b", lambda m: PT.test_decode_batches_kv_heads_and_groups(m)),
    ("first sequence's selection for every sequence", "else [int(b) for b in sel[s]]",
     "else [int(b) for b in sel[0]]", lambda m: PT.test_decode_batches_kv_heads_and_groups(m)),
    ("first pool's budget for every pool", "int(budgets[p]), eps2, policy, seed, p)",
     "int(budgets[0]), eps2, policy, seed, p)", lambda m: PA.test_compress_several_pools(m)),
]


@pytest.mark.parametrize("name,old,new,pin", PY_MUTATIONS, ids=[m[0] for m in PY_MUTATIONS])
def test_pin_catches_python_mutation(name, old, new, pin):
    import importlib.util
    import sys
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    spec = importlib.util.spec_from_loader("oracle_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    mod.__file__ = PY_SRC  # so that it loads the same liboracle.so
    sys.modules["oracle_mutant"] = mod
    try:
        exec(compile(src.replace(old, new), PY_SRC, "exec"), mod.__dict__)
        with pytest.raises(AssertionError):
            pin(mod)
    finally:
        del sys.modules["oracle_mutant"]


def test_unmutated_python_pins_pass():
    for _, _, _, pin in PY_MUTATIONS:
        pin(oracle)
