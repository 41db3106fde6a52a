"""Each plausible mistake planted in a copy of the oracle fails some pin.

The real oracle source is never modified: every mutant is a text edit of a
temporary copy, compiled with gcc on the CPU into a temporary directory.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "pkm_oracle.c")

# (name, original text, mistaken text): each original must occur exactly once.
MUTANTS = [
    ("swapped query halves",
     "const int64_t q_off = (t * H + h) * (int64_t)d_k + (int64_t)s * half;\n    const int64_t k_off",
     "const int64_t q_off = (t * H + h) * (int64_t)d_k + (int64_t)(1 - s) * half;\n    const int64_t k_off"),
    ("dropped last term of a half score",
     "for (int c = 0; c < half; ++c)\n        acc += elem(q, q_dt, q_off + c)",
     "for (int c = 0; c < half - 1; ++c)\n        acc += elem(q, q_dt, q_off + c)"),
    ("transposed slot index",
     "out[(int64_t)i * n + j] = left[i] + right[j];",
     "out[(int64_t)j * n + i] = left[i] + right[j];"),
    ("right score subtracted",
     "out[(int64_t)i * n + j] = left[i] + right[j];",
     "out[(int64_t)i * n + j] = left[i] - right[j];"),
    ("ascending sort",
     "if (x->score > y->score)\n        return -1;\n    if (x->score < y->score)\n        return 1;",
     "if (x->score > y->score)\n        return 1;\n    if (x->score < y->score)\n        return -1;"),
    ("ties to the highest slot",
     "return (x->slot > y->slot) - (x->slot < y->slot);",
     "return (x->slot < y->slot) - (x->slot > y->slot);"),
    ("unnormalised weights",
     "w[r] /= z;",
     "w[r] /= 1.0 + 0.0 * z;"),
    ("off-by-one (k+1)-th score",
     "kth1[t * H + h] = (k < nn) ? all[k].score : -INFINITY;",
     "kth1[t * H + h] = (k < nn) ? all[k - 1].score : -INFINITY;"),
    ("only the first head summed",
     "for (int h = 0; h < H; ++h)\n        for (int r = 0; r < k; ++r) {\n            const int64_t e = (t * H + h) * (int64_t)k + r;\n            const int64_t row",
     "for (int h = 0; h < 1; ++h)\n        for (int r = 0; r < k; ++r) {\n            const int64_t e = (t * H + h) * (int64_t)k + r;\n            const int64_t row"),
    ("weight dropped in the output sum",
     "yt[x] += w[e] * elem(values, v_dt, row + x);",
     "yt[x] += elem(values, v_dt, row + x);"),
    ("dw against the wrong row",
     "acc += elem(dy, dy_dt, t * d_v + x) * elem(values, v_dt, row + x);",
     "acc += elem(dy, dy_dt, t * d_v + x) * elem(values, v_dt, x);"),
    ("softmax backward sign",
     "ds[base + r] = weights[base + r] * (dw[base + r] - wdw);",
     "ds[base + r] = weights[base + r] * (wdw - dw[base + r]);"),
    ("right gradient routed to the left index",
     "dS[((t * H + h) * 2 + 1) * (int64_t)n + f % n] += ds[e];",
     "dS[((t * H + h) * 2 + 1) * (int64_t)n + f / n] += ds[e];"),
    ("value gradient without the weight",
     "row[x] += weights[e] * elem(dy, dy_dt, t * d_v + x);",
     "row[x] += elem(dy, dy_dt, t * d_v + x);"),
    ("dq from the other codebook",
     "acc += g[i] * elem(keys, k_dt, (((int64_t)h * 2 + s) * n + i) * half + c);",
     "acc += g[i] * elem(keys, k_dt, (((int64_t)h * 2 + (1 - s)) * n + i) * half + c);"),
    ("given selection: slot decoded with the halves swapped",
     "scores[base + r] = half_score(t, h, 0, f / n, H, n, d_k, q, q_dt, keys, k_dt) +\n"
     "                                   half_score(t, h, 1, f % n, H, n, d_k, q, q_dt, keys, k_dt);",
     "scores[base + r] = half_score(t, h, 0, f % n, H, n, d_k, q, q_dt, keys, k_dt) +\n"
     "                                   half_score(t, h, 1, f / n, H, n, d_k, q, q_dt, keys, k_dt);"),
    ("given selection: right half dropped",
     "scores[base + r] = half_score(t, h, 0, f / n, H, n, d_k, q, q_dt, keys, k_dt) +\n"
     "                                   half_score(t, h, 1, f % n, H, n, d_k, q, q_dt, keys, k_dt);",
     "scores[base + r] = half_score(t, h, 0, f / n, H, n, d_k, q, q_dt, keys, k_dt) +\n"
     "                                   0.0 * half_score(t, h, 1, f % n, H, n, d_k, q, q_dt, keys, k_dt);"),
    ("given selection: right half scored on the left codebook",
     "                                   half_score(t, h, 1, f % n, H, n, d_k, q, q_dt, keys, k_dt);",
     "                                   half_score(t, h, 0, f % n, H, n, d_k, q, q_dt, keys, k_dt);"),
    ("dkeys from the other query half",
     "const int64_t q_off = (t * H + h) * (int64_t)d_k + (int64_t)s * half;\n                for",
     "const int64_t q_off = (t * H + h) * (int64_t)d_k + (int64_t)(1 - s) * half;\n                for"),
]


@pytest.fixture(scope="module")
def source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,orig,bad", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, orig, bad):
    assert source.count(orig) == 1, f"mutation target for '{name}' not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "mutant.c")
        with open(src, "w") as f:
            f.write(source.replace(orig, bad))
        lib = oracle.build(src=src, out=os.path.join(d, "libmutant.so"))
        failed = oracle_pins.failing_pins(oracle.Oracle(lib))
    assert failed, f"no pin catches the planted mistake '{name}'"
