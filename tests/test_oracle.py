"""The fp64 oracle against its pins (CPU only), the hand-worked example, and a
mutation check: each plausible mistake planted in a copy of the oracle source
must make at least one pin fail."""
import json
import math
import os
import tempfile

import numpy as np
import pytest
import torch

import oracle
import oracle_pins
from oracle_pins import PINS, shape

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle()


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_worked_example(orc):
    g = json.load(open(GOLDEN))
    w = shape(**g["shape"])
    kidx = torch.tensor(g["inputs"]["k_idx"], dtype=torch.float32)[None]
    qidx = torch.tensor(g["inputs"]["q_idx"], dtype=torch.float32)[None, None]
    v = torch.tensor(g["inputs"]["v"], dtype=torch.float32)[None, None]
    inp = dict(q=torch.zeros(1, 2, 6, 2), k=torch.zeros(1, 1, 6, 2), v=v, q_idx=qidx, k_idx=kidx)
    out = orc.run(w, inp, block_scores=True)
    exp = g["expected"]
    bs = np.array([[-math.inf if x is None else x for x in row] for row in exp["block_scores"]])
    assert np.array_equal(out["block_scores"][0, 0], bs)
    assert out["sel"][0, 0].tolist() == exp["sel"]
    for h in range(2):
        assert np.allclose(out["o"][0, h], np.array(exp["o"]), atol=1e-14)
        assert np.allclose(np.exp(out["lse"][0, h]), exp["lse_exp"], atol=1e-12)


# Plausible mistakes: (name, [(source text, replacement), ...]).
MUTANTS = [
    ("index scores see one future key", [("if (hi > p + 1) hi = p + 1;\n    double m",
                                          "if (hi > p + 2) hi = p + 2;\n    double m")]),
    ("tie goes to the higher block", [("return (x->block > y->block) - (x->block < y->block);",
                                       "return (x->block < y->block) - (x->block > y->block);")]),
    ("lowest score first", [("if (x->score > y->score) return -1;",
                             "if (x->score > y->score) return 1;"),
                            ("if (x->score < y->score) return 1;",
                             "if (x->score < y->score) return -1;")]),
    ("local block not forced", [("for (int i = 0; i < top_k - 1; ++i) sel[n_sel++] = cand[i].block;\n"
                                 "    sel[n_sel++] = (int32_t)local;",
                                 "for (int i = 0; i < top_k; ++i) sel[n_sel++] = cand[i].block;")]),
    ("own block taken from position p-1", [("const int64_t local = p / block_size;",
                                            "const int64_t local = (p > 0 ? p - 1 : 0) / block_size;")]),
    ("take-all branch skips block 0", [("for (int c = 0; c <= local; ++c) sel[n_sel++] = c;",
                                        "for (int c = 1; c <= local; ++c) sel[n_sel++] = c;")]),
    ("no 1/sqrt(d_h) scale", [("const double scale = 1.0 / sqrt((double)d_h);",
                               "const double scale = 1.0;")]),
    ("head to group by modulo", [("const int r = h / group;", "const int r = h % h_kv;")]),
    ("attention sees future keys in the local block",
     [("if (hi > p + 1) hi = p + 1;\n    for (int64_t j = lo; j < hi; ++j) {\n      double s = 0.0;\n      for (int d = 0; d < d_h",
       "if (hi > p + 2) hi = p + 2;\n    for (int64_t j = lo; j < hi; ++j) {\n      double s = 0.0;\n      for (int d = 0; d < d_h"),
      ("if (hi > p + 1) hi = p + 1;\n    for (int64_t j = lo; j < hi; ++j) {\n      double w",
       "if (hi > p + 2) hi = p + 2;\n    for (int64_t j = lo; j < hi; ++j) {\n      double w")]),
    ("lse without the max shift", [("*lse = mu + log(total);", "*lse = log(total);")]),
    ("index key rows transposed", [("elem(k_idx_seq, j * d_idx + d, type)",
                                    "elem(k_idx_seq, d * (p + 1) + j, type)")]),
    ("bf16 widened with the wrong shift", [("((uint32_t)((const uint16_t *)base)[i]) << 16",
                                            "((uint32_t)((const uint16_t *)base)[i]) << 15")]),
    ("student scores without 1/sqrt(d_idx)", [("sidx[n] = s / sqrt((double)d_idx);",
                                              "sidx[n] = s;")]),
    ("teacher sums the heads", [("/ hs / (double)group;", "/ hs;")]),
    ("teacher without 1/sqrt(d_h)", [("zh[j] = s * scale;", "zh[j] = s;")]),
    ("KL in the reverse direction", [("if (t[j] > 0.0) loss += t[j] * (log(t[j]) - (sidx[j] - lse_s));",
                                      "loss += exp(sidx[j] - lse_s) * ((sidx[j] - lse_s) - log(t[j]));")]),
    ("student normaliser without the max", [("const double lse_s = mu + log(zsum);",
                                             "const double lse_s = log(zsum);")]),
    ("teacher heads of group r taken from r on", [("(((int64_t)b * h_q + (int64_t)r * group) * n_q + tq) * d_h",
                                                    "(((int64_t)b * h_q + (int64_t)r) * n_q + tq) * d_h")]),
    ("teacher head stride of one row", [("(const char *)q + q_off * (int64_t)es, (int64_t)n_q * d_h,",
                                         "(const char *)q + q_off * (int64_t)es, (int64_t)d_h,")]),
    ("gradient without the softmax's D term", [("const double dz = z[j] * (dp[j] - dsum);",
                                                "const double dz = z[j] * dp[j];")]),
    ("dk without 1/sqrt(d_h)", [("dk[key[j] * d_h + d] += dz * elem(q_row, d, type) * scale;",
                                 "dk[key[j] * d_h + d] += dz * elem(q_row, d, type);")]),
    ("dv weighted by dP instead of P", [("dv[key[j] * d_h + d] += z[j] * elem(do_row, d, type);",
                                         "dv[key[j] * d_h + d] += dp[j] * elem(do_row, d, type);")]),
    ("dq from v instead of k", [("dq[d] += dz * elem(k_plane, key[j] * d_h + d, type) * scale;",
                                 "dq[d] += dz * elem(v_plane, key[j] * d_h + d, type) * scale;")]),
    ("gradients land in the next group's planes", [("const int64_t kv_off = ((int64_t)b * h_kv + r) * (int64_t)n_k * d_h;\n      const void *kp",
                                                    "const int64_t kv_off = ((int64_t)b * h_kv + (r + 1) % h_kv) * (int64_t)n_k * d_h;\n      const void *kp")]),
    ("projection weights read column-major", [("elem(w_q, wo + i, type)",
                                               "elem(w_q, (int64_t)i * h_kv * d_idx + (int64_t)r * d_idx + d, type)")]),
    ("index queries stored row-major over groups", [("q_idx[((b * h_kv + r) * n + t) * d_idx + d] = s;",
                                                    "q_idx[((b * n + t) * h_kv + r) * d_idx + d] = s;")]),
    ("index key projected with the query weights", [("s += elem(x, xo + i, type) * elem(w_k, (int64_t)d * d_model + i, type);",
                                                    "s += elem(x, xo + i, type) * elem(w_q, (int64_t)d * d_model + i, type);")]),
    ("projection drops the last input coordinate", [("for (int i = 0; i < d_model; ++i) s += elem(x, xo + i, type) * elem(w_q",
                                                    "for (int i = 0; i < d_model - 1; ++i) s += elem(x, xo + i, type) * elem(w_q")]),
    ("query position ignores q_start", [("const int64_t t = rows[i], p = (int64_t)q_start + t;\n      const int64_t qoff = (((int64_t)b * h_kv",
                                         "const int64_t t = rows[i], p = t;\n      const int64_t qoff = (((int64_t)b * h_kv")]),
]


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, edits):
    src = open(oracle.SRC).read()
    for old, new in edits:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        open(path, "w").write(src)
        lib = oracle.build(src=path, out=os.path.join(d, "libmutant.so"))
        mutant = oracle.Oracle(lib)
        caught = []
        for pin in PINS:
            try:
                pin(mutant)
            except (AssertionError, RuntimeError):
                caught.append(pin.__name__)
        assert caught, f"no pin caught the mutant '{name}'"
