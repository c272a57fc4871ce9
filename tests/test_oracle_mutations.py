"""Plant plausible mistakes in a copy of the oracle and check that the pins
catch each of them. This shows the pins constrain every part of the oracle
(predicates, score_mods, the softmax, its normalisation and log, the scale,
the operand order, grouped heads, block classification and index lists).
The mistakes are planted on the CPU, in a throwaway module built from the
oracle's source text; the real oracle is left untouched.
"""
import importlib.util
import inspect
import types

import numpy as np
import pytest

import oracle.oracle as ORACLE
from tests import test_oracle_pins as pins

SRC = inspect.getsource(ORACLE)

MUTATIONS = [
    # (name, original text, planted text, pin tests expected to fail)
    ("window off by one", "return (d >= 0) & (d < int(window))",
     "return (d >= 0) & (d <= int(window))",
     ["test_sliding_window_printed_matrix"]),
    ("window drops causality", "return (d >= 0) & (d < int(window))",
     "return (d > -int(window)) & (d < int(window))",
     ["test_sliding_window_printed_matrix"]),
    ("strict causal", "        return i >= j\n",
     "        return i > j\n",
     ["test_sliding_window_special_cases"]),
    ("document ignores causality",
     "return (i >= j) & (doc[i] == doc[j])",
     "return (doc[i] == doc[j])",
     ["test_document_mask_block_diagonal_small"]),
    ("alibi sign", "return s - alibi_slope(h, H) * (i - j)",
     "return s + alibi_slope(h, H) * (i - j)",
     ["test_alibi_closed_form"]),
    ("alibi slope exponent", "return 2.0 ** (-8.0 * (h + 1) / H)",
     "return 2.0 ** (-8.0 * h / H)",
     ["test_alibi_closed_form"]),
    ("softcap inverted", "return softcap * np.tanh(s / softcap)",
     "return np.tanh(s * softcap) / softcap",
     ["test_softcap_closed_form"]),
    ("scale dropped", "s = scale * (q[b, h, ri] @ kb.T)",
     "s = (q[b, h, ri] @ kb.T)",
     ["test_sdpa_library_cross_check"]),
    ("operand transposed", "out[b, h, r0:r0 + len(ri)] = np.where(\n"
     "                    live[:, None], (w @ vb) / safe[:, None], 0.0)",
     "out[b, h, r0:r0 + len(ri)] = np.where(\n"
     "                    live[:, None], (w.T @ vb) / safe[:, None], 0.0)",
     ["test_sdpa_library_cross_check"]),
    ("log base", "mx + np.log(safe)", "mx + np.log10(safe)",
     ["test_rows_sum_to_one_and_uniform_weights"]),
    ("max not added back", "mx + np.log(safe)", "np.log(safe)",
     ["test_single_key_rows"]),
    ("unnormalised", "(w @ vb) / safe[:, None]", "(w @ vb)",
     ["test_rows_sum_to_one_and_uniform_weights"]),
    ("grouped heads interleaved", "kb = k[b, h // group]",
     "kb = k[b, h % H_kv]", ["test_attention_matches_brute_force"]),
    ("full threshold", "np.where(count == area, FULL, PARTIAL)",
     "np.where(count >= area // 2, FULL, PARTIAL)",
     ["test_block_counts_sliding_window_8k_seven_eighths_empty"]),
    ("ragged tile counted full", "padded = np.zeros((len(rows), nkvb * block_n), dtype=bool)",
     "padded = np.ones((len(rows), nkvb * block_n), dtype=bool)",
     ["test_block_mask_lists_are_permutations_and_partition"]),
    ("row chunk shifted", "ri = rows[r0:r0 + step]",
     "ri = rows[r0 + (r0 > 0):r0 + step + (r0 > 0)]",
     ["test_row_chunks_match_brute_force"]),
    ("row chunk skipped", "for r0 in range(0, len(rows), step):",
     "for r0 in range(0, len(rows), step + (step > 2)):",
     ["test_row_chunks_match_brute_force"]),
    ("index tail reversed",
     "idx[m] = np.concatenate([cols[selected[m]], cols[~selected[m]]])",
     "idx[m] = np.concatenate([cols[selected[m]], cols[~selected[m]][::-1]])",
     ["test_block_mask_matches_brute_force"]),
]


def _mutant(old, new):
    assert SRC.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(SRC.replace(old, new), "oracle_mutant", "exec"),
         mod.__dict__)
    return mod


def _run(test_name, monkeypatch):
    fn = getattr(pins, test_name)
    params = inspect.signature(fn).parameters
    # call with the first value of each parametrisation
    marks = {m.args[0]: m.args[1] for m in getattr(fn, "pytestmark", [])
             if m.name == "parametrize"}
    kwargs = {}
    for p in params:
        vals = marks[p]
        kwargs[p] = vals[0] if p != "mask" else "causal"
    fn(**kwargs)


@pytest.mark.parametrize("name,old,new,catchers", MUTATIONS,
                         ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, catchers, monkeypatch):
    mutant = _mutant(old, new)
    monkeypatch.setattr(pins, "O", mutant)
    for test_name in catchers:
        with pytest.raises(AssertionError):
            _run(test_name, monkeypatch)


def test_unmutated_copy_passes(monkeypatch):
    monkeypatch.setattr(pins, "O", _mutant("EMPTY, PARTIAL, FULL = 0, 1, 2",
                                           "EMPTY, PARTIAL, FULL = 0, 1, 2"))
    for _, _, _, catchers in MUTATIONS:
        for t in catchers:
            _run(t, monkeypatch)
