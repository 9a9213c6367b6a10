"""Mutation check of the oracle's pins (CPU only).

Each mutant is a copy of the oracle's source with one plausible slip planted
in it: a block mask off by one, a dropped softmax scale, a wrong head or page
mapping, the wrong end of a tie, a swapped acceptance test, a residual of the
wrong sign, a shifted cache slot, a skipped prompt row.  The copy is compiled
as a separate module; the pins of test_oracle_pins.py then run against it and
at least one must fail.  The oracle file itself is never changed, and the
unmutated copy must pass every pin, which checks the harness.
"""

import importlib.util
import itertools
import os
import types

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
with open(os.path.join(ROOT, "oracle", "orthrus_oracle.py")) as fh:
    SOURCE = fh.read()

# name -> (text in the oracle, replacement); each text occurs exactly once
MUTANTS = {
    "ar_mask_sees_the_next_row": ("blk = list(range(i + 1))", "blk = list(range(min(i + 2, K)))"),
    "diff_mask_drops_the_last_key": ("blk = list(range(K))", "blk = list(range(K - 1)) if i != K - 1 else list(range(K))"),
    "softmax_scale_dropped": ("scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)\n"
                              "    out = np.full((B, K, Hq, D), np.nan)",
                              "scale = 1.0 if softmax_scale is None else float(softmax_scale)\n"
                              "    out = np.full((B, K, Hq, D), np.nan)"),
    "gqa_head_interleaved": ("g = h * Hkv // Hq\n            if g not in ctx:", "g = h % Hkv\n            if g not in ctx:"),
    "pages_in_reverse": ("pages = _i64(page_table_row)[:n_pages]", "pages = _i64(page_table_row)[:n_pages][::-1]"),
    "argmax_ties_to_highest": ("g[r] = np.flatnonzero(flat[r] == m)[0]", "g[r] = np.flatnonzero(flat[r] == m)[-1]"),
    "accept_counts_past_a_mismatch": ("        if int(d) != int(t):\n            break\n        a += 1",
                                      "        if int(d) != int(t):\n            continue\n        a += 1"),
    "next_token_one_row_early": ("nxt = np.array([g[b, min(acc[b], K - 1)] for b in range(B)], dtype=np.int64)",
                                 "nxt = np.array([g[b, max(acc[b] - 1, 0)] for b in range(B)], dtype=np.int64)"),
    "commit_without_correction": ("return min(int(accept_len) + 1, K)", "return min(int(accept_len), K)"),
    "append_slot_shifted": ("            slot = pos % page_size\n", "            slot = (pos + 1) % page_size\n"),
    "sample_accept_test_swapped": ("ua[b, i] * q[x] < p[x]", "ua[b, i] * p[x] < q[x]"),
    "sample_residual_sign": ("r = np.maximum(p - q, 0.0)", "r = np.maximum(q - p, 0.0)"),
    "sample_cdf_target_unscaled": ("np.flatnonzero(c > ur[b] * total)[0]", "np.flatnonzero(c > ur[b])[0]"),
    "temperature_ignored": ("x = _f64(logits) / float(temperature)", "x = _f64(logits)"),
    "lm_head_weight_rows_shifted": ("return h @ w.T", "return h @ np.roll(w, 1, axis=0).T"),
    "confidence_without_max_shift": ("return greedy_argmax(x), 1.0 / np.exp(x - m).sum(axis=-1)",
                                     "return greedy_argmax(x), 1.0 / np.exp(x).sum(axis=-1)"),
    "denoise_unmasks_least_confident": ("key=lambda i: (-c[b, i], i)", "key=lambda i: (c[b, i], i)"),
    "denoise_ties_to_higher_row": ("key=lambda i: (-c[b, i], i)", "key=lambda i: (-c[b, i], -i)"),
    "prefill_sees_the_next_row": ("s = scale * (keys[:L + i + 1] @ q[b, i, h])\n"
                                  "                w = np.exp(s - s.max())\n"
                                  "                out[b, i, h] = (w @ vals[:L + i + 1]) / w.sum()",
                                  "s = scale * (keys[:L + i + 2] @ q[b, i, h])\n"
                                  "                w = np.exp(s - s.max())\n"
                                  "                out[b, i, h] = (w @ vals[:L + i + 2]) / w.sum()"),
    "prompt_write_slot_shifted": ("            kc[page, :, pos % page_size, :] = kr[b, r]\n"
                                  "            vc[page, :, pos % page_size, :] = vr[b, r]",
                                  "            kc[page, :, (pos + 1) % page_size, :] = kr[b, r]\n"
                                  "            vc[page, :, (pos + 1) % page_size, :] = vr[b, r]"),
    "prefill_gqa_head_interleaved": ("g = h * Hkv // Hq\n            keys = np.concatenate",
                                     "g = h % Hkv\n            keys = np.concatenate"),
    "prefill_scale_dropped": ("scale = 1.0 / np.sqrt(D) if softmax_scale is None else float(softmax_scale)\n"
                              "    out = np.full((B, S, Hq, D), np.nan)",
                              "scale = 1.0 if softmax_scale is None else float(softmax_scale)\n"
                              "    out = np.full((B, S, Hq, D), np.nan)"),
    "accept_compare_inverted": ("        if int(d) != int(t):\n            break", "        if int(d) == int(t):\n            break"),
    "sample_accept_len_one_late": ("            acc[b] = i\n", "            acc[b] = i + 1\n"),
    "softmax_t_unnormalised": ("    return e / np.sum(e, axis=-1, keepdims=True)", "    return e"),
    "denoise_unmasks_one_too_few": ("for i in order[:max(int(n[b]), 0)]:", "for i in order[:max(int(n[b]) - 1, 0)]:"),
    "lm_head_hidden_reversed": ("return h @ w.T", "return h[..., ::-1] @ w.T"),
    "prompt_write_skips_row_0": ("        for r in range(int(n[b])):\n            pos = L + r",
                                 "        for r in range(1, int(n[b])):\n            pos = L + r"),
}


def oracle_module(source):
    mod = types.ModuleType("orthrus_oracle_variant")
    mod.__file__ = os.path.join(ROOT, "oracle", "orthrus_oracle.py")
    exec(compile(source, "orthrus_oracle_variant.py", "exec"), mod.__dict__)
    return mod


def pin_cases():
    """(name, function, kwargs) of every pin, parametrized cases expanded."""
    spec = importlib.util.spec_from_file_location("oracle_pins_for_mutants", os.path.join(HERE, "test_oracle_pins.py"))
    pins = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(pins)
    cases = []
    for name in dir(pins):
        fn = getattr(pins, name)
        if not (name.startswith("test_") and callable(fn)):
            continue
        grids = []
        for mark in getattr(fn, "pytestmark", []):
            if mark.name != "parametrize":
                continue
            names = [n.strip() for n in mark.args[0].split(",")]
            grids.append([dict(zip(names, v if len(names) > 1 else (v,))) for v in mark.args[1]])
        for combo in itertools.product(*grids):
            kw = {}
            for part in combo:
                kw.update(part)
            cases.append((name, fn, kw))
    return pins, cases


def failing_pin(source):
    """The first pin that fails with the oracle built from `source`, or None."""
    pins, cases = pin_cases()
    pins.O = oracle_module(source)
    for name, fn, kw in cases:
        try:
            fn(**kw)
        except Exception as e:  # an assertion, or a crash the slip causes
            return f"{name}{kw or ''}: {type(e).__name__}"
    return None


def test_unmutated_oracle_passes_every_pin():
    assert failing_pin(SOURCE) is None


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_fails_a_pin(mutant):
    old, new = MUTANTS[mutant]
    assert SOURCE.count(old) == 1, f"the text of {mutant} must occur once in the oracle"
    assert failing_pin(SOURCE.replace(old, new)) is not None, f"no pin catches {mutant}"
