"""The oracle's results on the seeded tiny fp32 workload equal the stored
fixture (tests/golden/tiny_fp32_oracle.txt, written by
tests/golden/make_oracle_golden.py from the oracle alone): integers
exactly, floating-point summaries to 1e-9 relative (host BLAS summation
order may differ between machines).  A change to the oracle's arithmetic
shows up here and must be justified by the pages."""

import importlib.util
import os

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def load_script():
    spec = importlib.util.spec_from_file_location("make_oracle_golden",
                                                  os.path.join(HERE, "golden", "make_oracle_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def stored():
    out = {}
    for line in open(os.path.join(HERE, "golden", "tiny_fp32_oracle.txt")):
        if line.strip() and not line.startswith("#"):
            k, v = line.split("=", 1)
            out[k.strip()] = v.strip()
    return out


def test_oracle_matches_stored_tiny_results():
    now = load_script().summarise()
    ref = stored()
    assert set(now) == set(ref)
    for k, v in ref.items():
        a, b = v.split(), now[k].split()
        assert len(a) == len(b), k
        for x, y in zip(a, b):
            if "e" in x or "." in x:
                assert float(y) == pytest.approx(float(x), rel=1e-9, abs=1e-12), k
            else:
                assert int(y) == int(x), k
