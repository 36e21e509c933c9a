import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running exhaustive check")


def parse_num(tok: str) -> float:
    """Python float literal, hex float or 0b... integer."""
    tok = tok.strip()
    if tok.startswith("0b"):
        return float(int(tok, 2))
    try:
        return float(tok)
    except ValueError:
        return float.fromhex(tok)


def read_golden(name: str):
    """Non-comment lines of tests/golden/<name>, split on whitespace."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.split())
    return rows


def read_golden_kv(name: str):
    """{test: {key: value-string}} for key=value fixture files."""
    out = {}
    for row in read_golden(name):
        out[row[0]] = dict(tok.split("=", 1) for tok in row[1:])
    return out


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle as o
    o.lib()
    return o


@pytest.fixture(scope="session")
def fqlib():
    """The HIP binding, on a machine with a GPU (the GPU tests skip elsewhere)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from fake_quant_amd import fq
    return fq


def log(msg):
    """Flushed progress line naming the case about to run on the GPU."""
    print(msg, flush=True)
