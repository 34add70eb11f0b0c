import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def pytest_collection_modifyitems(config, items):
    """GPU tests need a visible device; on a CPU-only machine they are skipped
    (they are selected with -m gpu on the GPU machine)."""
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def parse_packed_blocks():
    """Rows of tests/golden/packed_blocks.txt as (bits, codes, words)."""
    out = []
    with open(os.path.join(GOLDEN, "packed_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split("|")]
            bits = int(parts[0].split()[1])
            codes = []
            for tok in parts[1].split()[1:]:
                if ".." in tok:
                    a, b = tok.split("..")
                    codes.extend(range(int(a), int(b) + 1))
                else:
                    codes.append(int(tok))
            codes += [0] * (32 - len(codes))
            words = [int(w, 16) for w in parts[2].split()[1:]]
            out.append((bits, codes, words))
    return out
