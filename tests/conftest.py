"""Shared pytest configuration: the ``gpu`` marker and golden-file loading."""

import os
import sys
from fractions import Fraction

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def load_golden(name):
    """Parse ``key value...`` lines of a golden file; '#' starts a comment.
    Values that look like fractions become Fraction, others float/int."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            conv = []
            for v in vals:
                if "/" in v:
                    conv.append(Fraction(v))
                elif any(c in v for c in ".eE"):
                    conv.append(float(v))
                else:
                    conv.append(int(v))
            out[key] = conv if len(conv) > 1 else conv[0]
    return out
