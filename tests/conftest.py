"""Shared test configuration.

Markers: ``gpu`` tests need an MI355X (gfx950) and the built HIP library;
everything else runs on the CPU.  GPU tests are skipped cleanly when no GPU
is visible.
"""
from __future__ import annotations

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available() and torch.cuda.device_count() > 0
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def golden_path(name: str) -> str:
    return os.path.join(GOLDEN, name)


def read_golden_rows(name: str):
    """Non-comment, non-empty lines of a golden file, split on '|'."""
    rows = []
    with open(golden_path(name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([part.strip() for part in line.split("|")])
    return rows


@pytest.fixture(scope="session")
def gaussian400k():
    from bit_quantized_matmul_amd import inputs
    return inputs.gaussian_samples()


@pytest.fixture(scope="session")
def raw_fits(gaussian400k):
    """Unrounded oracle Lloyd-Max fits keyed by bits (seed 0, 400k, 200 it)."""
    from oracle import codebook
    return {b: codebook.lloyd_max_fit(gaussian400k, n) for b, n in codebook.CODEBOOK_LEVELS.items()}


@pytest.fixture(scope="session")
def codebooks(raw_fits):
    """Shipped cb2/cb3/cb4 tables (bf16-rounded oracle fits)."""
    from oracle import codebook
    return {b: codebook.shipped_table(r) for b, r in raw_fits.items()}


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the element-wise parity statistics the GPU tests recorded."""
    try:
        from tests import parity
    except Exception:
        return
    for line in parity.summary_lines():
        terminalreporter.write_line(line)
