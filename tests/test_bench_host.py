"""Host-side checks of the measurement script (CPU only).

The algorithmic bytes that ``bench.py`` divides by a kernel's duration are
pinned to the figures the pages' formats give: one index of `bits` bits per
weight plus one fp16 norm per 128-wide group ([Needle W4A8] section 1), i.e.
0.140625 / 0.265625 / 0.390625 / 0.515625 bytes per weight at 1 / 2 / 3 / 4
bits.  The one-GPU rule is checked without touching a device.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

BENCH = os.path.join(ROOT, "bench.py")


def _run_bench(args, extra_env=None):
    env = dict(os.environ)
    env.update(extra_env or {})
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, env=env,
                          timeout=120)


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], None), (["--gpus", "8"], None),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(args, env):
    r = _run_bench(args, env)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""                          # no JSON line is printed


@pytest.fixture(scope="module")
def bench_mod():
    from bit_quantized_matmul_amd import binding
    if not os.path.exists(binding.library_path()):
        pytest.fail("libbqm.so is not built (run python -m bit_quantized_matmul_amd.build)")
    binding.load_library()
    sys.path.insert(0, ROOT)
    import bench
    return bench


# weight bytes (indices + fp16 norms) of the 14336 x 4096 sweep matrix per
# index width: rows * cols * (bits / 8 + 2 / 128)
SWEEP_BYTES = {1: 8_257_536, 2: 15_597_568, 3: 22_937_600, 4: 30_277_632, 5: 15_597_568}


@pytest.mark.parametrize("bits", sorted(SWEEP_BYTES))
def test_payload_bytes_match_the_format(bench_mod, bits):
    from bit_quantized_matmul_amd import binding
    lay = binding.cq_pack_info(14336, 4096, 128, bits)
    assert bench_mod.payload_bytes(lay) == SWEEP_BYTES[bits]
    ib = 2 if bits == 5 else bits
    assert SWEEP_BYTES[bits] == 14336 * 4096 * ib // 8 + 2 * 14336 * 4096 // 128


def test_dominant_and_step_bytes(bench_mod):
    """The roofline's bytes for the 4096x14336 launch (weights + fp32 x + fp32
    y) and the decode step's weight bytes (the four layer shapes)."""
    from bit_quantized_matmul_amd import binding
    lay = binding.cq_pack_info(4096, 14336, 128, 4)
    assert bench_mod.payload_bytes(lay) + 14336 * 4 + 4096 * 4 == 30_351_360
    shapes = [(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)]
    step = sum(bench_mod.payload_bytes(binding.cq_pack_info(r, c, 128, 4)) for r, c in shapes)
    assert step == 71_368_704


def test_cold_pool_size_covers_the_infinity_cache(bench_mod):
    """Each HBM-cold measurement cycles >= 1 GiB of copies (the 256 MB
    Infinity Cache cannot hold them between uses)."""
    for nbytes in (135_168, 2_162_688, 30_277_632, 71_368_704):
        assert bench_mod.pool_copies(nbytes) * nbytes >= 1 << 30
    assert bench_mod.pool_copies(1 << 31) == 2
