"""bench.py contract checks that need no GPU: the roofline picks the binding
roof of each workload, and more than one GPU is refused with a message."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

import bench
import workload as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _shape(cfg):
    """The sizes config_flops_bytes reads, without generating the cache (the
    ragged workload's lengths at their mean)."""
    c = wl.CONFIGS[cfg]
    L = c["seqlens"] if isinstance(c["seqlens"], int) else 4096
    max_blocks = c.get("max_blocks", (L + 63) // 64)
    return SimpleNamespace(B=c["B"], s_q=c["s_q"], H=c["H"], rows=c["B"] * c["s_q"] * c["H"],
                           seqlens=np.full(c["B"], L, dtype=np.int32), max_blocks=max_blocks,
                           kv_dtype=c.get("kv_dtype", "bf16"))


@pytest.mark.parametrize("cfg,bound", [(2, "hbm"), (3, "hbm"), (4, "mfma"), (5, "mfma")])
def test_roofline_takes_the_binding_roof(cfg, bound):
    # the roof whose ideal time is longer binds: bytes / 8 TB/s vs flops / 2.5 PF
    nbytes, flops, _ = wl.config_flops_bytes(_shape(cfg))
    r = bench.roofline(nbytes, flops, 1.0, None)
    assert r["bound"] == bound
    if bound == "hbm":
        assert r["unit"] == "GB/s" and r["peak"] == 8000.0
        assert r["achieved"] == pytest.approx(nbytes / 1e-3 / 1e9, rel=1e-4)
        assert r["frac"] == pytest.approx(r["achieved"] / 8000.0, abs=1e-4)
        assert r["mfma_frac"] == pytest.approx(flops / 1e-3 / 1e12 / 2500.0, abs=1e-4)
    else:
        assert r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
        assert r["achieved"] == pytest.approx(flops / 1e-3 / 1e12, rel=1e-4)
        assert r["hbm_frac"] == pytest.approx(nbytes / 1e-3 / 1e9 / 8000.0, abs=1e-4)


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
