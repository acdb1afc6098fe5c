"""Host logic of bench.py (no GPU): the flop accounting behind the reported
rates, the refusal of a multi-GPU request, and the amd-smi sample parser."""
import itertools
import json
import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _count_products(rows, cols, c_nonzero):
    """Multiply-adds of one Newton-Schulz step, counted entry by entry: the
    symmetric products (GRAM X X^T, POLY A A) once per unique entry, COMBINE
    (B X) for every entry; two flops each."""
    m, n = min(rows, cols), max(rows, cols)
    gram = sum(n for i, j in itertools.product(range(m), range(m)) if i <= j)
    poly = sum(m for i, j in itertools.product(range(m), range(m)) if i <= j) if c_nonzero else 0
    comb = sum(m for _ in itertools.product(range(m), range(n)))
    return 2 * gram, 2 * poly, 2 * comb


@pytest.mark.parametrize("shape", [(1, 1), (2, 3), (5, 2), (4, 4), (3, 7)])
@pytest.mark.parametrize("c_nonzero", [True, False])
def test_algorithmic_flops_count_unique_entries(shape, c_nonzero):
    steps = 3
    nominal, alg = bench.ns_flops([shape], steps, c_nonzero)
    g, p, c = _count_products(*shape, c_nonzero)
    assert alg["gram"] == steps * g
    assert alg["poly"] == steps * p
    assert alg["combine"] == steps * c
    m, n = min(shape), max(shape)
    # nominal: both halves of every product (X X^T: 2 m^2 n, A A: 2 m^3, B X: 2 m^2 n)
    assert nominal == steps * (2 * m * m * n + (2 * m ** 3 if c_nonzero else 0) + 2 * m * m * n)


def test_d24_step_counts():
    # 24 layers x {Q, K, V, O 1536^2, up 1536 x 6144, down 6144 x 1536}, 5 quintic steps
    shapes = [(1536, 1536)] * 4 * 24 + [(1536, 6144), (6144, 1536)] * 24
    nominal, alg = bench.ns_flops(shapes, 5, True)
    assert nominal == pytest.approx(26.0919263232e12, rel=1e-12)
    assert sum(alg.values()) == pytest.approx(18.2694445056e12, rel=1e-12)
    # per COMBINE launch: 2 m^2 n over the stack
    assert alg["combine"] / 5 == pytest.approx(2.087e12, rel=1e-3)


def test_more_than_one_gpu_is_refused():
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_amd_smi_sample_parser():
    sample = [{"gpu": 0,
               "power": {"socket_power": {"value": 1357, "unit": "W"}, "gfx_voltage": {"value": 800, "unit": "mV"}},
               "clock": {"gfx_0": {"clk": {"value": 1860, "unit": "MHz"}},
                         "gfx_1": {"clk": {"value": 1880, "unit": "MHz"}},
                         "gfx_2": {"clk": {"value": "N/A", "unit": "MHz"}},
                         "mem_0": {"clk": {"value": 2000, "unit": "MHz"}}}}]
    pw, clk = bench.parse_amd_smi_metric(json.dumps(sample))
    assert pw == 1357.0
    assert clk == 1870.0
    wrapped = {"gpu_data": [{"power": {"socket_power": 1100}, "clock": {"gfx_0": {"clk": {"value": 2400}}}}]}
    assert bench.parse_amd_smi_metric(json.dumps(wrapped)) == (1100.0, 2400.0)
