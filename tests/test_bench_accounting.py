"""The benchmark's algorithmic-work accounting against the pages' cost model.

bench.py reports each kernel's roofline as algorithmic work per launch over
the launch's measured duration; the work comes from bench.kernel_work.  Here
its Newton-Schulz FLOP totals are checked against two things that do not
come from bench.py: the closed-form cost the pages print ("Dion3: Full-Stack
Orthogonal Updates", Section 4: (4T + 3 alpha - 3) n^3 for Gram NS without
restart, plus 3 (alpha - 1) n^3 per restart; Section 2: standard NS), read
from tests/golden/flop_claims.txt, and the oracle's instrumented tally of the
same products (itself pinned to the pages in test_oracle.py).

kernel_work counts a symmetric k x k product by its lower triangle,
k (k + 1) / 2 entries, where the pages count k^2 / 2; the symmetric classes
are rescaled by k / (k + 1) before comparing, so the comparison is exact.
"""

import importlib.util
import math
import os

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")
SYM = ("syrk", "sym_sq_add", "sym_mul")
RECT = ("gemm_qx", "qx_apply")


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)       # defines functions only; main() is not run
    return mod


def _golden():
    rows = {}
    with open(os.path.join(GOLDEN, "flop_claims.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].split()
            if len(line) == 4:
                rows[line[0]] = float(line[3])
    return rows


def _pages_count(work, k):
    """kernel_work's FLOPs per class in the pages' counting (symmetric
    products at k^2 / 2 entries)."""
    out = {}
    for name in SYM + RECT:
        v = work[name][1]
        out[name] = v * k / (k + 1) if name in SYM else v
    return out


@pytest.mark.parametrize("k,m", [(16, 64), (256, 1024), (1024, 4096), (1024, 2752), (512, 512 * 3)])
def test_gram_ns_flops_match_closed_form(bench, k, m):
    g = _golden()
    T, b = 5, 3
    alpha = m / k
    work = _pages_count(bench.kernel_work([(2 * k, m, b)], [k]), k)   # k of 2k <= m rows: not square
    total = sum(work.values())
    per = (g["gram_coeff_T"] * T + g["gram_coeff_alpha"] * alpha + g["gram_coeff_const"]
           + g["restart_extra_coeff_alpha"] * alpha + g["restart_extra_coeff_const"]) * k ** 3
    assert math.isclose(total, b * per, rel_tol=1e-12), (total, b * per)


@pytest.mark.parametrize("k,m", [(16, 64), (16, 48), (32, 32 * 5)])
def test_gram_ns_flops_match_oracle_tally(bench, k, m):
    """Class by class: X X^T (syrk) against the oracle's gram products, the
    k x k products (sym_sq_add + sym_mul) against its square ones, Q X
    against its rectangular ones, for T = 5 with the restart after 2."""
    rng = np.random.default_rng(7)
    X = rng.standard_normal((k, m))
    tally = {}
    O.ns_gram(X, restart_after=(2,), flops=tally)
    work = _pages_count(bench.kernel_work([(2 * k, m, 1)], [k]), k)
    assert math.isclose(work["syrk"], tally["gram"], rel_tol=1e-12)
    assert math.isclose(work["sym_sq_add"] + work["sym_mul"], tally["square"], rel_tol=1e-12)
    assert math.isclose(work["gemm_qx"] + work["qx_apply"], tally["rect"], rel_tol=1e-12)


@pytest.mark.parametrize("n", [16, 256, 4096])
def test_square_class_uses_standard_ns_cost(bench, n):
    """A square selection (k = n = m) runs standard Newton-Schulz: its total
    is the pages' symmetric standard-NS cost T (m n^2 + n^3 + 2 m n^2)."""
    work = _pages_count(bench.kernel_work([(n, n, 2)], [n]), n)
    assert math.isclose(sum(work.values()), 2 * O.ns_standard_flops(n, n, 5, symmetric=True), rel_tol=1e-12)
    assert math.isclose(work["syrk"], 2 * 5 * n ** 3, rel_tol=1e-12)


def test_fused_group_moves_last_product_and_drops_update(bench):
    """A group whose update runs in the last Q X epilogue: the same FLOPs, the
    last product under qx_apply, and no separate update pass."""
    k, m, b = 1024, 4096, 4
    assert bench.fuses_update(2 * k, m, b, k, "muon")
    assert not bench.fuses_update(2 * k, m, b, k, "normuon")
    fused = bench.kernel_work([(2 * k, m, b)], [k], flavor="muon")
    plain = bench.kernel_work([(2 * k, m, b)], [k], flavor="normuon")
    assert fused["apply_update"][1] == 0 and plain["apply_update"][1] == b * k * m * 6
    assert fused["qx_apply"][1] == b * 2 * k * k * m and plain["qx_apply"][1] == 0
    assert fused["gemm_qx"][1] + fused["qx_apply"][1] == plain["gemm_qx"][1]
    # a column-selected group (rows > cols) never fuses
    assert not bench.fuses_update(m, 2 * k, b, k, "muon")


def test_7b_momentum_bytes(bench):
    """The momentum pass moves M, G in and M out once per parameter: 6 bytes
    per bf16 parameter over the 7B shape set's 6,476,005,376 parameters."""
    from muon_momentum_amd import synth
    groups = synth.shape_groups("7b")
    params = sum(r * c * b for r, c, b in groups)
    assert params == 32 * (4 * 4096 * 4096 + 2 * 4096 * 11008 + 11008 * 4096) == 6476005376
    ks = [math.ceil(min(r, c) / 4) for r, c, _ in groups]
    work = bench.kernel_work(groups, ks)
    assert work["momentum_keys"] == ("hbm", 6 * params)


def test_traffic_lookup_follows_the_source(bench, tmp_path, monkeypatch):
    """bench.py reports a kernel's counter-measured HBM bytes only while the
    kernel's source (and common.h) hash equals the one recorded beside the
    counters, and only for the workload they were taken on."""
    import hashlib
    h = hashlib.sha256()
    for name in ("rowsel.hip", "common.h"):
        with open(os.path.join(ROOT, "muon_momentum_amd", "csrc", name), "rb") as fh:
            h.update(fh.read())
    good = h.hexdigest()[:16]
    f = tmp_path / "traffic.txt"
    f.write_text("# header\n"
                 f"traffic kernel=momentum_keys launches=2 fetch_bytes=1e9 write_bytes=5e8 total_bytes=1.5e9 "
                 f"source=rowsel.hip src_sha256={good}\n"
                 "traffic kernel=topk_select launches=2 fetch_bytes=1 write_bytes=1 total_bytes=2 "
                 "source=rowsel.hip src_sha256=0000000000000000\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("momentum_keys", "7b", 0.25) == 1.5e9
    assert bench.measured_traffic("topk_select", "7b", 0.25) is None        # stale hash
    assert bench.measured_traffic("momentum_keys", "1b", 0.125) is None     # another workload
    assert bench.measured_traffic("gemm_qx", "7b", 0.25) is None            # no line


def test_bench_refuses_more_than_one_gpu():
    """The benchmark has no multi-GPU path: --gpus above 1 exits with a
    message, before touching a GPU."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
