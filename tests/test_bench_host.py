"""Host-side checks of bench.py: the algorithmic cost model behind its roofline
fractions, counted entry by entry on small shapes, and the one-GPU contract."""
import importlib.util
import os
import subprocess
import sys
from types import SimpleNamespace

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_cost_model_counts_entries():
    """Covariance flops: 2 per multiply-add, over the entries each output
    keeps (lower triangles of H_X and H_G with their diagonals, all of D);
    BiIP bytes: a read and a write of fp32 per element and single-side pass
    (two per matrix) over W, H_X, D, H_G, plus one read of W for its norms."""
    b = _bench()
    for m, n, N in ((3, 5, 7), (8, 4, 2), (16, 16, 10)):
        c = b.stage_costs(SimpleNamespace(d_out=m, d_in=n, n_tok=N))
        lower = lambda d: sum(1 for i in range(d) for j in range(d) if j <= i)
        assert c["cov_flops"] == 2 * N * (lower(n) + n * n + lower(m))
        passes = 2
        assert c["biip_bytes"] == passes * 8 * (m * n + n * n + n * n + m * m) + 4 * m * n
        assert c["biip_min_bytes"] == 8 * (m * n + n * n + n * n + m * m)


def test_cost_model_at_the_bench_layer():
    b = _bench()
    c = b.stage_costs(SimpleNamespace(d_out=4096, d_in=4096, n_tok=131072))
    assert abs(c["cov_flops"] / 8.797e12 - 1) < 1e-3
    assert abs(c["biip_bytes"] / 1.141e9 - 1) < 1e-3
    assert abs(c["chol_flops"] / 4.58e10 - 1) < 1e-3
    assert abs(c["solve_flops"] / 1.832e11 - 1) < 1e-3


def test_cost_model_at_the_down_proj_layer():
    """W 8192 x 28672, 131072 tokens: S1 = n(n+1)N + 2n^2 N + m(m+1)N, the
    factorization and P 2n^3/3 each, the trailing updates 2 m n^2, BiIP two
    single-side passes over W, H_X, D and H_G (31.1 GB) plus the norm read of
    W (0.94 GB), against a read-once floor of 15.6 GB."""
    b = _bench()
    c = b.stage_costs(SimpleNamespace(d_out=8192, d_in=28672, n_tok=131072))
    assert abs(c["cov_flops"] / 3.3206e14 - 1) < 1e-4
    assert abs(c["chol_flops"] / 1.5714e13 - 1) < 1e-4
    assert abs(c["solve_flops"] / (1.5714e13 + 1.3469e13) - 1) < 1e-4
    assert abs((c["biip_bytes"] - 4 * 8192 * 28672) / 31.14e9 - 1) < 1e-3
    assert abs(c["biip_min_bytes"] / 15.57e9 - 1) < 1e-3


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "--gpus 1" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a run that did not happen
