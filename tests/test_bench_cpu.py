"""Host-side checks of bench.py's accounting (no GPU): the algorithmic bytes of the prefill and how the
path-level roofline splits them over the five kernels."""
import os

import bench

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_algorithmic_bytes_of_the_64k_workload():
    # 1,796 B per token-head over 65,536 x 16 token-heads, plus S0 and S_final (64 KiB per head each)
    assert bench.alg_bytes(65536 * 16, 16) == 1796 * 1048576 + 2 * 65536 * 16 == 1885339648
    assert bench.BYTES_PER_TOKEN_HEAD == 3 * 256 + 512 + 4 + 512
    assert bench.FLOPS_PER_TOKEN_HEAD == 126976


def test_per_kernel_split_adds_up_to_the_path():
    stage = {n: 0.1 * (i + 1) for i, n in enumerate(bench.STAGES)}
    r = bench.roofline(1.0, stage, 65536 * 16, 16, {})
    assert sum(k["algorithmic_bytes"] for k in r["per_kernel"].values()) == r["algorithmic_bytes_per_launch"]
    assert abs(r["frac"] - 1885339648 / 1e-3 / 8e12) < 1e-12
    assert r["traffic"] is None
    tr = {n: 1e9 for n in bench.STAGES}
    assert bench.roofline(1.0, stage, 16, 1, tr)["traffic"] == 5e9


def test_flop_figure_follows_the_pages_formula():
    """The TFLOP/s bench.py reports counts the FLOP formula of the Kimi Linear summary, section 6.3
    (6 T d^2 + 3 T C d + T C^2 per head), whose values at d = 128, C = 64 are in the golden file."""
    for line in open(os.path.join(GOLDEN, "flops_formula.txt")):
        if line.startswith("#") or not line.strip():
            continue
        T, d, C, f = (int(x) for x in line.split())
        assert d == 128 and C == 64 and bench.FLOPS_PER_TOKEN_HEAD * T == f
