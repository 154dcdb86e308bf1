"""Host logic of bench.py that needs no GPU: the one-GPU guard, the algorithmic work that
the roofline entry divides by, and the rule that a committed HBM-traffic figure is used
only while the kernel sources it was measured on are unchanged."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixture_experts_layer_stable_amd import inputs  # noqa: E402


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_gemm_flops_of_the_kimi_k2_step():
    """Per launch: FC1 and dX 4*R*H*I, FC2, dH, dW2 2*R*H*I, dW1 4*R*H*I (R = T*k)."""
    w = inputs.WORKLOADS["kimi_k2_bf16"]
    R, H, I = w.T * w.k, w.H, w.I
    want = {"fc1": 4, "fc2": 2, "dh": 2, "dx": 4, "dw2": 2, "dw1": 4}
    for name, m in want.items():
        bound, work = bench.kernel_work(w, name)
        assert bound == "mfma"
        assert work == m * R * H * I
        assert bench.launches_per_step(w, name) == 1
    total = sum(bench.launch_flops(w, n) for n in want)
    assert abs(total - 34.64e12) < 0.01e12  # 34.6 TFLOP of expert GEMMs per step


def test_streamed_mxfp8_launches_and_weight_bytes():
    """Row GEMMs run once per micro-batch on R/M rows; the weight gradients once per step
    over all rows. An MXFP8 row GEMM is priced by its weight stream: 33/32 bytes per
    element of every active expert's panel (plus activation rows) when that exceeds the
    flops at 5 PFLOP/s."""
    w = inputs.WORKLOADS["kimi_k2_mxfp8_stream"]
    M = w.micro_batches
    R, H, I = (w.T // M) * w.k, w.H, w.I
    assert bench.launches_per_step(w, "fc1") == M and bench.launches_per_step(w, "dw1") == 1
    assert bench.launch_flops(w, "fc1") == 4 * R * H * I
    assert bench.launch_flops(w, "dw1") == 4 * M * R * H * I
    bound, b = bench.kernel_work(w, "fc1", active_experts=100)
    assert bound == "hbm"
    weights = 2 * I * H * 33 / 32 * 100
    assert weights < b < weights + 1.0e9  # plus the token rows of one micro-batch
    bound, b2 = bench.kernel_work(w, "fc1", active_experts=200)
    assert b2 - b == pytest.approx(weights)


def test_traffic_figure_only_for_the_measured_sources(tmp_path, monkeypatch):
    csrc = tmp_path / "mixture_experts_layer_stable_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text("// kernel v1\n")
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.source_hash()
    (tmp_path / "profiles" / "traffic_dw1_demo.md").write_text(
        "# demo\n\n<!-- source_hash = %s -->\n<!-- hbm_bytes_per_launch = 5.2e+10 -->\n" % h)
    assert bench.measured_traffic("dw1", "demo") == 5.2e10
    assert bench.measured_traffic("dw2", "demo") is None  # no summary for that kernel
    (csrc / "k.hip").write_text("// kernel v2\n")
    assert bench.measured_traffic("dw1", "demo") is None  # sources changed since the counters


def test_bandwidth_kernels_count_compulsory_bytes():
    """The elementwise kernels' algorithmic bytes at the Kimi-K2 shape (bf16, R = T*k routed
    rows): combine reads the R partial rows and writes the T output rows; dX reduce does the
    same plus the router-weight matrix once (each slot's Wr row comes from cache) and the
    dz/idx words; dWr reads the routed x rows and also writes them in routed order for dW1;
    the dO gather reads the routed dY rows and writes g*dY in routed order."""
    w = inputs.WORKLOADS["kimi_k2_bf16"]
    T, R, H, E = w.T, w.T * w.k, w.H, w.E
    assert bench.kernel_work(w, "combine") == ("hbm", 2 * R * H + 2 * T * H + 4 * R)
    assert bench.kernel_work(w, "dx_reduce") == ("hbm", 2 * R * H + 2 * T * H + 8 * R + 2 * E * H)
    assert bench.kernel_work(w, "dwr") == ("hbm", 2 * R * H + 2 * E * H + 8 * R + 2 * R * H)
    assert bench.kernel_work(w, "gather") == ("hbm", 4 * R * H + 8 * R)
