"""bench.py's host-side legs, on the CPU: it refuses more than one GPU, and its CPU-oracle leg,
which also checks the output of the last timed GPU step, reports parity for a correct output and
fails one with a planted error (AG+GEMM bf16 and fp8 inputs, GEMM+RS D and send)."""
import os
import subprocess
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from oracle import ringag_oracle as O  # noqa: E402
from ring_all_gather_amd import workloads as W  # noqa: E402


def _bf16(x: np.ndarray) -> torch.Tensor:
    """fp32 values -> bf16 tensor (round to nearest even)."""
    return torch.from_numpy(O.f32_to_bf16(np.asarray(x, dtype=np.float32)).view(np.int16)).view(
        torch.bfloat16)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_ag_checks_the_timed_output():
    inp = W.make_ag(W.ag_shape(2, 1, 96, 128, 80, seed=5))
    _, D = O.ag_gemm(W.bits_u16(inp.A), [W.bits_u16(c) for c in inp.chunks])
    D_timed = _bf16(D)
    base, par = bench.cpu_baseline_ag(inp, 0.01, D_timed)
    assert base["kind"] == "oracle" and base["unit"] == "TFLOP/s" and base["value"] > 0
    assert base["cores"] >= 1
    assert par["ok"] and par["rows_checked"] == par["of_rows"] == 192
    assert par["max_rel_err"] <= 2 ** -8
    # a wrong row (the result of another row of the gathered input) must fail
    bad = D.copy()
    bad[37] = D[38]
    _, par = bench.cpu_baseline_ag(inp, 0.01, _bf16(bad))
    assert not par["ok"]


def test_cpu_baseline_ag_fp8_checks_the_timed_output():
    inp = W.make_ag(W.ag_shape(2, 0, 64, 128, 96, dtype="fp8", dist="normal", seed=6))
    _, D = O.ag_gemm_fp8(W.bits_u8(inp.A), inp.scale_A, [W.bits_u8(c) for c in inp.chunks],
                         inp.scale_B)
    base, par = bench.cpu_baseline_ag(inp, 0.01, _bf16(D))
    assert par["ok"] and par["tolerance"] == 5e-2
    bad = D.copy()
    bad[:, 5] = -bad[:, 5]
    _, par = bench.cpu_baseline_ag(inp, 0.01, _bf16(bad))
    assert not par["ok"]


def test_cpu_baseline_rs_checks_d_and_send():
    shape = W.rs_shape(4, 2, 4 * 32, 128, 96, seed=9)
    inp = W.make_rs(shape)
    peers = [None if p is None else p.numpy() for p in inp.partials]
    D, send, _ = O.gemm_rs(W.bits_u16(inp.X), W.bits_u16(inp.W), peers, shape.tp,
                           shape.self_rank)
    send_t = torch.from_numpy(np.ascontiguousarray(send, dtype=np.float32))
    base, par = bench.cpu_baseline_rs(inp, 0.01, _bf16(D), send_t)
    assert base["kind"] == "oracle" and base["value"] > 0
    assert par["ok"] and par["rows_checked"] == par["of_rows"] == shape.T
    assert par["D_rows_checked"] == shape.nc
    assert par["max_rel_err_send"] <= 1e-6
    # a wrong outgoing chunk (another chunk's rows) and a wrong reduced row must each fail
    bad_send = send_t.clone()
    bad_send[0] = send_t[1]
    _, par = bench.cpu_baseline_rs(inp, 0.01, _bf16(D), bad_send)
    assert not par["ok"]
    bad_D = D.copy()
    bad_D[3] += np.abs(D).max()
    _, par = bench.cpu_baseline_rs(inp, 0.01, _bf16(bad_D), send_t)
    assert not par["ok"]
