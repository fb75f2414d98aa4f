"""Host-side checks of bench.py: the one-GPU guard, the algorithmic work it prices the
rooflines with, and when it trusts a recorded HBM-traffic summary."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

import synth_inputs as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_kernel_work_matches_the_block_totals():
    wl = S.WORKLOADS["block_l16384"]
    d, F, L = wl.d, wl.d_ff, wl.L
    w = bench.kernel_work(wl, L)
    gemm = sum(w[k][1] for k in ("gemm_qkv", "gemm_o", "gemm_up", "gemm_down"))
    assert gemm == 24.0 * d * d * L  # 2 (3d + d + F + F) d L with F = 4d: 10.31 TOP
    assert abs(gemm - 10.31e12) < 0.01e12
    assert w["attention"][1] == 4.0 * L * L * d  # QK^T and PV, 2 flops per multiply-add
    assert abs(w["attention"][1] - 5.498e12) < 0.001e12
    assert all(w[k][2] == "int8" for k in ("gemm_qkv", "gemm_o", "gemm_up", "gemm_down"))
    assert w["attention"][2] == "fp16"
    # bandwidth-bound kernels: bytes read once and written once
    assert w["ln_quant"][1] == L * (2 * d + d + 4)
    assert w["rowquant_g"][1] == L * (2 * F + F + 4)
    assert w["adaln"][1] == 6 * d * wl.d_cond * 2


def _summary(tmp_path, src_hash):
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps({
        "workload": "block_l16384",
        "sources": {"k_attn.hip": src_hash},
        "kernels": {"attn_v2_kernel<true>": {"kind": "attention", "source": "k_attn.hip",
                                             "read_bytes": 1000.4, "write_bytes": 200.2}},
    }))
    return str(path)


def test_traffic_used_only_for_the_source_it_was_measured_on(tmp_path):
    src = os.path.join(ROOT, "video_diffusion_transformer_03_amd", "csrc", "k_attn.hip")
    h = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    assert bench.measured_traffic(_summary(tmp_path, h), "block_l16384", "attention") == 1201
    # another workload, another kernel, or a changed source: no traffic figure
    assert bench.measured_traffic(_summary(tmp_path, h), "block_l4096", "attention") is None
    assert bench.measured_traffic(_summary(tmp_path, h), "block_l16384", "gemm_qkv") is None
    assert bench.measured_traffic(_summary(tmp_path, "0" * 16), "block_l16384", "attention") is None
    assert bench.measured_traffic(str(tmp_path / "missing.json"), "block_l16384", "attention") is None


@pytest.mark.parametrize("path", ["profiles/traffic.json"])
def test_committed_traffic_summary_is_well_formed(path):
    tr = json.load(open(os.path.join(ROOT, path)))
    assert tr["workload"] == "block_l16384"
    att = [k for k in tr["kernels"] if k.startswith("attn_v2_kernel")]
    assert att and tr["kernels"][att[0]]["read_bytes"] > 0
    assert set(tr["copy_factor"]) == {"fetch", "write"}


def test_weight_bytes_per_variant():
    # AdaLN bf16 in every variant; a W8A8 projection: one byte per weight plus a 4-byte
    # scale per output channel; a bf16 projection: two bytes per weight
    wl = S.WORKLOADS["block_l16384"]
    d, F, dc = wl.d, wl.d_ff, wl.d_cond
    wb = bench.weight_bytes(wl)
    ada = 6 * d * dc * 2
    w8 = ada + (3 * d * d + d * d + F * d + d * F) + 4 * (3 * d + d + F + d)
    b16 = ada + 2 * (3 * d * d + d * d + F * d + d * F)
    assert wb["w8a8"]["per_block_GiB"] == round(w8 / 2**30, 4)
    assert wb["bf16"]["per_block_GiB"] == round(b16 / 2**30, 4)
    assert wb["w8a8"]["per_block_GiB"] < wb["int8_mlp_qkv"]["per_block_GiB"] < \
        wb["int8_mlp"]["per_block_GiB"] < wb["bf16"]["per_block_GiB"]
