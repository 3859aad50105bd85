"""The roofline accounting bench.py reports: algorithmic FLOPs and HBM bytes
of the measured workloads, checked against figures derived by hand from the
operation's inputs and outputs (no GPU needed)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_fwdbwd_model_flops_and_bytes():
    # B8 H16 T4096 d56, chunk 64: 8192 chunk-heads; per chunk-head
    # fwd 10 C^2 d + 6 C d^2 + C^3 / 3, bwd 20 C^2 d + 12 C d^2 + 4 C^3
    flops, nbytes = bench.step_model(8, 4096, 16, 56)
    assert flops == pytest.approx(95.27e9, rel=1e-3)
    # read q, k, v, do (bf16), g, beta; write o, dq, dk, dv (bf16), dg, dbeta;
    # h0 and dh0 / hT states fp32, dA_log
    assert nbytes == pytest.approx(664.93e6, rel=1e-4)


def test_per_kernel_bytes_sum_to_the_step():
    per = bench.kernel_bytes_per_token_head(56)
    th = 8 * 4096 * 16
    states = 8 * 16 * 56 * 56 * 4
    total = sum(per.values()) * th
    # every tensor of the step is counted by exactly one kernel except k and g
    # (read by both forward kernels) and q, k, do and g (read by both backward
    # kernels); the states and dA_log belong to no per-token figure
    e = 2 * 56
    double_counted = th * ((e + 4) + (3 * e + 4))
    _, step_bytes = bench.step_model(8, 4096, 16, 56)
    assert total - double_counted == step_bytes - 4 * states - 16 * 4


def test_decode_step_bytes():
    # 256 x 16 states of 56 x 56 fp32 read and written, bf16 q, k, v in, o out,
    # fp32 g and beta in
    assert bench.decode_bytes_per_step(256, 16, 56, 56) == 104_628_224
    assert bench.decode_bytes_per_step(256, 16, 56, 56) == pytest.approx(104.63e6, rel=1e-4)


def test_multi_gpu_request_is_refused(capsys, monkeypatch):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def _write_counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "p_counter_collection.csv"), "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for disp, (name, val) in enumerate(rows):
            f.write(f'{disp},"{name}",{counter},{val}\n')


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    """HBM traffic = counter KiB x 1024 x (copy bytes / copy counter bytes),
    per counter, averaged over dispatches; written with the kernel's source
    hash. Synthetic counter files: the 256 MiB copy reads as 2x its size on
    FETCH_SIZE and 1x on WRITE_SIZE."""
    root = tmp_path / "repo"
    (root / "profiles").mkdir(parents=True)
    os.symlink(os.path.join(ROOT, "gated_delta_rule_74_amd"), root / "gated_delta_rule_74_amd")
    monkeypatch.setattr(bench, "ROOT", str(root))
    copy_kib = bench.COPY_BYTES / 1024
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE",
                    [("__amd_rocclr_copyBuffer", 2 * copy_kib), ("void gdn::bwd_local_kernel<true, 64, true>(x)", 1000.0),
                     ("void gdn::bwd_local_kernel<true, 64, true>(x)", 3000.0)])
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE",
                    [("__amd_rocclr_copyBuffer", copy_kib), ("void gdn::bwd_local_kernel<true, 64, true>(x)", 500.0),
                     ("void gdn::bwd_local_kernel<true, 64, true>(x)", 500.0)])
    bench.traffic_summary(str(tmp_path / "fetch"), str(tmp_path / "write"), bench.HEADLINE)
    import json

    with open(root / "profiles" / f"bwd_local_{bench.HEADLINE}_traffic.json") as f:
        rec = json.load(f)
    assert rec["copy_fetch_scale"] == 0.5 and rec["copy_write_scale"] == 1.0
    assert rec["read_bytes"] == round(2000.0 * 1024 * 0.5)
    assert rec["write_bytes"] == round(500.0 * 1024)
    assert rec["traffic_bytes"] == rec["read_bytes"] + rec["write_bytes"]
    assert rec["source_hash"] == bench.source_hash("bwd_local")
    assert bench.load_traffic("bwd_local", bench.HEADLINE) == rec["traffic_bytes"]
    assert bench.load_traffic("bwd_local", "long_ctx") is None
    assert (root / "profiles" / "traffic_fwdbwd_model.txt").exists()


def test_mfma_summary_arithmetic(tmp_path, monkeypatch):
    """busy % = MFMA busy cycles / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs);
    flops = MOPS x 512; TFLOP/s over the dispatch's own duration. Synthetic
    counters: 25 % busy, 1e6 bf16 MOPS in 1 ms."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda kernel=None: "test")
    d = tmp_path / "mfma"
    d.mkdir()
    name = "void gdn::bwd_local_kernel<true, 64, true>(x)"
    vals = {"GRBM_GUI_ACTIVE": 8000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 0.25 * 1000 * bench.SIMD_NUM,
            "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1e6, "SQ_INSTS_VALU_MFMA_MOPS_F32": 0.0}
    with open(d / "p_counter_collection.csv", "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n")
        for cn, v in vals.items():
            f.write(f'7,"{name}",{cn},{v},1000,1001000\n')
    bench.mfma_summary(str(d), bench.HEADLINE)
    row = [ln for ln in open(tmp_path / "profiles" / f"mfma_{bench.HEADLINE}.txt") if ln.startswith("bwd_local")]
    assert len(row) == 1
    f = row[0].split()
    assert f[1] == "1" and float(f[2]) == 25.0
    assert float(f[3]) == 0.512 and float(f[4]) == 0.0
    assert float(f[6]) == 1000.0 and float(f[7]) == 0.5


def test_kernel_names_map_to_timed_kernels():
    """Device kernel symbols (every instance, the wave-specialised and wide
    variants included) are grouped under the timed kernel they belong to."""
    assert bench.kernel_of("void gdn::fwd_chain_ws_kernel<64, true>(gdn::FwdChainArgs)") == "fwd_chain"
    assert bench.kernel_of("void gdn::bwd_local_wide_kernel<true>(gdn::BwdLocalArgs)") == "bwd_local"
    assert bench.kernel_of("gdn::dA_reduce_kernel(float const*, float*, int, int, int)") == "dA_reduce"
    assert bench.kernel_of("void gdn::step_kernel<true, 64, true>(gdn::StepArgs)") is None
    assert bench.kernel_of("__amd_rocclr_copyBuffer") is None


def test_long_context_model():
    # B1 H16 T32768 d128: 8192 chunk-heads
    flops, nbytes = bench.step_model(1, 32768, 16, 128)
    assert flops == pytest.approx(292.77e9, rel=1e-3)
    assert nbytes == pytest.approx(1493.17e6, rel=1e-4)


def test_sample_units():
    assert bench._sample_units(1.0, 128, 16, 4.0) == 64     # 4 s x 16 threads of 1 s units
    assert bench._sample_units(0.001, 128, 16, 4.0) == 128  # capped at the whole workload
    assert bench._sample_units(100.0, 128, 16, 4.0) == 1    # at least one unit
