"""Host-side logic of bench.py and the rocprofv3 summary tool (no GPU)."""

import hashlib
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from frame_wise_gated_amd import inputs as gi  # noqa: E402
from frame_wise_gated_amd import profsum  # noqa: E402


def test_gpus_other_than_one_exit(monkeypatch, capsys):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_per_frame_head_bytes_and_flops():
    w = gi.workload(4)
    pf = bench.per_frame_head(w)
    S, D = 3600, 128
    # phase 1 as the step runs it: bf16 A_t and fp32 U_t in the scan's layout
    assert pf["terms_bytes"] == 2 * S * D * 2 + 4 * S + D * D * (2 + 4)
    assert pf["step_bytes"] == 3766340
    assert pf["readout_bytes"] == 2 * S * D * 2 + 4 * D * D
    assert pf["terms_flop"] == 4 * D * D * S
    assert pf["step_flop"] == 4 * D * D * S + 2 * D * D * S + 2 * D ** 3


def _traffic_file(tmp_path, kernel, variant, workload, sha, nbytes):
    (tmp_path / "profiles").mkdir(exist_ok=True)
    (tmp_path / "profiles" / f"{kernel}__{workload}__hbm_traffic.txt").write_text(
        f"header\nkernel_instance {kernel}{variant}\nsource_sha256 {sha}\n"
        f"hbm_bytes_per_launch {nbytes}\n"
        f"(notes: a later line may start with a field name;\n"
        f"kernel_instance is what the first such line says)\n")


def test_recorded_traffic_follows_source_hash(tmp_path, monkeypatch):
    src_dir = tmp_path / "frame_wise_gated_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (src_dir / "k.hip").write_text("kernel v1\n")
    sha = hashlib.sha256(b"kernel v1\n").hexdigest()
    _traffic_file(tmp_path, "kern", "<false, true>", "wl", sha, 1234)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.recorded_traffic("kern", "<false, true>", "k.hip", "wl") == 1234
    # another instance of the same kernel, another workload: no figure
    assert bench.recorded_traffic("kern", "<true, true>", "k.hip", "wl") is None
    assert bench.recorded_traffic("kern", "<false, true>", "k.hip", "wl_qk_rmsnorm") is None
    (src_dir / "k.hip").write_text("kernel v2\n")      # source changed: counters are stale
    assert bench.recorded_traffic("kern", "<false, true>", "k.hip", "wl") is None
    assert bench.recorded_traffic("other", "<false, true>", "k.hip", "wl") is None


def test_kernel_names_match_launched_instances():
    from frame_wise_gated_amd.inputs import workload
    w = workload(4)
    plain, normed = bench.kernel_names(w, False), bench.kernel_names(w, True)
    assert plain["terms"][:2] == ("terms_dma_bf16_d128", "<true, false, false, false, false>")
    assert plain["readout"][:2] == ("readout_mfma_bf16_d128", "<false>")
    assert normed["terms"][1] == "<true, false, true, false, false>"
    assert normed["readout"][1] == "<true>"
    assert bench.kernel_names(workload(1), False)["terms"][0] == "terms_generic"


def test_profsum_trace_and_pmc(tmp_path):
    (tmp_path / "run_kernel_trace.csv").write_text(
        "Kernel_Name,Grid_Size_X,Start_Timestamp,End_Timestamp\n"
        "gdn::terms_dma_bf16_d128<true>(x),991232,0,1000\n"
        "gdn::terms_dma_bf16_d128<true>(x),991232,0,3000\n"
        "gdn::terms_dma_bf16_d128<true>(x),991232,0,5000\n")
    lines = profsum.trace(str(tmp_path), skip=1)
    row = [l for l in lines if l.startswith("terms_dma_bf16_d128")][0].split()
    assert row[2] == "2" and float(row[3]) == pytest.approx(4.0)
    (tmp_path / "run_counter_collection.csv").write_text(
        "Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n"
        "readout_mfma_bf16_d128,64,FETCH_SIZE,100\n"
        "readout_mfma_bf16_d128,64,FETCH_SIZE,300\n")
    lines = profsum.pmc(str(tmp_path), scale=2.0)
    row = [l for l in lines if l.startswith("readout_mfma_bf16_d128")][0].split()
    assert float(row[4]) == pytest.approx(200.0)
    assert float(row[5]) == pytest.approx(200 * 1024 * 2 / 1e6, rel=1e-3)


def test_profsum_mfma_utilisation(tmp_path):
    # 1000 MFMA instructions of 32 busy cycles each over 10 us on 4 SIMDs at
    # 1 GHz: 32000 busy cycles of 40000 available
    (tmp_path / "run_counter_collection.csv").write_text(
        "Kernel_Name,Grid_Size,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
        "readout_mfma_bf16_d128<false>(x),64,SQ_INSTS_MFMA,1000,0,10000\n"
        "readout_mfma_bf16_d128<false>(x),64,SQ_VALU_MFMA_BUSY_CYCLES,32000,0,10000\n"
        "grad_init_kernel(x),64,SQ_INSTS_MFMA,0,0,1000\n"
        "grad_init_kernel(x),64,SQ_VALU_MFMA_BUSY_CYCLES,0,0,1000\n")
    lines = profsum.mfma(str(tmp_path), simds=4, clock_ghz=1.0)
    assert not any(l.startswith("grad_init_kernel") for l in lines)
    row = [l for l in lines if l.startswith("readout_mfma_bf16_d128<false>")][0].split()
    assert row[-5:] == ["1", "10.0", "1000", "32.0", "0.800"]


def test_summarize_calls_median_min_and_phases():
    calls = [{"total": 3.0, "terms": 1.0, "readout": 1.5},
             {"total": 1.0, "terms": 0.4, "readout": 0.5, "scan": 0.1},
             {"total": 2.0, "terms": 0.7, "readout": 1.0}]
    s = bench.summarize_calls(calls)
    assert s["mean"] == pytest.approx(2.0) and s["median"] == 2.0 and s["min"] == 1.0
    assert s["phase_median"]["terms"] == 0.7 and s["phase_median"]["readout"] == 1.0
    # a phase missing from a call counts as zero time in that call
    assert s["phase_median"]["scan"] == 0.0
    assert s["phase_mean"]["scan"] == pytest.approx(0.1 / 3)


def test_pages_context_is_labelled_not_comparable():
    assert bench.PAGES_CONTEXT["comparable"] is False
    assert "34 s" in bench.PAGES_CONTEXT["whole_model_60s_720p"]
    assert "1.5-2x" in bench.PAGES_CONTEXT["fused_kernel_speedup"]
