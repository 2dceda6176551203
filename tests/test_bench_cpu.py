"""CPU checks of bench.py's bookkeeping: the byte and flop counts behind the
roofline, the kernel the dispatch rule picks, the stage lists, and the
counter summaries the roofline's traffic is read from (no GPU needed)."""
import os

import bench


def test_projection_bytes_match_the_formats():
    H, I = 2816, 704
    # NVFP4: packed nibbles, one E4M3 code per 16, one FP32 scale per tensor
    assert bench.proj_bytes(H, I) == H * I // 2 + H * I // 16 + 4 == 1115140
    # q4_0: one fp16 d per 32; aff4: fp16 s and b per 32; no tensor scale
    assert bench.proj_bytes(H, I, "q4_0") == H * I // 2 + H * I // 16
    assert bench.proj_bytes(H, I, "aff4") == H * I // 2 + H * I // 8
    assert bench.expert_bytes_per_expert(H, I) == 3 * 1115140


def test_gate_up_kernel_follows_the_dispatch_rule():
    # GEMV mode below 24 rows per active expert on average: 8-row tiles up
    # to 4 rows per expert, else 16; the tiled GEMM above
    assert bench.gate_up_kernel_name(64, 8, 128) == "k_expert_gemv<8, 2, true, 4, 0, 1>"
    assert bench.gate_up_kernel_name(4, 8, 128) == "k_expert_gemv<8, 2, true, 4, 0, 1>"
    assert bench.gate_up_kernel_name(128, 8, 128) == "k_expert_gemv<16, 2, true, 4, 0, 1>"
    assert bench.gate_up_kernel_name(2048, 8, 128) == "k_expert_gemm<8, 2, true, 0>"
    assert bench.gate_up_kernel_name(2040, 8, 128) == "k_expert_gemm<4, 2, true, 0>"
    assert bench.gate_up_kernel_name(3072, 8, 128) == "k_expert_gemm<8, 2, true, 0>"
    assert bench.gate_up_kernel_name(16384, 8, 128) == "k_expert_gemm<8, 2, true, 0>"
    assert bench.gate_up_kernel_name(64, 8, 128, "aff4") == "k_expert_gemv<8, 2, true, 4, 2, 1>"


def test_stage_lists():
    assert bench.STAGES == ("route_bucket_prep", "gate_up", "down", "combine")
    assert bench.SEPARATE_STAGES == ("route_bucket", "prep", "gate_up", "down", "combine")


def test_committed_counter_summaries_name_the_dominant_kernels():
    here = os.path.dirname(bench.__file__)
    for wl, T in (("moe_layer_decode_T64", 64), ("moe_layer_prefill_T2048_zipf1.2", 2048),
                  ("moe_layer_prefill_T16384_zipf1.2_outliers", 16384)):
        path = os.path.join(here, "profiles", f"hbm_traffic__{wl}.txt")
        rec = dict(l.split(":", 1) for l in open(path) if ":" in l and not l.startswith("#"))
        assert rec["kernel"].strip() == bench.gate_up_kernel_name(T, 8, 128)
        assert float(rec["hbm_bytes_per_launch"]) > 0
        assert len(rec["source_sha256"].strip()) == 64


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    import pytest
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
