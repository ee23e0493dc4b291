"""Host-side parts of the benchmark (CPU): the byte and FLOP model behind the
roofline figures, the one-GPU refusal, and the rocprofv3 summary."""

import os
import subprocess
import sys

import bench
from sparse_attention_09_amd import dsa, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_verify_batch():
    """128 requests x 8 verify tokens at 64K context, top-2048, FP8 rows of
    612 bytes (576 codes + 9 fp32 scales), worked out by hand."""
    s = synth.spec("verify_fp8_64k")
    plan = dsa.plan_partial(1024, 2048, 0, 0, 256)
    row = dsa.pool_layout(s.kv_dtype, 1).latent_row_bytes
    assert row == 612
    b = bench.algorithmic_bytes(s, plan, row, fused=True)
    T, k = 1024, 2048
    keys = 128 * 65536 * 256                       # one read of every request's keys
    q_idx_w = T * (16 * 128 * 2 + 16 * 4)          # indexer queries and head weights
    vis = 128 * sum(p + 1 for p in range(65528, 65536))   # visible positions of the 8 tokens
    assert b["index_topk"] == keys + q_idx_w + T * k * 4 == 2_160_132_096
    assert b["index_scores"] == keys + q_idx_w + vis * 4
    assert b["topk"] == vis * 4 + T * k * 4
    # Partial with one split: indices, selected rows, q in; bf16 output and lse out
    assert b["partial"] == T * k * 4 + T * k * 612 + T * 64 * 576 * 2 + T * 64 * (512 * 2 + 4)
    assert b["partial"] == 1_434_714_112
    f = bench.flops(s)
    assert f["partial"] == T * 64 * k * (576 + 512) * 2
    assert f["index_topk"] == vis * 16 * 128 * 2


def test_split_plan_counts_partials_and_combine():
    s = synth.spec("longctx_fp8_1m")
    plan = dsa.plan_partial(8, 2048, 0, 0, 256)
    b = bench.algorithmic_bytes(s, plan, 612, fused=False)
    S = plan.splits
    assert S == 16
    parts = 8 * S * 64 * (512 + 1) * 4
    assert b["combine"] == parts + 8 * 64 * (512 * 2 + 4)
    assert b["partial"] == 8 * 2048 * 4 + 8 * 2048 * 612 + 8 * 64 * 576 * 2 + parts


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stats_summary_sums_the_fused_selection(tmp_path):
    csv = tmp_path / "k.csv"
    rows = [("void (anonymous namespace)::index_kernel<1>(x)", 10, 20000),
            ("(anonymous namespace)::threshold_kernel(x)", 10, 9000),
            ("void (anonymous namespace)::index_kernel<2>(x)", 10, 400000),
            ("(anonymous namespace)::select_kernel(x)", 10, 35000),
            ("(anonymous namespace)::fallback_kernel(x)", 10, 4000),
            ("void (anonymous namespace)::partial_v2_kernel<1, 64, true>(x)", 10, 460000),
            ("some_other_kernel", 3, 1000)]
    lines = ["Name,Calls,AverageNs,MinNs,MaxNs"]
    lines += [f'"{n}",{c},{a},{a},{a}' for n, c, a in rows]
    csv.write_text("\n".join(lines) + "\n")
    out = bench.summarize_stats(str(csv), "cmd")
    got = {l.split()[0]: l.split() for l in out.splitlines() if not l.startswith("#")}
    assert "some_other_kernel" not in out
    assert float(got["partial"][2]) == 460.0
    assert float(got["index_topk"][2]) == (20000 + 9000 + 400000 + 35000 + 4000) / 1e3


def test_mfma_summary_from_counters(tmp_path):
    """MFMA use per launch from a counter CSV: counted FLOPs (512 per MOPS
    unit) over the dispatch time, busy share of the 1024 SIMDs' cycles."""
    csv = tmp_path / "c.csv"
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp"
    rows = [head]
    name = '"void (anonymous namespace)::partial_ws_kernel<1, true>(x)"'
    # 1e9 MOPS units over 400 us -> 512e9 / 4e-4 s = 1280 TFLOP/s; busy 2.5e8 of 1e6 x 1024 cycles
    for c, v in (("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9), ("SQ_VALU_MFMA_BUSY_CYCLES", 2.56e8),
                 ("GRBM_GUI_ACTIVE", 8e6), ("MfmaUtil", 25.0)):
        rows.append(f"7,{name},{c},{v},1000,401000")
    csv.write_text("\n".join(rows) + "\n")
    out = bench.summarize_mfma(str(csv), "w", ["cmd"])
    k = out["kernels"]["partial"]
    assert k["mfma_tflops_counted"] == 1280.0
    assert k["busy_cycles_frac"] == 0.25
    assert k["mfma_util"] == 0.25


def test_lds_summary_from_counters(tmp_path):
    """LDS use per launch from a counter CSV: medians over dispatches and the
    share of LDS-active cycles spent in bank conflicts."""
    csv = tmp_path / "c.csv"
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp"
    rows = [head]
    name = '"void (anonymous namespace)::partial_q8_kernel(x)"'
    for d, conf in ((1, 10.0), (2, 30.0), (3, 20.0)):
        for c, v in (("SQ_LDS_BANK_CONFLICT", conf), ("SQ_LDS_IDX_ACTIVE", 200.0),
                     ("SQ_INSTS_LDS", 50.0), ("SQ_WAIT_INST_LDS", 7.0)):
            rows.append(f"{d},{name},{c},{v},1000,2000")
    csv.write_text("\n".join(rows) + "\n")
    out = bench.summarize_lds(str(csv), "w", ["cmd"])
    k = out["kernels"]["partial_q8"]
    assert k["dispatches"] == 3
    assert k["SQ_LDS_BANK_CONFLICT"] == 20 and k["SQ_LDS_IDX_ACTIVE"] == 200
    assert k["conflict_frac"] == 0.1

