"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the staleness
rule for committed HBM-traffic counters, and the report summary."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from rmsnorm_inputs import ALL_WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "single GPU" in (r.stdout + r.stderr)


@pytest.mark.parametrize("workload", ["bf16_4096x4096", "bf16_1024x8192", "bf16_512x2048"])
def test_committed_counters_belong_to_the_current_kernel(workload):
    """The bench reports counter traffic only when the committed counters were
    taken on the kernel sources and plan it runs; any other identity reads as
    stale (None)."""
    ident = bench.source_hash(bench.bwd_plan_for(ALL_WORKLOADS[workload]))
    t = bench.counters_traffic(ident, workload)
    assert t is not None, f"profiles/hbm_traffic_{workload}.txt is stale for the current sources"
    w = ALL_WORKLOADS[workload]
    from rmsnorm_inputs import algorithmic_bytes
    alg = algorithmic_bytes("bwd_main", w.M, w.N, w.elem_bytes)
    assert alg <= t <= 1.5 * alg  # traffic is at least the compulsory bytes
    assert bench.counters_traffic("0" * 16, workload) is None
    assert bench.counters_traffic(ident, "no_such_workload") is None


def test_report_summary_lists_every_op_and_the_workspace_column(tmp_path, capsys):
    cold = {"fwd_us": 10.0, "bwd_us": 20.0, "bwd_main_us": 17.0, "finalize_us": 3.0, "fwd_fp8_us": 11.0,
            "ln_fwd_us": 12.0, "ln_bwd_us": 22.0, "fwd_GBs": 5000.0, "fwd_pct_peak": 62.5, "bwd_GBs": 4000.0,
            "bwd_pct_peak": 50.0, "bwd_incl_ws_GBs": 4400.0, "ln_bwd_incl_ws_GBs": 4100.0, "fwd_graph_us": 9.5}
    rep = {"workloads": [{"workload": "bf16_4096x4096", "cold": cold, "hot": {"fwd_us": 9.0},
                          "ceilings": {"copy_GBs": 5500.0, "three_stream_GBs": 5900.0},
                          "plans": {"fwd": {"path": 0, "vec": 8, "team": 0, "threads": 256, "chunks": 2, "depth": 0,
                                            "w_regs": 0, "rows_per_step": 1, "grid": 4096}}}]}
    p = tmp_path / "rep.json"
    p.write_text(json.dumps(rep))
    bench.summarize_report(str(p))
    out = capsys.readouterr().out.splitlines()
    assert "incl. ws GB/s" in out[0]
    rows = {ln.split()[1]: ln.split() for ln in out[1:] if ln.strip().startswith("bf16_4096x4096") and
            "plan:" not in ln and "ceilings:" not in ln}
    assert set(rows) == {"fwd", "bwd", "bwd_main", "finalize", "fwd_fp8", "ln_fwd", "ln_bwd"}
    assert rows["bwd"][-1] == "4400.0" and rows["ln_bwd"][-1] == "4100.0" and rows["fwd"][-1] == "-"
    assert any("ceilings: copy 5500 GB/s, three-stream 5900 GB/s" in ln for ln in out)
    assert any("fwd plan: path 0 vec 8 team 0 threads 256 chunks 2" in ln for ln in out)
