"""Host-side logic of bench.py that runs before any GPU work: the gradual-filtering schedules it
times next to the step, for every workload (a start ratio at or below a workload's own ratio is
skipped rather than rejected), the GPU-count guard, and the traffic figure's workload guard."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_gradual_schedules_for_every_workload():
    for name, w in synth.WORKLOADS.items():
        g = bench.gradual_schedules(w)
        k = synth_budget(w)
        for label, sch in g.items():
            assert len(sch) == w.model.n_layers - w.sel_layer, (name, label)
            # narrows from above r; reaches r when the layers suffice (one scheduled layer is just the start)
            assert sch[0] > k and sch[-1] >= k, (name, label)
            assert all(a >= b for a, b in zip(sch, sch[1:])), (name, label)
            if len(sch) >= 8:
                assert sch[-1] == k, (name, label)
        starts = {int(label.split("%")[0]) for label in g}
        assert starts == {a for a in (20, 30) if a * w.rho_den > 100 * w.rho_num} or w.mode != "token", name


def synth_budget(w):
    return (w.n_ctx * w.rho_num) // w.rho_den if w.rho_num else 0


def test_traffic_only_for_the_profiled_workload():
    out = bench.gemm_traffic(1.0e8, "qwen8b")
    assert "traffic" not in out and "Llama-3-8B" in out["traffic_note"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr
