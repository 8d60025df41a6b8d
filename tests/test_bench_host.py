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


def test_row_step_and_deviation_bytes_are_the_scope_numerators():
    """The row steps (gather + norm + K/V scatter) and the selection-layer deviation are credited with
    the bytes the method must move, worked by hand for the Llama-3-8B request: per layer n_sel x d
    fp32 residual rows read once plus n_sel x kvd keys and values written once (all L rows on the
    full layer 0), plus the selection layer's norm of the N context rows and the final norm of the U
    query rows; the deviation reads the N stitched keys and writes N floats."""
    from selective_recompute_cf_amd import roofline as rl
    s = rl.shape_of(synth.LLAMA3_8B)
    N, U, k = 3072, 64, 460
    L, n = N + U, k + U
    w = rl.blend_step_work(s, N, U, k, 1)
    per = lambda rows: rows * 4096 * 4 + 2 * rows * 1024 * 2
    assert w["h4h6_rows"] == per(L) + 31 * per(n) + 4 * N * 4096 + 2 * 4 * U * 4096
    assert w["h2_deviation"] == N * 1024 * 2 + 4 * N
    assert abs(w["h4h6_rows"] / 1e6 - 449.33) < 0.01  # MB per request: 64.2 + 31 x 10.7 + 50.3 + 2.1
    # the unfused kernels' traffic is reported apart and is larger
    assert w["unfused:rows"] + w["unfused:qkv_post"] > w["h4h6_rows"]


def test_cpu_leg_compares_against_both_oracle_modes():
    """The CPU leg's end-to-end comparisons on the tiny bf16 model, fed the fp32 oracle's own result
    as the GPU's: against the fp32 oracle everything agrees exactly; the bf16-arithmetic oracle sits a
    small non-zero distance from it; and the 'GPU' (here the fp32 result) is exactly that distance
    from the bf16-arithmetic oracle, in both directions of the comparison."""
    import numpy as np
    import oracle
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(dtype="bf16", n_layers=2))
    k = synth_budget(w)
    model = synth.Model(w.model)
    chunks, _, toks = synth.request_tokens(w)
    ks, vs, tab, row = [], [], [], 0
    for c in chunks:
        a, b = oracle.chunk_prefill(model, c, np.float32)
        ks.append(a)
        vs.append(b)
        tab.append((row, 0, row, len(c)))
        row += len(c)
    spans = [i * w.chunk_len for i in range(w.n_chunks + 1)]
    r = oracle.blend_prefill(model, toks, w.n_ctx, np.concatenate(ks, 1), np.concatenate(vs, 1), tab, w.sel_layer, k,
                             w.mode, spans, np.float32)
    Ly, L = w.model.n_layers, w.n_total
    gpu = dict(sel=r.sel[:k], k=r.k.reshape(Ly, L, -1), v=r.v.reshape(Ly, L, -1), out=r.out)
    cpu, north = bench.cpu_baseline(w, k, gpu, runs=1)
    assert cpu["kind"] == "oracle" and cpu["value"] > 0
    assert north["selection_overlap"] == 1.0
    for t in ("out", "K", "V"):
        assert north[t]["norm_rel"] == 0.0 and north[t]["outside_bar_frac"] == 0.0
    b16, g16 = north["bf16_arithmetic_oracle_vs_fp32_oracle"], north["gpu_vs_bf16_arithmetic_oracle"]
    for t in ("out", "K", "V"):
        assert 1e-5 < b16[t]["norm_rel"] < 2e-2
        assert abs(g16[t]["max_abs"] - b16[t]["max_abs"]) < 1e-6
