"""Llama-3-70B-shaped requests (d 8192, 64/8 heads, FFN 28672; 16 chunks x 1024 + 256 query tokens,
top-10% selected on layer 1) on the GPU, at reduced depth.

* Full width, reduced length (4 x 1024 + 256, k = 409), 2 layers: parity with the fp32 oracle under
  the end-to-end bf16 bars of test_gpu_e2e (selection bit-exact on the GPU's own deviation).
* The full request (16 x 1024 + 256, k = 1638), 2 layers, in the launch configuration of a real
  request, through properties that hold at any size: rho = 100% reproduces the library's own full
  prefill bit for bit; the selection equals the exact top-k of the GPU's deviation; the first
  chunk (no preceding context) has near-zero deviation and is never selected."""
import numpy as np
import pytest

import oracle
import synth
from selective_recompute_cf_amd.device import DeviceModel
from tests._gpu import context, gpu_blend, gpu_chunk_store, host, say
from tests.test_gpu_e2e import _check, _run

pytestmark = pytest.mark.gpu


def test_llama3_70b_width_reduced_length():
    w = synth.WORKLOADS["llama70b"].replace(n_chunks=4)
    model, toks, g, r32, *_ = _run(w, n_layers=2)
    assert len(g["sel"]) == oracle.budget(w.n_ctx, w.rho_num, w.rho_den) == 409
    _check(w, g, r32)


def test_llama3_70b_full_request_properties():
    w = synth.WORKLOADS["llama70b"]
    ly = 2
    model = synth.Model(w.model)
    chunks, _, toks = synth.request_tokens(w)
    N, L = w.n_ctx, w.n_total
    k = oracle.budget(N, w.rho_num, w.rho_den)
    assert (N, L, k) == (16384, 16640, 1638)
    say(f"70b full request: N={N} L={L} k={k}, {ly} layers")
    ctx = context(w.model.replace(n_layers=ly), max_pos=L + 1)
    dm = DeviceModel(model, n_layers=ly)
    gk, gv, starts = gpu_chunk_store(ctx, dm, chunks)
    table = [(s, 0, s, len(c)) for s, c in zip(starts, chunks)]
    g = gpu_blend(ctx, dm, toks, N, gk, gv, table, w.sel_layer, k, "token")
    np.testing.assert_array_equal(g["sel"], oracle.select_topk(g["dev"], k))
    assert np.all(g["sel"] >= w.chunk_len), "first chunk selected"
    med = float(np.median(g["dev"][w.chunk_len:]))
    assert float(np.max(g["dev"][: w.chunk_len])) < 1e-3 * med
    say(f"  selection exact; first-chunk max deviation {np.max(g['dev'][: w.chunk_len]):.3e} vs median {med:.3e}")
    full = gpu_blend(ctx, dm, toks, N, None, None, None, 0, 0, "all")
    g100 = gpu_blend(ctx, dm, toks, N, gk, gv, table, w.sel_layer, N, "token")
    np.testing.assert_array_equal(g100["out"], full["out"])
    np.testing.assert_array_equal(g100["k"], full["k"])
    np.testing.assert_array_equal(g100["v"], full["v"])
    assert np.isfinite(g["out"]).all() and np.isfinite(g["k"]).all()
    say("  rho = 100% equals full prefill bit for bit")
