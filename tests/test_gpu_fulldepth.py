"""The Llama-3-8B-shaped request at full depth (32 layers, 6 x 512 + 64, k = 460), in the launch
configuration the benchmark times, and the Qwen3-8B-shaped one (36 layers, 10 x 1024 + 128, 30%,
qk-norm), checked through properties that hold at any size (a CPU oracle run of every layer at
this width is too slow for a test):
* the first layers of the full-depth run equal the short run (3 layers for the Llama shape, 2 for
  the Qwen shape) bit for bit, a layer's results depending only on the layers before it; the
  short runs are the ones test_gpu_e2e holds to the oracle;
* the selection is the exact top-k of the GPU's own selection-layer deviation;
* context rows outside the selection keep the re-positioned store at every layer >= 1, and the
  selected and query rows are rewritten at every layer;
* rho = 100% equals the library's own full prefill bit for bit;
* every output is finite."""
import numpy as np
import pytest

import oracle
import synth
from selective_recompute_cf_amd.device import DeviceModel
from tests._gpu import context, gpu_blend, gpu_chunk_store, host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,layers,k_want,short", [("llama8b", 32, 460, 3), ("qwen8b", 36, 3072, 2)])
def test_full_depth_properties(name, layers, k_want, short):
    import torch
    w = synth.WORKLOADS[name]
    N, L, U = w.n_ctx, w.n_total, w.n_query
    cfg = w.model
    assert cfg.n_layers == layers
    say(f"full depth {name}: uploading {layers} layers")
    model = synth.Model(cfg, cache_layers=False)
    chunks, _, toks = synth.request_tokens(w)
    ctx = context(cfg, max_pos=L + 1)
    dm = DeviceModel(model)
    gk, gv, starts = gpu_chunk_store(ctx, dm, chunks)
    table = [(s0, 0, s0, len(c)) for s0, c in zip(starts, chunks)]
    k = oracle.budget(N, w.rho_num, w.rho_den)
    assert k == k_want
    say(f"full depth {name}: blended prefill")
    g = gpu_blend(ctx, dm, toks, N, gk, gv, table, w.sel_layer, k, "token")
    for key in ("k", "v", "out", "dev"):
        assert np.isfinite(g[key]).all(), key
    np.testing.assert_array_equal(g["sel"], oracle.select_topk(g["dev"], k))

    # the first layers of the full-depth run are those of the short run (same kernels, same plans)
    say(f"full depth: {short}-layer run of the same model")
    ctx3 = context(cfg.replace(n_layers=short), max_pos=L + 1)
    dm3 = DeviceModel(model, n_layers=short)
    g3 = gpu_blend(ctx3, dm3, toks, N, gk[:short], gv[:short], table, w.sel_layer, k, "token")
    np.testing.assert_array_equal(g["k"][:short], g3["k"])
    np.testing.assert_array_equal(g["v"][:short], g3["v"])
    np.testing.assert_array_equal(g["sel"], g3["sel"])
    np.testing.assert_array_equal(g["dev"], g3["dev"])
    del dm3

    # unselected context rows keep the stitched cache at every layer from the selection layer on
    kb = torch.zeros(cfg.n_layers, L, ctx.kv_dim, dtype=torch.bfloat16, device="cuda")
    vb = torch.zeros_like(kb)
    ctx.rope_reposition(gk, gv, kb, vb, table, 0, cfg.n_layers)
    torch.cuda.synchronize()
    kst, vst = host(kb), host(vb)
    rest = np.setdiff1d(np.arange(N), g["sel"])
    rows = np.concatenate([g["sel"], np.arange(N, L)])
    for l in range(w.sel_layer, cfg.n_layers):
        np.testing.assert_array_equal(g["k"][l][rest], kst[l][rest], err_msg=f"layer {l}")
        np.testing.assert_array_equal(g["v"][l][rest], vst[l][rest], err_msg=f"layer {l}")
        assert np.any(g["k"][l][rows] != kst[l][rows], axis=1).mean() > 0.99, f"layer {l}: rows not rewritten"

    # rho = 100% is full prefill, bit for bit
    say("full depth: rho = 100% against full prefill")
    g_all = gpu_blend(ctx, dm, toks, N, gk, gv, table, w.sel_layer, N, "token")
    full = gpu_blend(ctx, dm, toks, N, None, None, None, 0, 0, "all")
    np.testing.assert_array_equal(g_all["out"], full["out"])
    np.testing.assert_array_equal(g_all["k"], full["k"])
    assert U == g["out"].shape[0]
