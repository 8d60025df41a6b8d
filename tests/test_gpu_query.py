"""GPU parity of cf_query_scores (QCFuse §3.2.1 Eq. 10 / Eq. 20: the query rows' attention mass on
each context position, over a set of layers, with the query probing the stitched cache) against
oracle.query_scores, and of the query-aware blend (cf_blend_prefill with the top of those scores
as a given set) against the oracle's blend of the same set.

Bars: fp32 models elementwise (scores within 1e-4 relative plus 1e-6 of the largest score);
bf16 models against the fp32 oracle under the end-to-end bf16 bars of the blend tests (norm-wise
drift of the scores within 2e-2 per layer the probe runs, no 128-position chunk 4x further; the
top-10% sets overlapping by >= 97%, every disagreement a near tie); the probe never writes context
rows."""
import numpy as np
import pytest

import oracle
import selective_recompute_cf_amd as cf
import synth
from selective_recompute_cf_amd.device import DeviceModel
from tests._gpu import compare, context, e2e_bf16, e2e_selection, gpu_blend, gpu_chunk_store, host, overlap, say

pytestmark = pytest.mark.gpu


def nrel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def _setup(w, ly):
    import torch
    model = synth.Model(w.model)
    chunks, _, toks = synth.request_tokens(w)
    N, L = w.n_ctx, w.n_total
    ctx = context(model.cfg.replace(n_layers=ly), max_pos=max(4096, L + 1))
    dm = DeviceModel(model, n_layers=ly)
    gk, gv, starts = gpu_chunk_store(ctx, dm, chunks)
    table = [(s0, 0, s0, len(c)) for s0, c in zip(starts, chunks)]
    kb = torch.zeros(ly, L, ctx.kv_dim, dtype=gk.dtype, device="cuda")
    vb = torch.zeros_like(kb)
    ctx.rope_reposition(gk, gv, kb, vb, table, 0, ly)
    torch.cuda.synchronize()
    return model, toks, ctx, dm, gk, gv, table, kb, vb


def _gpu_scores(ctx, dm, toks, N, kb, vb, layer_set):
    import torch
    U = len(toks) - N
    scores = torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(ctx.query_scores_workspace_size(N, U), dtype=torch.uint8, device="cuda")
    tok = torch.from_numpy(np.asarray(toks, np.int32)).cuda()
    ctx.query_scores(dm.array, dm.embed, tok, N, U, kb, vb, layer_set, scores, ws)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


def _oracle_scores(model, toks, N, gk, gv, table, ly, layer_set):
    cfg = model.cfg
    shape = (ly, gk.shape[1], cfg.n_kv_heads, cfg.head_dim)
    ks, vs = host(gk).reshape(shape), host(gv).reshape(shape)
    kst, vst = oracle.stitch(ks, vs, table, N, range(ly), cfg.rope_theta, np.float32, n_total=len(toks))
    return oracle.query_scores(model, toks, N, kst, vst, layer_set, np.float32), ks, vs


def _check(w, ly, layer_set):
    N = w.n_ctx
    model, toks, ctx, dm, gk, gv, table, kb, vb = _setup(w, ly)
    say(f"query scores {w.name} layers={ly} set={layer_set}")
    k_ctx_before = host(kb[:, :N])
    g = _gpu_scores(ctx, dm, toks, N, kb, vb, layer_set)
    np.testing.assert_array_equal(host(kb[:, :N]), k_ctx_before)  # context rows only read
    o32, *_ = _oracle_scores(model, toks, N, gk, gv, table, ly, layer_set)
    assert np.isfinite(g).all()
    if model.cfg.dtype != "bf16":
        compare("scores", g, o32, atol=1e-6 * float(o32.max()), rtol=1e-4)
        return g, o32
    e2e_bf16("scores", g, o32, max(layer_set) + 1, 128)
    k = max(1, N // 10)
    e2e_selection(oracle.select_topk(g, k), oracle.select_topk(o32, k), o32, k, True)
    return g, o32


def test_tiny_fp32_all_layers_and_one_layer():
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(n_layers=3))
    _check(w, 3, [0, 1, 2])
    _check(w, 3, [1])


def test_gqa4_hd128_bf16_critical_layers():
    m = synth.TINY.replace(name="mid", n_layers=4, d_model=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
                           d_ffn=2816, vocab=2000, rope_theta=5e5, dtype="bf16")
    w = synth.Workload("mid-5x200+40", m, 5, 200, 40, 15, 100)
    _check(w, 4, [1, 3])


def test_qknorm_hd64_bf16_many_query_rows():
    """qk-norm, head_dim 64, 130 query rows (the query rows pass through LDS in chunks of 64 rows
    x heads)."""
    m = synth.TINY.replace(name="mid-qk", n_layers=3, d_model=512, n_q_heads=8, n_kv_heads=1, head_dim=64,
                           d_ffn=1408, vocab=2000, rope_theta=1e6, rms_eps=1e-6, qk_norm=True, dtype="bf16")
    w = synth.Workload("mid-qk-4x256+130", m, 4, 256, 130, 30, 100)
    _check(w, 3, [0, 1, 2])


def test_llama3_8b_shape_three_layers():
    """Llama-3-8B width and request length (6 x 512 + 64), layers 0-2, scored on layers 1 and 2."""
    _check(synth.WORKLOADS["llama8b"], 3, [1, 2])


def test_query_aware_blend_given_set():
    """QCFuse's path on the tiny fp32 model: the top 15% of the GPU's scores over all layers,
    recomputed from layer 0 as a given set, against the oracle's blend of that same set."""
    import torch
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(n_layers=3))
    N, L = w.n_ctx, w.n_total
    model, toks, ctx, dm, gk, gv, table, kb, vb = _setup(w, 3)
    g = _gpu_scores(ctx, dm, toks, N, kb, vb, [0, 1, 2])
    k = oracle.budget(N, w.rho_num, w.rho_den)
    sel = torch.from_numpy(oracle.select_topk(g, k).astype(np.int32)).cuda()
    k_out = torch.zeros(3, L, ctx.kv_dim, dtype=torch.float32, device="cuda")
    v_out = torch.zeros_like(k_out)
    out = torch.zeros(L - N, dm.cfg.d_model, dtype=torch.float32, device="cuda")
    ws = torch.empty(ctx.blend_prefill_workspace_size(N, L - N, k, "given"), dtype=torch.uint8, device="cuda")
    tok = torch.from_numpy(np.asarray(toks, np.int32)).cuda()
    ctx.blend_prefill(dm.array, dm.embed, dm.final_norm, tok, N, L - N, gk, gv, table, 0, k, "given", None, k_out,
                      v_out, out, ws, out_sel=sel)
    torch.cuda.synchronize()
    shape = (3, N, w.model.n_kv_heads, w.model.head_dim)
    r = oracle.blend_prefill(model, toks, N, host(gk).reshape(shape), host(gv).reshape(shape), table, 0, k, "given",
                             sel.cpu().numpy(), np.float32, 3)
    compare("out", host(out), r.out, "f32")
    compare("K", host(k_out), r.k.reshape(3, L, -1), "f32")
    compare("V", host(v_out), r.v.reshape(3, L, -1), "f32")
    # with every token given, the blend is full prefill (QCFuse §4.1.4 endpoint)
    full = gpu_blend(ctx, dm, toks, N, None, None, None, 0, 0, "all")
    sel_all = torch.arange(N, dtype=torch.int32, device="cuda")
    ws2 = torch.empty(ctx.blend_prefill_workspace_size(N, L - N, N, "given"), dtype=torch.uint8, device="cuda")
    ctx.blend_prefill(dm.array, dm.embed, dm.final_norm, tok, N, L - N, gk, gv, table, 0, N, "given", None, k_out,
                      v_out, out, ws2, out_sel=sel_all)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), full["out"])


def test_invalid_arguments_rejected():
    import torch
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(n_layers=2))
    N, L = w.n_ctx, w.n_total
    model, toks, ctx, dm, gk, gv, table, kb, vb = _setup(w, 2)
    scores = torch.zeros(N, device="cuda")
    ws = torch.empty(ctx.query_scores_workspace_size(N, L - N), dtype=torch.uint8, device="cuda")
    tok = torch.from_numpy(np.asarray(toks, np.int32)).cuda()
    for bad in ([1, 0], [2], [], [0, 0]):
        with pytest.raises(cf.CfError) as e:
            ctx.query_scores(dm.array, dm.embed, tok, N, L - N, kb, vb, bad, scores, ws)
        assert e.value.status == cf.CF_EINVAL
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(cf.CfError) as e:
        ctx.query_scores(dm.array, dm.embed, tok, N, L - N, kb, vb, [0], scores, small)
    assert e.value.status == cf.CF_EWORKSPACE
    k_out = torch.zeros(2, L, ctx.kv_dim, device="cuda")
    with pytest.raises(cf.CfError) as e:  # a given set needs out_sel
        ctx.blend_prefill(dm.array, dm.embed, dm.final_norm, tok, N, L - N, gk, gv, table, 0, 5, "given", None, k_out,
                          k_out.clone(), torch.zeros(L - N, dm.cfg.d_model, device="cuda"),
                          torch.empty(ctx.blend_prefill_workspace_size(N, L - N, 5, "given"), dtype=torch.uint8,
                                      device="cuda"))
    assert e.value.status == cf.CF_EINVAL
