"""GPU parity of QCFuse's compressed token view: chunk anchors (§3.3.1 Eq. 14: Sink and Knorm rules,
r_a = ra_num / ra_den) and anchor-conditioned query probing with critical-layer scoring (§3.3.2
Eq. 15-17, §3.4 Eq. 18 and Eq. 20), cf_key_norms / cf_anchor_positions / cf_query_scores_anchored,
against oracle.key_norms / select_anchors / anchored_query_scores.

Bars: key norms within 1e-5 relative (fp32 sums against fp64); anchors bit-exact when both sides
rank the GPU's own norms; with every context position an anchor, the anchored scores equal the
full-view scores of cf_query_scores (same layers); fp32 models' scores elementwise (1e-4 relative
plus 1e-6 of the largest score); bf16 models under the end-to-end bf16 bars (tests/_gpu.py); the
probe never writes context rows."""
import numpy as np
import pytest

import oracle
import selective_recompute_cf_amd as cf
import synth
from tests._gpu import compare, e2e_bf16, e2e_selection, host, say
from tests.test_gpu_query import _gpu_scores, _setup

pytestmark = pytest.mark.gpu


def _anchored(ctx, dm, toks, N, kb, vb, anchors, layer_set):
    import torch
    U = len(toks) - N
    scores = torch.full((N,), -1.0, dtype=torch.float32, device="cuda")
    a = torch.from_numpy(np.asarray(anchors, np.int32)).cuda() if len(anchors) else None
    ws = torch.empty(ctx.query_scores_anchored_workspace_size(N, U, len(anchors)), dtype=torch.uint8, device="cuda")
    tok = torch.from_numpy(np.asarray(toks, np.int32)).cuda()
    ctx.query_scores_anchored(dm.array, dm.embed, tok, N, U, kb, vb, a, layer_set, scores, ws)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


def _check(w, ly, layer_set, rules=("sink", "knorm"), ratio=(1, 10)):
    import torch
    N = w.n_ctx
    model, toks, ctx, dm, gk, gv, table, kb, vb = _setup(w, ly)
    cfg = model.cfg
    shape = (ly, gk.shape[1], cfg.n_kv_heads, cfg.head_dim)
    ks, vs = host(gk).reshape(shape), host(gv).reshape(shape)
    kst, vst = oracle.stitch(ks, vs, table, N, range(ly), cfg.rope_theta, np.float32, n_total=len(toks))
    norms = torch.zeros(gk.shape[1], dtype=torch.float32, device="cuda")
    ctx.key_norms(gk, norms)
    torch.cuda.synchronize()
    g_norms = norms.cpu().numpy()
    compare("key norms", g_norms, oracle.key_norms(ks), atol=1e-30, rtol=1e-5)
    bf16 = cfg.dtype == "bf16"
    for rule in rules:
        anchors = cf.anchor_positions(rule, table, ratio, g_norms if rule != "sink" else None, gk.shape[1])
        want = np.concatenate([dst + oracle.select_anchors(n, ratio[0], ratio[1], rule, g_norms[row:row + n])
                               for row, _, dst, n in table])
        np.testing.assert_array_equal(anchors, np.sort(want))
        k_ctx_before = host(kb[:, :N])
        g = _anchored(ctx, dm, toks, N, kb, vb, anchors, layer_set)
        np.testing.assert_array_equal(host(kb[:, :N]), k_ctx_before)  # context rows only read
        o = oracle.anchored_query_scores(model, toks, N, kst, vst, anchors, layer_set)
        say(f"anchored scores {w.name} layers={ly} set={layer_set} rule={rule} r_a={ratio[0]}/{ratio[1]}: "
            f"{len(anchors)} anchors")
        assert np.isfinite(g).all()
        if not bf16:
            compare("scores", g, o, atol=1e-6 * float(o.max()), rtol=1e-4)
        else:
            e2e_bf16("scores", g, o, max(layer_set) + 1, 128)
            k = max(1, N // 10)
            e2e_selection(oracle.select_topk(g, k), oracle.select_topk(o, k), o, k, True)
    return model, toks, ctx, dm, kb, vb


def test_tiny_fp32_anchor_rules_and_every_anchor_is_full_view():
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(n_layers=3))
    N = w.n_ctx
    model, toks, ctx, dm, kb, vb = _check(w, 3, [0, 1, 2], ("sink", "knorm", "knorm_low"), (1, 10))
    _check(w, 3, [1], ("sink", "knorm"), (1, 4))
    full = _gpu_scores(ctx, dm, toks, N, kb, vb, [1, 2])
    every = _anchored(ctx, dm, toks, N, kb, vb, np.arange(N), [1, 2])
    compare("every anchor vs full view", every, full, atol=1e-7 * float(full.max()), rtol=1e-6)
    none = _anchored(ctx, dm, toks, N, kb, vb, [], [0])  # r_a = 0: the query alone conditions itself
    assert np.isfinite(none).all() and none.sum() > 0


def test_gqa4_hd128_bf16_critical_layers():
    m = synth.TINY.replace(name="mid", n_layers=4, d_model=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
                           d_ffn=2816, vocab=2000, rope_theta=5e5, dtype="bf16")
    w = synth.Workload("mid-5x200+40", m, 5, 200, 40, 15, 100)
    _check(w, 4, [1, 2])


def test_llama3_8b_shape_three_layers():
    """Llama-3-8B width and request length (6 x 512 + 64), layers 0-2, scored on layers 1 and 2, at
    the page's default anchor ratio r_a = 0.1."""
    _check(synth.WORKLOADS["llama8b"], 3, [1, 2])


def test_invalid_anchor_arguments_rejected():
    import torch
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(n_layers=2))
    N, L = w.n_ctx, w.n_total
    model, toks, ctx, dm, gk, gv, table, kb, vb = _setup(w, 2)
    scores = torch.zeros(N, device="cuda")
    tok = torch.from_numpy(np.asarray(toks, np.int32)).cuda()
    a = torch.arange(0, N, 7, dtype=torch.int32, device="cuda")
    ws = torch.empty(ctx.query_scores_anchored_workspace_size(N, L - N, a.numel()), dtype=torch.uint8, device="cuda")
    for bad in ([1, 0], [2], []):
        with pytest.raises(cf.CfError) as e:
            ctx.query_scores_anchored(dm.array, dm.embed, tok, N, L - N, kb, vb, a, bad, scores, ws)
        assert e.value.status == cf.CF_EINVAL
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(cf.CfError) as e:
        ctx.query_scores_anchored(dm.array, dm.embed, tok, N, L - N, kb, vb, a, [0], scores, small)
    assert e.value.status == cf.CF_EWORKSPACE
    assert ctx.query_scores_anchored_workspace_size(N, L - N, N + 1) == 0
