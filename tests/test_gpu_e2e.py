"""End-to-end GPU parity of cf_blend_prefill against the oracle on seeded random-init models and
token streams: chunk caches from standalone prefill at position 0, re-position + stitch, layer-0
full recompute, deviation and selection on layer 1, selective recompute of the remaining layers.

Bars: fused K/V and the final normed query rows within (2e-2, 1e-2) for bf16 and (1e-4, 1e-4)
for fp32; the GPU selection equals the oracle's selection run on the GPU's own deviation array
(bit-exact) and overlaps the oracle's end-to-end selection by >= 99%."""
import numpy as np
import pytest

import oracle
import synth
from selective_recompute_cf_amd.device import DeviceModel
from tests._gpu import compare, context, gpu_blend, gpu_chunk_store, host, overlap, say

pytestmark = pytest.mark.gpu


def _workload(w: synth.Workload, n_layers=None):
    model = synth.Model(w.model)
    chunks, q, toks = synth.request_tokens(w)
    return model, chunks, toks, (w.model.n_layers if n_layers is None else n_layers)


def _oracle_store(model, chunks, ly):
    ks, vs, table, row = [], [], [], 0
    for c in chunks:
        k, v = oracle.chunk_prefill(model, c, np.float32, ly)
        ks.append(k)
        vs.append(v)
        table.append((row, 0, row, len(c)))
        row += len(c)
    return np.concatenate(ks, 1), np.concatenate(vs, 1), table


def _run(w, n_layers=None, mode=None, k=None, check_store=True):
    model, chunks, toks, ly = _workload(w, n_layers)
    cfg = model.cfg
    mode = mode or w.mode
    N = w.n_ctx
    k = oracle.budget(N, w.rho_num, w.rho_den) if k is None else k
    say(f"e2e {w.name} layers={ly} mode={mode} k={k}")
    ctx = context(cfg, max_pos=max(4096, len(toks) + 1))
    dm = DeviceModel(model, n_layers=ly)
    gk, gv, starts = gpu_chunk_store(ctx, dm, chunks)
    table = [(s, 0, s, len(c)) for s, c in zip(starts, chunks)]
    spans = [i * w.chunk_len for i in range(w.n_chunks + 1)]
    g = gpu_blend(ctx, dm, toks, N, gk, gv, table, w.sel_layer, k, mode, spans)
    oks, ovs, otab = _oracle_store(model, chunks, ly)
    if check_store:
        compare("store K", host(gk), oks.reshape(gk.shape), cfg.dtype)
        compare("store V", host(gv), ovs.reshape(gv.shape), cfg.dtype)
    r = oracle.blend_prefill(model, toks, N, oks, ovs, otab, w.sel_layer, k, mode, spans, np.float32, ly)
    return model, toks, g, r, ctx, dm, (gk, gv, table, spans)


def _check(w, g, r, dtype):
    L = w.n_total
    compare("dev", g["dev"], r.dev, atol=1e-3 * float(np.median(r.dev)) + 1e-12, rtol=5e-2 if dtype == "bf16" else 1e-3)
    sel_from_gpu_dev = (oracle.select_topk(g["dev"], len(g["sel"])) if w.mode == "token" else
                        oracle.select_doc_spans(g["dev"], len(g["sel"]), [i * w.chunk_len for i in range(w.n_chunks + 1)]))
    np.testing.assert_array_equal(g["sel"], sel_from_gpu_dev)
    ov = overlap(g["sel"], r.sel)
    say(f"  selection overlap {ov:.4f} ({len(r.sel)} tokens)")
    assert ov >= 0.99
    compare("out", g["out"], r.out, dtype)
    compare("K", g["k"], r.k.reshape(g["k"].shape), dtype)
    compare("V", g["v"], r.v.reshape(g["v"].shape), dtype)


def test_tiny_fp32_workload():
    """C1 as configured: fp32, 2 layers, 4x128 + 32, top-15% selected on layer 1."""
    w = synth.WORKLOADS["tiny"]
    model, toks, g, r, *_ = _run(w)
    assert len(g["sel"]) == 76
    _check(w, g, r, "f32")


def test_tiny_bf16_three_layers_doc_spans():
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(dtype="bf16", n_layers=3), mode="doc",
                                        rho_num=30, rho_den=100)
    model, toks, g, r, *_ = _run(w)
    _check(w, g, r, "bf16")


@pytest.mark.parametrize("mode", ["token", "doc"])
def test_gqa4_hd128_bf16(mode):
    m = synth.TINY.replace(name="mid", n_layers=3, d_model=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
                           d_ffn=2816, vocab=2000, rope_theta=5e5, dtype="bf16")
    w = synth.Workload("mid-5x200+40", m, 5, 200, 40, 15, 100, mode=mode)
    model, toks, g, r, *_ = _run(w)
    _check(w, g, r, "bf16")


def test_qknorm_bf16():
    m = synth.TINY.replace(name="mid-qk", n_layers=3, d_model=512, n_q_heads=8, n_kv_heads=1, head_dim=64,
                           d_ffn=1408, vocab=2000, rope_theta=1e6, rms_eps=1e-6, qk_norm=True, dtype="bf16")
    w = synth.Workload("mid-qk-4x256+64", m, 4, 256, 64, 30, 100)
    model, toks, g, r, *_ = _run(w)
    _check(w, g, r, "bf16")


def test_endpoints_full_ratio_and_direct_reuse():
    """rho = 100% reproduces the library's own full prefill exactly (same kernels, same rows) and
    the oracle's full prefill within tolerance; rho = 0 reproduces the oracle's direct reuse."""
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(dtype="bf16", n_layers=3))
    N, L = w.n_ctx, w.n_total
    model, toks, g, r, ctx, dm, (gk, gv, table, spans) = _run(w, k=N)
    full = gpu_blend(ctx, dm, toks, N, None, None, None, 0, 0, "all")
    np.testing.assert_array_equal(g["out"], full["out"])
    np.testing.assert_array_equal(g["k"], full["k"])
    K, V, out, _ = oracle.full_prefill(model, toks, np.float32, 3)
    compare("full out", full["out"], out[N:], "bf16")
    compare("full K", full["k"], K.reshape(full["k"].shape), "bf16")
    g0 = gpu_blend(ctx, dm, toks, N, gk, gv, table, 1, 0, "token")
    oks, ovs, otab = _oracle_store(model, synth.request_tokens(w)[0], 3)
    Kd, Vd, outd = oracle.direct_reuse(model, toks, N, oks, ovs, otab, np.float32, 3)
    compare("reuse out", g0["out"], outd, "bf16")
    compare("reuse K[1:]", g0["k"][1:, :N], Kd[1:, :N].reshape(g0["k"][1:, :N].shape), "bf16")


def test_first_chunk_never_selected_and_empty_query():
    """The first chunk has no preceding context, so its deviation is ~0 and it is never picked
    while k <= N - |c_1|; U = 0 (no query rows) is a valid request."""
    w = synth.WORKLOADS["tiny"].replace(n_query=0, model=synth.TINY.replace(dtype="bf16"))
    model, toks, g, r, *_ = _run(w, check_store=False)
    assert g["out"].shape[0] == 0
    assert np.all(g["sel"] >= w.chunk_len)
    assert np.max(g["dev"][: w.chunk_len]) < 1e-3 * np.median(g["dev"][w.chunk_len:])


def test_llama3_8b_shape_reduced_depth():
    """Llama-3-8B shape at full width and full request length (6 x 512 + 64, k = 460), 3 layers."""
    w = synth.WORKLOADS["llama8b"]
    model, toks, g, r, *_ = _run(w, n_layers=3, check_store=False)
    assert len(g["sel"]) == 460
    _check(w, g, r, "bf16")
