"""GPU tests of cf_blend_prefill_streamed: the chunk store in pinned host memory, copied layer by
layer on the context's copy stream while earlier layers are recomputed (CacheBlend, "Hiding
Recompute Behind I/O"). The computation is that of cf_blend_prefill, so the bar is bit-for-bit
identity with the resident-store call (which the end-to-end tests hold to the oracle), plus one
oracle comparison here; non-pinned and device stores are rejected."""
import numpy as np
import pytest

import oracle
import selective_recompute_cf_amd as cf
import synth
from selective_recompute_cf_amd.device import DeviceModel
from tests._gpu import compare, context, e2e_bf16, e2e_selection, gpu_blend, gpu_chunk_store, host, say

pytestmark = pytest.mark.gpu


def _setup(w, ly):
    model = synth.Model(w.model)
    chunks, _, toks = synth.request_tokens(w)
    ctx = context(model.cfg.replace(n_layers=ly), max_pos=max(4096, len(toks) + 1))
    dm = DeviceModel(model, n_layers=ly)
    gk, gv, starts = gpu_chunk_store(ctx, dm, chunks)
    table = [(st, 0, st, len(c)) for st, c in zip(starts, chunks)]
    return model, chunks, toks, ctx, dm, gk, gv, table


def _pinned(t):
    import torch
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def _streamed(ctx, dm, toks, N, hk, hv, table, s, k, mode, spans=None):
    import torch
    L = len(toks)
    U = L - N
    dt = hk.dtype
    k_out = torch.zeros(dm.n_layers, L, ctx.kv_dim, dtype=dt, device="cuda")
    v_out = torch.zeros_like(k_out)
    out = torch.zeros(max(U, 1), dm.cfg.d_model, dtype=torch.float32, device="cuda")
    sel = torch.full((max(k, 1),), -1, dtype=torch.int32, device="cuda")
    dev = torch.zeros(max(N, 1), dtype=torch.float32, device="cuda")
    ws = torch.empty(ctx.blend_prefill_streamed_workspace_size(N, U, k, mode, hk.shape[1]), dtype=torch.uint8,
                     device="cuda")
    tok = torch.from_numpy(np.asarray(toks, np.int32)).cuda()
    ctx.blend_prefill_streamed(dm.array, dm.embed, dm.final_norm, tok, N, U, hk, hv, table, s, k, mode, spans, k_out,
                               v_out, out if U else None, ws, out_sel=sel, out_dev=dev)
    return dict(k=k_out, v=v_out, out=out[:U], sel=sel[:k], dev=dev[:N])


def _same(g, want):
    for name in ["k", "v", "out", "sel", "dev"]:
        np.testing.assert_array_equal(host(g[name]) if name not in ("sel",) else g[name].cpu().numpy(),
                                      want[name], err_msg=name)


@pytest.mark.parametrize("dtype,mode,ly,s", [("f32", "token", 3, 1), ("bf16", "token", 7, 1), ("bf16", "doc", 4, 2),
                                             ("bf16", "token", 4, 3)])
def test_streamed_equals_resident_store(dtype, mode, ly, s):
    """Same outputs as cf_blend_prefill; 7 layers reuse each staging slot three times, s = 3 of 4
    streams a single layer."""
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(dtype=dtype, n_layers=ly), mode=mode)
    N = w.n_ctx
    model, chunks, toks, ctx, dm, gk, gv, table = _setup(w, ly)
    k = oracle.budget(N, w.rho_num, w.rho_den)
    spans = [i * w.chunk_len for i in range(w.n_chunks + 1)]
    say(f"streamed tiny {dtype} {mode} layers={ly} s={s} k={k}")
    want = gpu_blend(ctx, dm, toks, N, gk, gv, table, s, k, mode, spans)
    g = _streamed(ctx, dm, toks, N, _pinned(gk), _pinned(gv), table, s, k, mode, spans)
    import torch
    torch.cuda.synchronize()
    _same(g, want)


def test_streamed_llama8b_width_against_oracle():
    """Llama-3-8B width and request length (6 x 512 + 64), 3 layers: identical to the resident
    call, and the query rows within the end-to-end bf16 drift bars against the fp32 oracle."""
    import torch
    w = synth.WORKLOADS["llama8b"]
    N = w.n_ctx
    model, chunks, toks, ctx, dm, gk, gv, table = _setup(w, 3)
    k = oracle.budget(N, w.rho_num, w.rho_den)
    want = gpu_blend(ctx, dm, toks, N, gk, gv, table, 1, k, "token")
    g = _streamed(ctx, dm, toks, N, _pinned(gk), _pinned(gv), table, 1, k, "token")
    torch.cuda.synchronize()
    _same(g, want)
    ks = host(gk).reshape(3, N, w.model.n_kv_heads, w.model.head_dim)
    vs = host(gv).reshape(ks.shape)
    t = [(a, 0, a, len(c)) for a, c in zip(range(0, N, w.chunk_len), chunks)]
    r32 = oracle.blend_prefill(model, toks, N, ks, vs, t, 1, k, "token", None, np.float32, 3)
    e2e_selection(g["sel"].cpu().numpy().astype(np.int64), r32.sel, r32.dev, k, True)
    e2e_bf16("out", host(g["out"]), r32.out, 3, 128)


def test_back_to_back_calls_share_the_slots():
    """Four streamed calls enqueued without a host wait in between (two requests, alternating
    stores and tokens): each call waits on the host for the previous streamed call to finish, and
    its copies come after the previous call's use of the staging slots."""
    import torch
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(dtype="bf16", n_layers=5))
    N = w.n_ctx
    model, chunks, toks, ctx, dm, gk, gv, table = _setup(w, 5)
    _, _, toks2 = synth.request_tokens(w, query_id=0, data_seed=synth.DATA_SEED + 1)
    k = oracle.budget(N, w.rho_num, w.rho_den)
    gk2, gv2 = gk.flip(1).contiguous(), gv.flip(1).contiguous()
    want1 = gpu_blend(ctx, dm, toks, N, gk, gv, table, 1, k, "token")
    want2 = gpu_blend(ctx, dm, toks2, N, gk2, gv2, table, 1, k, "token")
    h1, h2 = (_pinned(gk), _pinned(gv)), (_pinned(gk2), _pinned(gv2))
    torch.cuda.synchronize()
    gs = [_streamed(ctx, dm, t, N, *h, table, 1, k, "token") for t, h in [(toks, h1), (toks2, h2)] * 2]
    torch.cuda.synchronize()
    for i, g in enumerate(gs):
        _same(g, want1 if i % 2 == 0 else want2)


def test_store_must_be_pinned_host_memory():
    import torch
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(n_layers=2))
    N, L = w.n_ctx, w.n_total
    model, chunks, toks, ctx, dm, gk, gv, table = _setup(w, 2)
    k = oracle.budget(N, w.rho_num, w.rho_den)
    for store in [(gk.cpu(), gv.cpu()), (gk, gv)]:  # pageable host memory, device memory
        with pytest.raises(cf.CfError) as e:
            _streamed(ctx, dm, toks, N, store[0], store[1], table, 1, k, "token")
        assert e.value.status == cf.CF_EINVAL and "pinned" in str(e.value)
    # a later launch is not blamed for the failed pointer query
    g = _streamed(ctx, dm, toks, N, _pinned(gk), _pinned(gv), table, 1, k, "token")
    torch.cuda.synchronize()
    _same(g, gpu_blend(ctx, dm, toks, N, gk, gv, table, 1, k, "token"))


@pytest.mark.parametrize("mode", ["ranked", "heads", "token"])
def test_permuted_store_span_modes_no_query(mode):
    """A store that holds one spare chunk (NaN rows that no table entry names) and then the request's
    chunks in reverse order, a request without query rows, and the span modes: the streamed call
    equals the resident call on that store, and both equal the resident call on the store laid out
    in request order (the table's store rows alone decide where each chunk is read)."""
    import torch
    w = synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(dtype="bf16", n_layers=4))
    N, cl = w.n_ctx, w.chunk_len
    model, chunks, toks, ctx, dm, gk, gv, table = _setup(w, 4)
    toks = toks[:N]
    k = oracle.budget(N, w.rho_num, w.rho_den)
    docs = [i * cl for i in range(w.n_chunks + 1)]
    order = np.random.default_rng(9).permutation(w.n_chunks).tolist()
    spans = {"ranked": (docs, order), "heads": docs, "token": None}[mode]
    spare = torch.full((4, cl, ctx.kv_dim), float("nan"), dtype=gk.dtype, device="cuda")
    rev = list(range(w.n_chunks))[::-1]
    pk = torch.cat([spare] + [gk[:, docs[i]:docs[i + 1]] for i in rev], dim=1).contiguous()
    pv = torch.cat([spare] + [gv[:, docs[i]:docs[i + 1]] for i in rev], dim=1).contiguous()
    ptable = [(cl * (1 + rev.index(i)), 0, docs[i], cl) for i in range(w.n_chunks)]
    say(f"permuted store, mode {mode}, k={k}, no query rows")
    want = gpu_blend(ctx, dm, toks, N, gk, gv, table, 1, k, mode, spans)
    res = gpu_blend(ctx, dm, toks, N, pk, pv, ptable, 1, k, mode, spans)
    for name in ["k", "v", "out", "sel", "dev"]:
        np.testing.assert_array_equal(res[name], want[name], err_msg=name)
    assert np.isfinite(want["k"]).all() and want["out"].shape[0] == 0
    g = _streamed(ctx, dm, toks, N, _pinned(pk), _pinned(pv), ptable, 1, k, mode, spans)
    torch.cuda.synchronize()
    _same(g, want)
