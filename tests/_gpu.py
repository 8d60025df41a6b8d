"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare with the oracle."""
import sys

import numpy as np

import selective_recompute_cf_amd as cf
from selective_recompute_cf_amd.device import DeviceModel, to_device

TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 1e-2)}  # (atol, rtol): |gpu - ref| <= atol + rtol |ref|


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def compare(name, gpu, ref, dtype=None, atol=None, rtol=None, frac=1.0):
    """Elementwise |gpu - ref| <= atol + rtol |ref| (all elements, or at least `frac` of them)."""
    if atol is None:
        atol, rtol = TOL[dtype]
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    bad = err > atol + rtol * np.abs(ref)
    nrel = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-30))
    stats = dict(max_abs=float(err.max(initial=0.0)), norm_rel=nrel, bad=int(bad.sum()), n=int(err.size))
    say(f"  {name}: max_abs={stats['max_abs']:.3e} norm_rel={nrel:.3e} out_of_tol={stats['bad']}/{stats['n']}")
    assert np.isfinite(gpu).all(), f"{name}: non-finite GPU values"
    assert bad.sum() <= (1.0 - frac) * err.size, f"{name}: {int(bad.sum())} of {err.size} outside tolerance"
    return stats


def overlap(a, b) -> float:
    a, b = set(np.asarray(a).tolist()), set(np.asarray(b).tolist())
    return 1.0 if not a and not b else len(a & b) / max(len(a), 1)


# End-to-end comparisons of bf16 models against the fp32 oracle. The element-wise bf16 bar is held
# layer by layer with the GPU's own inputs (tests/_tf.py); over several stacked layers the bf16
# result drifts from fp32 by the arithmetic itself: one bf16 layer at Llama-3-8B width lands about
# 9e-3 norm-wise from fp32 (measured on the oracle's pinned bf16-arithmetic mode and on the GPU, layer
# by layer), the residual stream is renormalised before every layer, so the per-layer departures
# add rather than compound. Allowance: 2e-2 per layer norm-wise (about twice the per-layer floor),
# and no head-sized chunk of any row further than 4x that (a wrong row, head or tile is caught).
E2E_DRIFT_PER_LAYER = 2e-2
E2E_CHUNK_FACTOR = 4.0
E2E_OVERLAP = 0.97      # end-to-end selection overlap floor for bf16 models
NEAR_TIE = 0.05         # a selection disagreement must sit within 5% of the oracle's k-th deviation


def nrel(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


def e2e_bf16(name, gpu, ref, n_layers, chunk):
    """Norm-wise drift of a bf16 end-to-end result from the fp32 oracle within n_layers x 2e-2, and
    every `chunk`-element piece of it (one head of one row, say) within 4x that relative to the
    larger of its own norm and the tensor's typical chunk norm. The element-wise misses at the
    (2e-2, 1e-2) bar are printed, not asserted (see the module comment above)."""
    g = np.asarray(gpu, np.float64).reshape(-1)
    r = np.asarray(ref, np.float64).reshape(-1)
    assert g.shape == r.shape, name
    assert np.isfinite(g).all(), f"{name}: non-finite GPU values"
    bound = E2E_DRIFT_PER_LAYER * n_layers
    e = nrel(g, r)
    n_c = g.size // chunk
    gc, rc = g[: n_c * chunk].reshape(n_c, chunk), r[: n_c * chunk].reshape(n_c, chunk)
    typ = np.linalg.norm(r) / np.sqrt(max(n_c, 1))
    den = np.maximum(np.linalg.norm(rc, axis=1), typ)
    worst = float((np.linalg.norm(gc - rc, axis=1) / den).max(initial=0.0))
    miss = int((np.abs(g - r) > 2e-2 + 1e-2 * np.abs(r)).sum())
    say(f"  {name}: norm_rel={e:.3e} (bound {bound:.3e}); worst {chunk}-chunk {worst:.3e} "
        f"(bound {E2E_CHUNK_FACTOR * bound:.3e}); elements outside (2e-2, 1e-2): {miss}/{g.size}")
    assert e <= bound, f"{name}: norm-wise drift {e:.3e} > {bound:.3e}"
    assert worst <= E2E_CHUNK_FACTOR * bound, f"{name}: a {chunk}-element chunk is {worst:.3e} off"
    return dict(norm_rel=e, worst_chunk=worst, misses=miss, n=int(g.size))


def e2e_selection(sel_gpu, sel_ref, dev_ref, k, bf16, token_mode=True):
    """End-to-end selection against the fp32 oracle's: overlap >= 99% for fp32 models, >= 97% for
    bf16 ones (the benchmark spec's 99% is asserted layer-local in tests/_tf.py, where both sides rank the
    same inputs); in token mode every token that only one side selected must be a near tie, its
    oracle deviation within 5% of the oracle's k-th largest."""
    ov = overlap(sel_gpu, sel_ref)
    floor = E2E_OVERLAP if bf16 else 0.99
    diff = np.setxor1d(np.asarray(sel_gpu, np.int64), np.asarray(sel_ref, np.int64))
    msg = f"  selection overlap with the fp32 oracle {ov:.4f} ({k} tokens, {len(diff) // 2} swapped)"
    if token_mode and k > 0 and len(diff):
        d = np.asarray(dev_ref, np.float64).copy()
        d[np.isnan(d)] = np.inf
        t = float(np.sort(d)[-k])
        far = float(np.abs(d[diff] - t).max() / t)
        msg += f"; largest disagreement {far:.3%} of the k-th deviation"
        assert far <= NEAR_TIE, f"a disagreement is {far:.2%} away from the k-th deviation, not a near tie"
    say(msg)
    assert ov >= floor, f"overlap {ov:.4f} < {floor}"
    return ov


def context(cfg, max_pos, dtype=None):
    return cf.Context.from_model_cfg(cfg, max_pos=max_pos, dtype=dtype)


def gpu_chunk_store(ctx, dm, chunks):
    """Standalone prefill of every chunk at positions 0.. (mode "all"), written straight into one
    store [Ly, rows, kvd]. Returns (k_store, v_store, chunk rows)."""
    import torch
    Ly, kvd = dm.n_layers, ctx.kv_dim
    rows = sum(len(c) for c in chunks)
    dt = torch_dtype(dm.dtype)
    ks = torch.zeros(Ly, rows, kvd, dtype=dt, device="cuda")
    vs = torch.zeros_like(ks)
    r0, starts = 0, []
    for c in chunks:
        n = len(c)
        tok = torch.from_numpy(np.asarray(c, np.int32)).cuda()
        ws = torch.empty(ctx.blend_prefill_workspace_size(n, 0, n, "all"), dtype=torch.uint8, device="cuda")
        ctx.blend_prefill(dm.array, dm.embed, dm.final_norm, tok, n, 0, None, None, None, 0, 0, "all", None,
                          ks[:, r0:], vs[:, r0:], None, ws, out_layer_stride=rows * kvd)
        starts.append(r0)
        r0 += n
    return ks, vs, starts


def gpu_blend(ctx, dm, tokens, N, k_store, v_store, table, sel_layer, k, mode, spans=None):
    """One cf_blend_prefill call; returns dict of host arrays."""
    import torch
    L = len(tokens)
    U = L - N
    Ly, kvd, d = dm.n_layers, ctx.kv_dim, dm.cfg.d_model
    dt = torch_dtype(dm.dtype)
    k_out = torch.zeros(Ly, L, kvd, dtype=dt, device="cuda")
    v_out = torch.zeros_like(k_out)
    out = torch.zeros(max(U, 1), d, dtype=torch.float32, device="cuda")
    kk = N if mode == "all" else k
    sel = torch.full((max(kk, 1),), -1, dtype=torch.int32, device="cuda")
    dev = torch.zeros(max(N, 1), dtype=torch.float32, device="cuda")
    ws = torch.empty(ctx.blend_prefill_workspace_size(N, U, kk, mode), dtype=torch.uint8, device="cuda")
    tok = torch.from_numpy(np.asarray(tokens, np.int32)).cuda()
    ctx.blend_prefill(dm.array, dm.embed, dm.final_norm, tok, N, U, k_store, v_store, table, sel_layer, k, mode,
                      spans, k_out, v_out, out if U else None, ws, out_sel=None if mode == "all" else sel,
                      out_dev=None if mode == "all" else dev)
    torch.cuda.synchronize()
    r = dict(k=host(k_out), v=host(v_out), out=host(out)[:U])
    if mode != "all":
        r["sel"] = sel.cpu().numpy()[:k]
        r["dev"] = dev.cpu().numpy()[:N]
    return r


def gpu_blend_gradual(ctx, dm, tokens, N, k_store, v_store, table, sel_layer, k_sched):
    """One cf_blend_prefill_gradual call; returns dict of host arrays, with "sets" (one array per
    layer from sel_layer on) and "layer_devs" (one per layer strictly between sel_layer and the last)."""
    import torch
    L = len(tokens)
    U = L - N
    Ly, kvd, d = dm.n_layers, ctx.kv_dim, dm.cfg.d_model
    dt = torch_dtype(dm.dtype)
    k_sched = [int(x) for x in k_sched]
    k_out = torch.zeros(Ly, L, kvd, dtype=dt, device="cuda")
    v_out = torch.zeros_like(k_out)
    out = torch.zeros(max(U, 1), d, dtype=torch.float32, device="cuda")
    sets = torch.full((max(sum(k_sched), 1),), -1, dtype=torch.int32, device="cuda")
    n_dev = N + sum(k_sched[1:-1])
    devs = torch.full((max(n_dev, 1),), -1.0, dtype=torch.float32, device="cuda")
    ws = torch.empty(ctx.blend_prefill_gradual_workspace_size(N, U, sel_layer, k_sched), dtype=torch.uint8,
                     device="cuda")
    tok = torch.from_numpy(np.asarray(tokens, np.int32)).cuda()
    ctx.blend_prefill_gradual(dm.array, dm.embed, dm.final_norm, tok, N, U, k_store, v_store, table, sel_layer,
                              k_sched, k_out, v_out, out if U else None, ws, out_sets=sets, out_devs=devs)
    torch.cuda.synchronize()
    s_host, d_host = sets.cpu().numpy(), devs.cpu().numpy()
    r = dict(k=host(k_out), v=host(v_out), out=host(out)[:U], dev=d_host[:N], sets=[], layer_devs=[])
    o = 0
    for kk in k_sched:
        r["sets"].append(s_host[o:o + kk])
        o += kk
    o = N
    for kk in k_sched[1:-1]:
        r["layer_devs"].append(d_host[o:o + kk])
        o += kk
    return r
