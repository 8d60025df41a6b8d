#!/usr/bin/env python3
"""Benchmark of blended prefill (CacheBlend-style selective KV recompute) on one MI355X.

One step = one cf_blend_prefill call over one request of the Llama-3-8B-shaped random-init bf16
model (32 layers, d 4096, 32/8 heads, FFN 14336): 6 chunks x 512 tokens + a 64-token query,
chunk caches from standalone prefill at position 0 (prepared before timing, as offline cache
preparation is outside TTFT in QCFuse §4.1.4), RoPE re-position + stitch, layer 0 recomputed on
every row, deviation and token top-15% on layer 1, selective recompute of layers 1..31.
Weights, chunk store, tokens, outputs and workspace are resident in HBM before timing.

Prints ONE JSON line: context tokens/s (N x steps / wall time), the roofline of the dominant
kernel (the projection GEMM, timed live with HIP events on its stream), the other kernels'
fractions, the speedup over the library's own full prefill at each recompute ratio, and the CPU
oracle's throughput on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--profile-steps", type=int, default=5)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--full-compare", action="store_true",
                    help="with --no-sweep: still time full prefill of the same request, for the step's speedup")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--store-cache", default=None,
                    help="load the chunk store from this file if it exists, else build it and save it there")
    ap.add_argument("--prepare-only", action="store_true", help="build (and save) the chunk store, then exit")
    ap.add_argument("--store", choices=["device", "host"], default="device",
                    help="where the chunk store lives for the timed step: resident in HBM (cf_blend_prefill), or "
                         "in pinned host memory, streamed in per layer (cf_blend_prefill_streamed; PCIe-inclusive)")
    ap.add_argument("--sweeps", action="store_true",
                    help="only run the kernel sweeps beyond the request's own sizes (re-position over all layers, "
                         "deviation up to GB sizes, top-k up to 256M, measured copy and MFMA peaks), print them as one "
                         "JSON line and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (the reference for the FETCH_SIZE / "
                         "WRITE_SIZE counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); the path has no multi-GPU mode",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import selective_recompute_cf_amd as cf
    from selective_recompute_cf_amd import roofline as rl
    from selective_recompute_cf_amd.device import DeviceModel

    assert torch.cuda.is_available(), "bench needs a GPU"
    torch.cuda.set_device(0)
    if args.sweeps:
        print(json.dumps(kernel_sweeps()), flush=True)
        return
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {n} bytes 3 times")
        return
    w = synth.WORKLOADS[args.workload]
    cfg = w.model
    N, U, L = w.n_ctx, w.n_query, w.n_total
    k = cf.budget(N, w.rho_num, w.rho_den)
    kvd, Ly = cfg.kv_dim, cfg.n_layers
    log(f"[bench] workload {w.name}: N={N} U={U} k={k} layers={Ly}; generating and uploading weights")
    t0 = time.time()
    dm = DeviceModel(synth.Model(cfg, cache_layers=False),
                     on_layer=lambda l: log(f"[bench]   layer {l + 1} of {Ly} on GPU") if (l + 1) % 10 == 0 else None)
    log(f"[bench] weights on GPU ({dm.weight_bytes() / 1e9:.1f} GB) in {time.time() - t0:.1f}s")
    ctx = cf.Context.from_model_cfg(cfg, max_pos=L + 1)
    chunks, _, toks = synth.request_tokens(w)
    tok_dev = torch.from_numpy(toks).cuda()
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    table = [(i * w.chunk_len, 0, i * w.chunk_len, w.chunk_len) for i in range(w.n_chunks)]
    spans = [i * w.chunk_len for i in range(w.n_chunks + 1)]

    # ---------------------------------------------------------------- chunk store (untimed)
    if args.store_cache and os.path.exists(args.store_cache):
        st = torch.load(args.store_cache, weights_only=True)
        ks, vs = st["k"].cuda(), st["v"].cuda()
        log(f"[bench] chunk store loaded from {args.store_cache}")
    else:
        ks = torch.zeros(Ly, N, kvd, dtype=dt, device="cuda")
        vs = torch.zeros_like(ks)
        for i, c in enumerate(chunks):
            r0 = i * w.chunk_len
            n = len(c)
            wsc = torch.empty(ctx.blend_prefill_workspace_size(n, 0, n, "all"), dtype=torch.uint8, device="cuda")
            ctx.blend_prefill(dm.array, dm.embed, dm.final_norm, torch.from_numpy(c).cuda(), n, 0, None, None,
                              None, 0, 0, "all", None, ks[:, r0:], vs[:, r0:], None, wsc, out_layer_stride=N * kvd)
        torch.cuda.synchronize()
        if args.store_cache:
            torch.save({"k": ks.cpu(), "v": vs.cpu()}, args.store_cache)
            log(f"[bench] chunk store saved to {args.store_cache}")
    if args.prepare_only:
        return

    sweep = [0, 5, 10, 15, 30, 50, 100]
    k_of = {r: cf.budget(N, r, 100) for r in sweep}
    gradual = gradual_schedules(w)
    ws_bytes = max([ctx.blend_prefill_workspace_size(N, U, kk, w.mode) for kk in list(k_of.values()) + [k]] +
                   [ctx.blend_prefill_workspace_size(N, U, N, "all")] +
                   [ctx.blend_prefill_gradual_workspace_size(N, U, w.sel_layer, g) for g in gradual.values()])
    if args.store == "host":
        ws_bytes = max(ws_bytes, ctx.blend_prefill_streamed_workspace_size(N, U, k, w.mode, N))
        hks = torch.empty(ks.shape, dtype=ks.dtype, pin_memory=True)
        hvs = torch.empty(vs.shape, dtype=vs.dtype, pin_memory=True)
        hks.copy_(ks)
        hvs.copy_(vs)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    k_out = torch.zeros(Ly, L, kvd, dtype=dt, device="cuda")
    v_out = torch.zeros_like(k_out)
    out = torch.zeros(max(U, 1), cfg.d_model, dtype=torch.float32, device="cuda")
    sel = torch.zeros(N, dtype=torch.int32, device="cuda")

    def blend(kk=k):
        ctx.blend_prefill(dm.array, dm.embed, dm.final_norm, tok_dev, N, U, ks, vs, table, w.sel_layer, kk, w.mode,
                          spans, k_out, v_out, out if U else None, ws, out_sel=sel)

    def blend_host_store():
        ctx.blend_prefill_streamed(dm.array, dm.embed, dm.final_norm, tok_dev, N, U, hks, hvs, table, w.sel_layer, k,
                                   w.mode, spans, k_out, v_out, out if U else None, ws, out_sel=sel)

    step = blend_host_store if args.store == "host" else blend

    def full():
        ctx.blend_prefill(dm.array, dm.embed, dm.final_norm, tok_dev, N, U, None, None, None, 0, 0, "all", None,
                          k_out, v_out, out if U else None, ws)

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        t_start = time.perf_counter()
        ev[0].record()
        for i in range(steps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
        return wall, per

    # ---------------------------------------------------------------- headline timing
    log(f"[bench] timing {args.steps} steps after {args.warmup} warm-up steps")
    wall, per = timed(step, args.steps, args.warmup)
    value = N * args.steps / wall
    ms_step = wall / args.steps * 1e3
    sel_host = sel[:k].cpu().numpy()
    log(f"[bench] {ms_step:.3f} ms/step (median event {statistics.median(per):.3f} ms) -> {value:.0f} ctx tokens/s")

    # ---------------------------------------------------------------- per-kernel timing (HIP events)
    P = args.profile_steps
    cf.profile_enable(True)
    for _ in range(P):
        step()
    torch.cuda.synchronize()
    rep = cf.profile_report()
    cf.profile_enable(False)
    shape = rl.shape_of(cfg)
    work = rl.blend_step_work(shape, N, U, k, w.sel_layer, sel_host)
    kernels = {}
    for name, (launches, ms) in sorted(rep.items()):
        ent = {"launches_per_step": launches / P, "us_per_launch": ms / launches * 1e3 if launches else None,
               "ms_per_step": ms / P}
        if name in work and ms > 0:
            if name.startswith("gemm/") or name == "attention":
                ach = work[name] / (ms / P / 1e3) / 1e12
                ent.update(achieved=ach, unit="TFLOP/s", peak=rl.BF16_PEAK_TFLOPS, frac=ach / rl.BF16_PEAK_TFLOPS,
                           algorithmic_flops_per_step=work[name])
            else:
                ach = work[name] / (ms / P / 1e3) / 1e9
                ent.update(achieved=ach, unit="GB/s", peak=rl.HBM_PEAK_GBS, frac=ach / rl.HBM_PEAK_GBS,
                           algorithmic_bytes_per_step=work[name])
        if name == "reposition" and "frac" in ent:
            ent["note"] = ("in situ, on the request's own store; the all-layer sweep (bench.py --sweeps) gives the "
                           "kernel's rate from a cold HBM start, 66-69% of 8 TB/s")
        kernels[name] = ent
    # gather + norm + K/V scatter (H4/H6) and the deviation (H2) against the bytes the method must move;
    # the bytes the current unfused kernels move are reported beside them
    groups = {"row steps H4/H6 (rmsnorm_rows + reduce_resid_norm + splitk_reduce + qkv_post)":
              (("rmsnorm_rows", "reduce_resid_norm", "splitk_reduce", "qkv_post"), "h4h6_rows",
               ("unfused:rows", "unfused:qkv_post")),
              "deviation H2 (qkv_post/dev, fused numerator)": (("qkv_post/dev",), "h2_deviation",
                                                                ("unfused:deviation",))}
    for label, (names, key, unfused) in groups.items():
        g_ms = sum(v[1] for n, v in rep.items() if n in names)
        if g_ms <= 0:
            continue
        ach = work[key] / (g_ms / P / 1e3) / 1e9
        ent = {"ms_per_step": g_ms / P, "achieved": ach, "unit": "GB/s", "peak": rl.HBM_PEAK_GBS,
               "frac": ach / rl.HBM_PEAK_GBS, "algorithmic_bytes_per_step": work[key]}
        if unfused:
            moved = sum(work[u] for u in unfused)
            ent.update(bytes_moved_by_unfused_kernels_per_step=moved,
                       unfused_rate_GBs=moved / (g_ms / P / 1e3) / 1e9)
        kernels[label] = ent
    g_launch = sum(v[0] for n, v in rep.items() if n.startswith("gemm/"))
    g_ms = sum(v[1] for n, v in rep.items() if n.startswith("gemm/"))
    g_flops = rl.gemm_flops(work) * P
    g_ach = g_flops / (g_ms / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(g_ach, 2), "peak": rl.BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g_ach / rl.BF16_PEAK_TFLOPS, 4), "traffic": None,
                "kernel": "gemm_bf16_dtl (projection GEMMs, all block heights)",
                "avg_launch_us": round(g_ms / g_launch * 1e3, 2),
                "flops_per_launch": g_flops / g_launch, "launches_per_step": g_launch / P}
    roofline.update(gemm_traffic(rl.gemm_bytes(work) / (g_launch / P), args.workload))
    log(f"[bench] gemm: {g_ach:.1f} TFLOP/s ({roofline['frac'] * 100:.1f}% of bf16 peak), "
        f"{roofline['avg_launch_us']} us/launch")

    # ---------------------------------------------------------------- speedup over full prefill per ratio
    sweep_res = None
    if not args.no_sweep:
        _, pf = timed(full, 5, 2)
        t_full = statistics.median(pf)
        sweep_res = {"full_prefill_ms": round(t_full, 3), "ratios": {}}
        for r in sweep:
            _, pb = timed(lambda: blend(k_of[r]), 5, 2)
            tb = statistics.median(pb)
            sweep_res["ratios"][f"{r}%"] = {"k": k_of[r], "blend_ms": round(tb, 3), "speedup": round(t_full / tb, 3)}
        log(f"[bench] full prefill {t_full:.2f} ms; speedups " +
            ", ".join(f"{r}: {v['speedup']}x" for r, v in sweep_res["ratios"].items()))
        sweep_res["gradual"] = {}
        for name, sch in gradual.items():
            def run_g(sch=sch):
                ctx.blend_prefill_gradual(dm.array, dm.embed, dm.final_norm, tok_dev, N, U, ks, vs, table,
                                          w.sel_layer, sch, k_out, v_out, out if U else None, ws)
            _, pg = timed(run_g, 5, 2)
            tg = statistics.median(pg)
            sweep_res["gradual"][name] = {"schedule": sch, "rows_recomputed": sum(sch), "blend_ms": round(tg, 3),
                                          "speedup": round(t_full / tg, 3)}
            log(f"[bench] gradual {name}: {tg:.2f} ms ({t_full / tg:.2f}x), schedule {sch[:4]}..{sch[-1]}")
        sweep_res["streamed"] = streamed_pipeline(ctx, dm, w, tok_dev, ks, vs, table, spans, k_out, v_out, out,
                                                  k_of, sweep_res, timed)
        sweep_res["query_aware"] = query_aware(ctx, dm, w, tok_dev, ks, vs, table, k_out, v_out, out, k, sweep_res,
                                               timed)
        if args.workload == "llama8b":
            sweep_res["rolling_window"] = rolling_steps(dm)
    elif args.full_compare:
        # full prefill of the same request next to the timed step only (the whole sweep is long at 70B size)
        _, pf = timed(full, 2, 1)
        t_full, t_step = statistics.median(pf), statistics.median(per)
        sweep_res = {"full_prefill_ms": round(t_full, 3),
                     "ratios": {f"{w.rho_num * 100 // w.rho_den}%": {"k": k, "blend_ms": round(t_step, 3),
                                                                     "speedup": round(t_full / t_step, 3)}}}
        log(f"[bench] full prefill {t_full:.2f} ms; blended step {t_step:.2f} ms: {t_full / t_step:.2f}x")

    # ---------------------------------------------------------------- CPU oracle baseline (bounded sample)
    cpu, north = None, None
    if not args.no_cpu_baseline:
        blend()  # the timed request again (deterministic): the sweeps above reused the output buffers
        torch.cuda.synchronize()
        gpu_res = dict(sel=sel[:k].cpu().numpy(), k=k_out.float().cpu().numpy(), v=v_out.float().cpu().numpy(),
                       out=out[:U].cpu().numpy())
        cpu, north = cpu_baseline(w, k, gpu_res)

    line = {
        "metric": "blended-prefill context tokens/s per GPU at r=15%",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "median_step_ms_events": round(statistics.median(per), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded uniform-random tokens, N(0,0.02) random-init weights)",
        "config": {"workload": w.name, "dims": cfg.name, "layers": Ly, "n_ctx": N, "n_query": U,
                   "chunks": f"{w.n_chunks}x{w.chunk_len}", "recompute_ratio": f"{w.rho_num}/{w.rho_den}",
                   "k": k, "selection": w.mode, "selection_layer": w.sel_layer,
                   "chunk_store": "HBM" if args.store == "device" else "pinned host memory, streamed per layer",
                   "all_tokens_per_s": round((N + U) * args.steps / wall, 1)},
        "roofline": roofline,
        "kernels": kernels,
        "speedup_vs_full_prefill": sweep_res,
        "cpu_baseline": cpu,
        "north_star_parity": north,
    }
    print(json.dumps(line), flush=True)


def streamed_pipeline(ctx, dm, w, tok_dev, ks, vs, table, spans, k_out, v_out, out, k_of, sweep_res, timed):
    """The store in pinned host memory, loaded layer by layer under the recompute
    (cf_blend_prefill_streamed), and the loading controller's ratio (CacheBlend, "Hiding Recompute
    Behind I/O"): per-layer load time of one store layer, per-layer recompute time of one
    cf_blend_layer pass at each ratio, r = max(r_load, 15%), and the streamed prefill against the
    resident-store prefill at 15% and at the controller's r."""
    import torch
    import selective_recompute_cf_amd as cf
    cfg = dm.cfg
    N, U, L = w.n_ctx, w.n_query, w.n_total
    kvd = cfg.n_kv_heads * cfg.head_dim
    hk = torch.empty(ks.shape, dtype=ks.dtype, pin_memory=True)
    hv = torch.empty(vs.shape, dtype=vs.dtype, pin_memory=True)
    hk.copy_(ks)
    hv.copy_(vs)
    stage = torch.empty(2, N, kvd, dtype=ks.dtype, device="cuda")

    def load_layer():
        stage[0].copy_(hk[w.sel_layer], non_blocking=True)
        stage[1].copy_(hv[w.sel_layer], non_blocking=True)

    _, pl = timed(load_layer, 10, 3)
    t_load = statistics.median(pl)
    layer_bytes = 2 * N * kvd * ks.element_size()
    # one selective layer pass at each ratio (selected rows: the first k context rows + the query)
    hidden = (0.1 * torch.randn(L, cfg.d_model, device="cuda")).float()
    kc, vc = k_out[w.sel_layer].clone(), v_out[w.sel_layer].clone()
    t_layer = {}
    for r, kk in k_of.items():
        sel = torch.cat([torch.arange(kk), torch.arange(N, L)]).int().cuda()
        lws = torch.empty(ctx.blend_layer_workspace_size(L, kk + U), dtype=torch.uint8, device="cuda")
        _, pr = timed(lambda: ctx.blend_layer(dm.array[w.sel_layer], hidden, kc, vc, sel, lws), 5, 2)
        t_layer[(r, 100)] = statistics.median(pr)
    r_ctl = cf.loading_controller(t_load, t_layer, (w.rho_num, w.rho_den))
    res = {"h2d_GBs": round(layer_bytes / (t_load / 1e3) / 1e9, 1), "load_ms_per_layer": round(t_load, 4),
           "recompute_ms_per_layer": {f"{a}%": round(t, 4) for (a, _), t in t_layer.items()},
           "controller_ratio": f"{r_ctl[0]}/{r_ctl[1]}", "runs": {}}
    ws = torch.empty(max(ctx.blend_prefill_streamed_workspace_size(N, U, cf.budget(N, *q), w.mode, N)
                         for q in [(w.rho_num, w.rho_den), r_ctl]), dtype=torch.uint8, device="cuda")
    for q in dict.fromkeys([(w.rho_num, w.rho_den), r_ctl]):
        kk = cf.budget(N, *q)

        def run_s(kk=kk):
            ctx.blend_prefill_streamed(dm.array, dm.embed, dm.final_norm, tok_dev, N, U, hk, hv, table, w.sel_layer,
                                       kk, w.mode, spans, k_out, v_out, out if U else None, ws)

        _, ps = timed(run_s, 5, 2)
        t_s = statistics.median(ps)
        resident = sweep_res["ratios"].get(f"{q[0] * 100 // q[1]}%", {}).get("blend_ms") if q[1] == 100 else None
        res["runs"][f"{q[0]}/{q[1]}"] = {"k": kk, "streamed_ms": round(t_s, 3), "resident_ms": resident,
                                         "load_ms_all_layers": round(t_load * (cfg.n_layers - w.sel_layer), 3)}
    log(f"[bench] streamed store: {res['h2d_GBs']} GB/s host->device, {t_load:.3f} ms load per layer; "
        f"controller r = {res['controller_ratio']}; runs {res['runs']}")
    return res


def rolling_steps(dm, steps=50):
    """The rolling-agent window at the same model shape, as configured (Request Order Matters §4.1: 20
    documents of 512 tokens, a fresh 64-token query per step, 5%, 50 steps): time per step of the blend
    and the write-back, token top-k against document-aligned spans. Arriving documents are prefilled
    before each timed step (the arrival path), as the window driver does."""
    import torch
    import synth
    import selective_recompute_cf_amd as cf
    from selective_recompute_cf_amd.rolling import RollingWindow
    w = synth.WORKLOADS["rolling"]
    cfg = dm.cfg
    ctx = cf.Context.from_model_cfg(cfg, max_pos=w.n_total + w.chunk_len * (steps + 4) + 1)
    res = {"workload": w.name}
    for mode in ("token", "doc"):
        rw = RollingWindow(ctx, dm, w.n_chunks, w.chunk_len, w.n_query, w.rho_num, w.rho_den,
                           lambda j: synth.doc_tokens(j, w.chunk_len, cfg.vocab),
                           lambda r: synth.query_tokens(r, w.n_query, cfg.vocab), mode=mode)
        times = []
        for i in range(steps + 1):
            rw.prepare()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rw.step()
            e1.record()
            torch.cuda.synchronize()
            if i:  # the first step warms up
                times.append(e0.elapsed_time(e1))
        times.sort()
        res[mode] = {"k": rw.k, "steps": len(times), "step_ms": round(statistics.median(times), 3),
                     "step_ms_p95": round(times[int(0.95 * (len(times) - 1))], 3),
                     "step_ms_mean": round(statistics.mean(times), 3),
                     "context_tokens_per_s": round(rw.N / (statistics.median(times) / 1e3), 1)}
        del rw
    log(f"[bench] rolling window: {res}")
    return res


def query_aware(ctx, dm, w, tok_dev, ks, vs, table, k_out, v_out, out, k, sweep_res, timed):
    """QCFuse's query-aware selection (§3.2.1 Eq. 10 over all layers, Eq. 20 over three middle
    layers) on the same request: the probe of the query rows over the stitched cache with the
    per-layer attention mass (cf_query_scores), or over the chunk anchors only (§3.3, Sink or Knorm
    anchors at r_a = 0.1, cf_query_scores_anchored), the top-k of the scores, and the blend of that
    set from layer 0 (CF_SEL_GIVEN); times per step and the selection's share of the total."""
    import torch
    import selective_recompute_cf_amd as cf
    cfg = dm.cfg
    N, U, L, Ly = w.n_ctx, w.n_query, w.n_total, cfg.n_layers
    kvd = cfg.n_kv_heads * cfg.head_dim
    kb = torch.empty(Ly, L, kvd, dtype=ks.dtype, device="cuda")
    vb = torch.empty_like(kb)
    ctx.rope_reposition(ks, vs, kb, vb, table, 0, Ly)
    scores = torch.empty(N, dtype=torch.float32, device="cuda")
    sel = torch.empty(max(k, 1), dtype=torch.int32, device="cuda")
    wsq = torch.empty(ctx.query_scores_workspace_size(N, U), dtype=torch.uint8, device="cuda")
    wst = torch.empty(max(ctx.blend_prefill_workspace_size(N, U, k, "given"), cf.topk_workspace_size(N, "token"), 1),
                      dtype=torch.uint8, device="cuda")
    mid = Ly // 2
    res = {}
    # QCFuse's chunk anchors at r_a = 0.1 (§3.3.3): Sink, and Knorm from the store's key norms (offline, untimed)
    norms = torch.empty(ks.shape[1], dtype=torch.float32, device="cuda")
    ctx.key_norms(ks, norms)
    anchors = {"sink": cf.anchor_positions("sink", table, (1, 10)),
               "knorm": cf.anchor_positions("knorm", table, (1, 10), norms.cpu().numpy(), ks.shape[1])}
    anchors = {r: torch.tensor(a, dtype=torch.int32, device="cuda") for r, a in anchors.items()}
    wsa = torch.empty(max(ctx.query_scores_anchored_workspace_size(N, U, int(a.numel())) for a in anchors.values()),
                      dtype=torch.uint8, device="cuda")
    cases = [("all_layers", list(range(Ly)), None), ("three_middle_layers", [mid - 1, mid, mid + 1], None)]
    cases += [(f"anchors_{r}_r0.1_three_middle_layers", [mid - 1, mid, mid + 1], r) for r in anchors]
    cases += [(f"anchors_{r}_r0.1_all_layers", list(range(Ly)), r) for r in anchors]
    for name, lset, rule in cases:
        def select(lset=lset, rule=rule):
            if rule is None:
                ctx.query_scores(dm.array, dm.embed, tok_dev, N, U, kb, vb, lset, scores, wsq)
            else:
                ctx.query_scores_anchored(dm.array, dm.embed, tok_dev, N, U, kb, vb, anchors[rule], lset, scores, wsa)
            cf.topk_select(scores, k, sel, "token", None, wst)

        def blend_given():
            ctx.blend_prefill(dm.array, dm.embed, dm.final_norm, tok_dev, N, U, ks, vs, table, 0, k, "given", None,
                              k_out, v_out, out if U else None, wst, out_sel=sel)

        _, p_sel = timed(select, 5, 2)
        _, p_bl = timed(blend_given, 5, 2)
        t_sel, t_bl = statistics.median(p_sel), statistics.median(p_bl)
        res[name] = {"layers": len(lset), "anchors": None if rule is None else int(anchors[rule].numel()),
                     "select_ms": round(t_sel, 3), "blend_ms": round(t_bl, 3),
                     "total_ms": round(t_sel + t_bl, 3), "selection_share": round(t_sel / (t_sel + t_bl), 3),
                     "speedup_vs_full_prefill": round(sweep_res["full_prefill_ms"] / (t_sel + t_bl), 3)}
    log(f"[bench] query-aware: {res}")
    return res


def _event_ms(fn, reps=5, warmup=2):
    """Median HIP-event time (ms) of fn() on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return statistics.median(ts)


def kernel_sweeps():
    """The HBM-bound steps at sizes beyond one request, through the C ABI, against the published
    peaks and the peaks measured here (a plain device copy; the library's MFMA loop)."""
    import torch
    import synth
    import selective_recompute_cf_amd as cf
    from selective_recompute_cf_amd import roofline as rl

    res = {}
    # measured peaks
    n = 4 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    t = _event_ms(lambda: cf.copy_loop(a, b))
    copy_gbs = 2 * n / (t / 1e3) / 1e9
    del a, b
    out = torch.empty(64 * 256 * 256, dtype=torch.float32, device="cuda")
    fl = {}
    t = _event_ms(lambda: fl.__setitem__("f", cf.mfma_loop(out, 4, 20000)))
    mfma_tf = fl["f"] / (t / 1e3) / 1e12
    res["measured_peaks"] = {"hbm_copy_GBs": round(copy_gbs, 1), "copy": "4 GiB streaming copy (cf_copy_loop), read + write",
                             "mfma_bf16_TFs": round(mfma_tf, 1),
                             "mfma": "32x32x16 bf16 MFMA loop, 16 waves per CU, no memory traffic",
                             "spec_hbm_GBs": rl.HBM_PEAK_GBS, "spec_bf16_TFs": rl.BF16_PEAK_TFLOPS}
    log(f"[sweeps] copy {copy_gbs:.0f} GB/s, MFMA loop {mfma_tf:.0f} TF/s")

    def frac(gbs):
        return {"achieved_GBs": round(gbs, 1), "frac_spec": round(gbs / rl.HBM_PEAK_GBS, 4),
                "frac_measured": round(gbs / copy_gbs, 4)}

    # H1: re-position + stitch of every layer after the selection layer, in one call
    rows = []
    for name, Ly, N, kvd in (("llama3-8b 6x512, layers 1..31", 31, 3072, 1024),
                             ("llama3-70b 16x1024, layers 1..79", 79, 16384, 1024)):
        cfg = synth.LLAMA3_8B.replace(n_layers=Ly)
        ctx = cf.Context.from_model_cfg(cfg, max_pos=2 * N + 1)
        ks = torch.randn(Ly, N, kvd, device="cuda").to(torch.bfloat16)
        vs = torch.randn_like(ks)
        kb, vb = torch.empty_like(ks), torch.empty_like(vs)
        chunk = 512 if N == 3072 else 1024
        tab = [(i * chunk, 0, i * chunk, chunk) for i in range(N // chunk)]
        t = _event_ms(lambda: ctx.rope_reposition(ks, vs, kb, vb, tab, 0, Ly))
        byt = rl.kv_bytes_per_layer(N, 8, 128, 2) * 2 * Ly
        rows.append({"case": name, "bytes": byt, "ms": round(t, 4), **frac(byt / (t / 1e3) / 1e9)})
        del ks, vs, kb, vb
        ctx.close()
    res["reposition"] = rows
    log(f"[sweeps] reposition {[r['achieved_GBs'] for r in rows]} GB/s")

    # H2: deviation sum_c (K_new - K_ref)^2 over kvd = 1024, bf16 inputs
    rows = []
    for name, n_tok in (("one layer, 3072 rows", 3072), ("one layer, 16384 rows", 16384),
                        ("all 32 layers of 3072 rows", 32 * 3072), ("1M rows", 1 << 20)):
        kn = torch.randn(n_tok, 1024, device="cuda").to(torch.bfloat16)
        kr = torch.randn_like(kn)
        dev = torch.empty(n_tok, dtype=torch.float32, device="cuda")
        t = _event_ms(lambda: cf.kv_deviation(kn, kr, dev))
        byt = 2 * n_tok * 1024 * 2 + 4 * n_tok
        rows.append({"case": name, "bytes": byt, "ms": round(t, 4), **frac(byt / (t / 1e3) / 1e9)})
        del kn, kr, dev
    res["deviation"] = rows
    log(f"[sweeps] deviation {[r['achieved_GBs'] for r in rows]} GB/s")

    # H3: token top-k (exact), k = 15% of n
    rows = []
    for n_tok in (3072, 16384, 16 << 20, 64 << 20, 256 << 20):
        d = torch.rand(n_tok, device="cuda")
        k = cf.budget(n_tok, 15, 100)
        o = torch.empty(k, dtype=torch.int32, device="cuda")
        ws = torch.empty(max(cf.topk_workspace_size(n_tok, "token"), 1), dtype=torch.uint8, device="cuda")
        t = _event_ms(lambda: cf.topk_select(d, k, o, "token", None, ws))
        byt = 4 * n_tok + 4 * k
        rows.append({"n": n_tok, "k": k, "us": round(t * 1e3, 1), "bytes": byt, **frac(byt / (t / 1e3) / 1e9)})
        del d, o, ws
    res["topk_token"] = rows
    log(f"[sweeps] topk {[(r['n'], r['us']) for r in rows]}")
    return {"sweeps": res}


def gradual_schedules(w):
    """Gradual filtering schedules timed next to the step (the set narrows layer by layer toward the
    workload's ratio r): 20% or 30% on the selection layer, kept 90% or 80% per layer, where that
    start is above r; token selection only."""
    import selective_recompute_cf_amd as cf
    Ly = w.model.n_layers
    if w.mode != "token" or w.sel_layer >= Ly:
        return {}
    return {f"{a}%->{w.rho_num}% x{b}/10": cf.gradual_schedule(w.n_ctx, Ly - w.sel_layer, (a, 100), (b, 10),
                                                               (w.rho_num, w.rho_den))
            for a, b in [(20, 9), (30, 8)] if a * w.rho_den > 100 * w.rho_num}


def gemm_traffic(alg_bytes_per_launch, workload="llama8b"):
    """HBM bytes per GEMM launch from the committed FETCH_SIZE / WRITE_SIZE counter summary of the
    Llama-3-8B-shaped workload, if that is the workload and the GEMM sources have not changed since
    the counters were taken (else traffic stays null)."""
    from selective_recompute_cf_amd import profiles
    path = os.path.join(ROOT, "profiles", "gemm_bf16_dtl_llama3-8b_hbm_traffic.json")
    out = {"traffic_unit": "bytes per launch (HBM fetch + write, rocprofv3 counters)",
           "algorithmic_bytes_per_launch": round(alg_bytes_per_launch)}
    if workload != "llama8b":
        out["traffic_note"] = "counters were taken on the Llama-3-8B-shaped workload only"
        return out
    try:
        with open(path) as f:
            t = json.load(f)
    except OSError:
        out["traffic_note"] = "no counter summary"
        return out
    if t.get("source_sha256") != profiles.sources_sha256():
        out["traffic_note"] = "GEMM sources changed since the counters were taken"
        return out
    out["traffic"] = round(t["traffic_bytes_per_launch"])
    return out


def cpu_info():
    """The host CPU as /proc/cpuinfo names it (model string, family / model / stepping, sockets)."""
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    continue
                key, val = (x.strip() for x in line.split(":", 1))
                if key in ("model name", "cpu family", "model", "stepping", "cpu MHz", "physical id") and key not in info:
                    info[key] = val
                if key == "physical id":
                    info.setdefault("sockets", set()).add(val)
    except OSError:
        pass
    if "sockets" in info:
        info["sockets"] = len(info["sockets"])
    info.pop("physical id", None)
    return info


def cpu_baseline(w, k, gpu=None, runs=2):
    """The oracle (numpy, as written) on the host cores: blended prefill of the same request at full
    depth, width and length, timed over `runs` runs (the chunk caches are the oracle's own standalone
    prefills, computed untimed first, as the GPU's chunk store is). With the GPU's result of the same
    request, also the spec comparison of the two end to end: selection overlap and, for the
    final query rows and the fused K/V (rows whose selection agrees), the norm-wise error and the share
    of elements outside max-abs 2e-2 / relative 1e-2."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    import oracle
    import synth

    cores = len(os.sched_getaffinity(0))
    cfg = w.model
    N, L = w.n_ctx, w.n_total
    log(f"[bench] CPU oracle on {cores} host threads: chunk caches at full depth (untimed)")
    ctx_mgr = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        model = synth.Model(cfg)
        chunks, _, toks = synth.request_tokens(w)
        t0 = time.perf_counter()
        ks, vs, tab, row = [], [], [], 0
        for c in chunks:
            a, b = oracle.chunk_prefill(model, c, np.float32)
            ks.append(a)
            vs.append(b)
            tab.append((row, 0, row, len(c)))
            row += len(c)
        ks, vs = np.concatenate(ks, 1), np.concatenate(vs, 1)
        t_chunks = time.perf_counter() - t0
        spans = [i * w.chunk_len for i in range(w.n_chunks + 1)]
        ts, res = [], None
        for _ in range(runs):
            t0 = time.perf_counter()
            res = oracle.blend_prefill(model, toks, N, ks, vs, tab, w.sel_layer, k, w.mode, spans, np.float32)
            ts.append(time.perf_counter() - t0)
        t_blend = statistics.median(ts)
    finally:
        if ctx_mgr is not None:
            ctx_mgr.__exit__(None, None, None)
    log(f"[bench] CPU oracle: chunk caches {t_chunks:.1f}s; blended prefill {t_blend:.2f}s (median of {runs})")
    cpu = {"value": round(N / t_blend, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": (f"{w.name}: the whole request, oracle blend_prefill at full depth ({cfg.n_layers} layers), width "
                      f"and length, median of {runs} runs = {t_blend:.2f}s per request; the oracle's own chunk caches "
                      f"prepared untimed first ({t_chunks:.1f}s)"),
           "cpu": cpu_info()}
    if gpu is None:
        return cpu, None

    def stats(g, r):
        g, r = np.asarray(g, np.float64), np.asarray(r, np.float64)
        bad = np.abs(g - r) > 2e-2 + 1e-2 * np.abs(r)
        return {"norm_rel": float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-30)),
                "max_abs": float(np.abs(g - r).max(initial=0.0)), "outside_bar_frac": float(bad.mean()),
                "n": int(g.size)}

    agree = np.zeros(L, bool)
    a_g, a_o = np.zeros(N, bool), np.zeros(N, bool)
    a_g[gpu["sel"]] = True
    a_o[res.sel] = True
    agree[:N] = a_g == a_o
    agree[N:] = True
    shape = gpu["k"].shape
    ov = len(set(gpu["sel"].tolist()) & set(res.sel.tolist())) / max(k, 1)
    north = {"reference": f"fp32 oracle end to end at full depth ({cfg.n_layers} layers), same request",
             "bar": "selection overlap >= 0.99; max-abs 2e-2 / relative 1e-2 per element",
             "selection_overlap": round(ov, 4),
             "out": stats(gpu["out"], res.out),
             "K": stats(gpu["k"][:, agree], res.k.reshape(shape)[:, agree]),
             "V": stats(gpu["v"][:, agree], res.v.reshape(shape)[:, agree]),
             "layer_by_layer": "K/V of every layer within the bar element-wise and the selection overlap 1.0 when "
                               "the oracle is fed the GPU's own layer inputs (tests/test_gpu_teacher_forced.py)"}
    log(f"[bench] north-star parity vs the fp32 oracle: overlap {ov:.4f}; out {north['out']}; K {north['K']}")

    # The same request through the oracle in its bf16-arithmetic mode (bf16 rounding at the points where
    # the GPU path stores bf16: normed rows, Q, K/V, softmax weights, attention output, SwiGLU
    # activation; chunk caches prefilled the same way), untimed: how far bf16 arithmetic alone drifts
    # from the fp32 oracle at full depth, beside the GPU's own distance from each.
    t0 = time.perf_counter()
    ctx_mgr = threadpool_limits(limits=cores) if threadpool_limits else None
    try:
        kb, vb = [], []
        for c in chunks:
            a, b = oracle.chunk_prefill(model, c, np.float32, bf16_ops=True)
            kb.append(a)
            vb.append(b)
        kb, vb = np.concatenate(kb, 1), np.concatenate(vb, 1)
        rb = oracle.blend_prefill(model, toks, N, kb, vb, tab, w.sel_layer, k, w.mode, spans, np.float32,
                                  bf16_ops=True)
    finally:
        if ctx_mgr is not None:
            ctx_mgr.__exit__(None, None, None)

    def vs(sel_a, out_a, k_a, v_a, sel_b, out_b, k_b, v_b):
        both = np.zeros(L, bool)
        x, y = np.zeros(N, bool), np.zeros(N, bool)
        x[sel_a] = True
        y[sel_b] = True
        both[:N] = x == y
        both[N:] = True
        return {"selection_overlap": round(len(set(np.asarray(sel_a).tolist()) & set(np.asarray(sel_b).tolist())) /
                                           max(k, 1), 4),
                "out": stats(out_a, out_b), "K": stats(k_a[:, both], k_b[:, both]),
                "V": stats(v_a[:, both], v_b[:, both])}

    north["bf16_arithmetic_oracle_vs_fp32_oracle"] = vs(rb.sel, rb.out, rb.k.reshape(shape), rb.v.reshape(shape),
                                                        res.sel, res.out, res.k.reshape(shape), res.v.reshape(shape))
    north["gpu_vs_bf16_arithmetic_oracle"] = vs(gpu["sel"], gpu["out"], gpu["k"], gpu["v"],
                                                rb.sel, rb.out, rb.k.reshape(shape), rb.v.reshape(shape))
    log(f"[bench] bf16-arithmetic oracle ({time.perf_counter() - t0:.1f}s) vs the fp32 oracle: "
        f"{north['bf16_arithmetic_oracle_vs_fp32_oracle']}; GPU vs it: {north['gpu_vs_bf16_arithmetic_oracle']}")
    return cpu, north


if __name__ == "__main__":
    main()
