"""GPU rolling agent window (Request Order Matters §2.1, §4.1; write-back per §5) against the oracle.

Pins:
* rho = 100%: every step equals the library's own full prefill of the current window bit for bit
  (all rows recomputed, the store is never read) and the oracle's full prefill, whatever the
  history (write-back mode, negative re-position offsets from the second step on);
* pristine mode at rho = 0: every step equals the oracle's direct reuse of the standalone caches;
* write-back: after a step, each document's store slot holds exactly the fused rows of its window
  position, and its base position is that window position;
* step-local parity at 0 < rho < 1: the oracle is fed the GPU's store state before each step
  (caches and base positions) and must reproduce the step: selection bit-exact on the GPU's own
  deviation and overlapping the oracle's selection by the end-to-end selection bar (tests/_gpu.py);
  fused K/V and the normed query rows within the fp32 bound (tiny fp32 model) or the end-to-end
  bf16 drift bars (Llama-3-8B width; the full-size window is held layer by layer to the
  element-wise bar in test_gpu_teacher_forced)."""
import numpy as np
import pytest

import oracle
import synth
from selective_recompute_cf_amd.device import DeviceModel
from selective_recompute_cf_amd.rolling import RollingWindow
from tests._gpu import compare, context, e2e_bf16, e2e_selection, host, overlap, say

pytestmark = pytest.mark.gpu


def _window(model_cfg, n_docs, doc_len, n_query, rho, mode, write_back, ly, steps_hint=4):
    model = synth.Model(model_cfg)
    ctx = context(model_cfg.replace(n_layers=ly), max_pos=4 * (n_docs + steps_hint) * doc_len + 64)
    dm = DeviceModel(model, n_layers=ly)
    v = model_cfg.vocab
    rw = RollingWindow(ctx, dm, n_docs, doc_len, n_query, rho[0], rho[1],
                       doc_tokens=lambda j: synth.doc_tokens(j, doc_len, v),
                       query_tokens=lambda t: synth.query_tokens(t, n_query, v), mode=mode, write_back=write_back)
    return model, ctx, dm, rw


def _oracle_step(model, rw, state, ly):
    """oracle.blend_prefill on the given store state (per window doc: K, V, base)."""
    docs = rw.window()
    ks = np.concatenate([s[0] for s in state], axis=1)
    vs = np.concatenate([s[1] for s in state], axis=1)
    table = [(i * rw.doc_len, s[2], i * rw.doc_len, rw.doc_len) for i, s in enumerate(state)]
    bounds = [i * rw.doc_len for i in range(rw.n_docs + 1)]
    ks = ks.reshape(ks.shape[0], ks.shape[1], model.cfg.n_kv_heads, model.cfg.head_dim)
    vs = vs.reshape(ks.shape)
    return oracle.blend_prefill(model, rw.tokens(), rw.N, ks, vs, table, rw.s, rw.k, rw.mode, bounds, np.float32,
                                ly), table, docs


def test_full_ratio_equals_full_prefill_each_step():
    cfg = synth.TINY.replace(n_layers=2)
    model, ctx, dm, rw = _window(cfg, 4, 64, 16, (100, 100), "doc", True, 2)
    import torch
    for step in range(3):
        table = rw.step()
        say(f"rolling rho=100% step {step}: source positions {[t[1] for t in table]}")
        if step > 0:
            assert [t[1] for t in table][:3] == [64, 128, 192]  # write-back: re-positioned by -64
        toks = torch.from_numpy(rw.tokens(rw.t - 1)).cuda()
        ws = torch.empty(ctx.blend_prefill_workspace_size(rw.N, rw.n_query, rw.N, "all"), dtype=torch.uint8,
                         device="cuda")
        k_full, v_full = torch.zeros_like(rw.k_out), torch.zeros_like(rw.v_out)
        out_full = torch.zeros_like(rw.out)
        ctx.blend_prefill(dm.array, dm.embed, dm.final_norm, toks, rw.N, rw.n_query, None, None, None, 0, 0, "all",
                          None, k_full, v_full, out_full, ws)
        np.testing.assert_array_equal(host(rw.out), host(out_full))
        np.testing.assert_array_equal(host(rw.k_out), host(k_full))
        np.testing.assert_array_equal(host(rw.v_out), host(v_full))
        K, V, out, _ = oracle.full_prefill(model, rw.tokens(rw.t - 1), np.float32, 2)
        compare("out vs oracle full prefill", host(rw.out), out[rw.N:], "f32")
        compare("K vs oracle full prefill", host(rw.k_out), K.reshape(host(rw.k_out).shape), "f32")


def test_pristine_zero_ratio_equals_direct_reuse():
    cfg = synth.TINY.replace(n_layers=2)
    model, ctx, dm, rw = _window(cfg, 4, 64, 16, (0, 100), "doc", False, 2)
    for step in range(2):
        rw.prepare()
        state = rw.store_state()
        table = rw.step()
        assert [t[1] for t in table] == [0, 0, 0, 0]  # pristine: standalone caches at position 0
        ks = np.concatenate([s[0] for s in state], axis=1)
        vs = np.concatenate([s[1] for s in state], axis=1)
        sh = (2, rw.N, cfg.n_kv_heads, cfg.head_dim)
        otab = [(i * rw.doc_len, 0, i * rw.doc_len, rw.doc_len) for i in range(rw.n_docs)]
        K, V, out = oracle.direct_reuse(model, rw.tokens(rw.t - 1), rw.N, ks.reshape(sh), vs.reshape(sh), otab,
                                        np.float32, 2)
        say(f"rolling pristine rho=0 step {step}")
        compare("out vs oracle direct reuse", host(rw.out), out, "f32")
        compare("K[1:] vs oracle direct reuse", host(rw.k_out)[1:, : rw.N],
                K[1:, : rw.N].reshape(host(rw.k_out)[1:, : rw.N].shape), "f32")


def test_write_back_step_local_parity_tiny_fp32():
    cfg = synth.TINY.replace(n_layers=3)
    model, ctx, dm, rw = _window(cfg, 5, 64, 16, (30, 100), "doc", True, 3)
    for step in range(4):
        rw.prepare()
        state = rw.store_state()
        table = rw.step()
        res, otab, docs = _oracle_step(model, rw_view(rw), state, 3)
        assert [t[1] for t in table] == [s[2] for s in state]
        sel = host(rw.sel)[: rw.k].astype(np.int64)
        dev = host(rw.dev)
        bounds = [i * rw.doc_len for i in range(rw.n_docs + 1)]
        np.testing.assert_array_equal(sel, oracle.select_doc_spans(dev, rw.k, bounds))
        ov = overlap(sel, res.sel)
        say(f"rolling write-back step {step}: sources {[t[1] for t in table]}, k={rw.k}, overlap {ov:.3f}")
        assert ov >= 0.99
        compare("out", host(rw.out), res.out, "f32")
        compare("K", host(rw.k_out), res.k.reshape(host(rw.k_out).shape), "f32")
        compare("V", host(rw.v_out), res.v.reshape(host(rw.v_out).shape), "f32")
        # write-back: each document's slot now holds its fused rows; base = its window position
        ks = host(rw.k_store)
        ko = host(rw.k_out)
        for i, j in enumerate(rw.window(rw.t - 1)):
            r0 = rw.slot(j) * rw.doc_len
            np.testing.assert_array_equal(ks[:, r0:r0 + rw.doc_len], ko[:, i * rw.doc_len:(i + 1) * rw.doc_len])
            assert rw.base[j] == i * rw.doc_len


def rw_view(rw):
    """The window as it was for the step just taken (the oracle step reads t - 1)."""
    class V:
        pass
    v = V()
    for name in ("doc_len", "n_docs", "N", "s", "k", "mode"):
        setattr(v, name, getattr(rw, name))
    t = rw.t - 1
    v.window = lambda: rw.window(t)
    v.tokens = lambda: rw.tokens(t)
    return v


def test_write_back_step_local_parity_llama8b_width():
    """Llama-3-8B width (bf16), 4 documents of 512 tokens + 64 query tokens, document-aligned
    top-5%, 2 layers, 3 steps, against the end-to-end bf16 bars."""
    cfg = synth.LLAMA3_8B.replace(n_layers=2)
    model, ctx, dm, rw = _window(cfg, 4, 512, 64, (5, 100), "doc", True, 2)
    for step in range(3):
        rw.prepare()
        state = rw.store_state()
        table = rw.step()
        view = rw_view(rw)
        r32, _, _ = _oracle_step(model, view, state, 2)
        sel = host(rw.sel)[: rw.k].astype(np.int64)
        bounds = [i * rw.doc_len for i in range(rw.n_docs + 1)]
        np.testing.assert_array_equal(sel, oracle.select_doc_spans(host(rw.dev), rw.k, bounds))
        say(f"rolling llama8b-width step {step}: sources {[t[1] for t in table]}, k={rw.k}")
        e2e_selection(sel, r32.sel, r32.dev, rw.k, True, token_mode=False)
        e2e_bf16("out", host(rw.out), r32.out, 2, 128)
        e2e_bf16("dev", host(rw.dev), r32.dev, 2, 128)
