"""Teacher-forced, per-layer, element-wise parity at the workloads' full sizes (see tests/_tf.py
for the procedure and the bars). These are the sizes at which the library runs its real launch
plans: 256x256 GEMM blocks on the 3136-10368-row full layers, 128x192 blocks with split-K on the
selected rows, K loops of 4096-28672, multi-piece sparse-query attention at L = 3136-16640.

* Llama-3-8B shape, 6 x 512 + 64 tokens, top-15% on layer 1: all 32 layers checked, every row.
* Qwen3-8B shape (qk-norm), 10 x 1024 + 128, 30%: all 36 layers run, layers 0, 1, 2, 18 and 35
  checked (the layer outputs on a seeded sample of 384 rows; K/V of every recomputed row).
* Rolling window, Llama-3-8B shape, 20 x 512 + 64 at 5% with document-aligned spans: one
  write-back step on the GPU, then the next step (documents 1..20: the retained ones re-positioned
  by -512 from the GPU's written-back store, document 20 prefilled at position 0) checked at
  layers 0, 1, 2 and 31.
* Llama-3-70B shape, 16 x 1024 + 256, 10%, at full width and length with 4 layers (the depth
  does not change any launch plan): every layer checked (layer outputs on 384 sampled rows).
* Smaller shapes with ragged tiles (GQA 4 at head_dim 128, qk-norm at head_dim 64 with one kv head,
  document-aligned spans on the tiny model in bf16): every layer, every row."""
import numpy as np
import pytest

import oracle
import synth
from selective_recompute_cf_amd.device import DeviceModel
from tests._gpu import context, gpu_chunk_store, say
from tests._tf import Keep, teacher_forced

pytestmark = pytest.mark.gpu


def _request(w, depth, check, sample):
    cfg = w.model.replace(n_layers=depth)
    chunks, _, toks = synth.request_tokens(w)
    N, L = w.n_ctx, w.n_total
    k = oracle.budget(N, w.rho_num, w.rho_den)
    say(f"teacher-forced {w.name}: {depth} layers, N={N} L={L} k={k}, checked layers {sorted(check)}")
    keep = Keep(synth.Model(cfg, cache_layers=False), check)
    ctx = context(cfg, max_pos=L + 1)
    dm = DeviceModel(keep)
    gk, gv, starts = gpu_chunk_store(ctx, dm, chunks)
    table = [(s0, 0, s0, len(c)) for s0, c in zip(starts, chunks)]
    spans = [i * w.chunk_len for i in range(w.n_chunks + 1)] if w.mode == "doc" else None
    return teacher_forced(ctx, dm, keep, toks, N, k, w.mode, spans, gk, gv, table, w.sel_layer, check, sample)


def test_llama3_8b_every_layer():
    w = synth.WORKLOADS["llama8b"]
    res = _request(w, 32, range(32), None)
    assert sorted(l for l in res if isinstance(l, int)) == list(range(32))


def test_qwen3_8b_sampled_layers():
    w = synth.WORKLOADS["qwen8b"]
    _request(w, 36, [0, 1, 2, 18, 35], 384)


def test_llama3_70b_full_width_and_length():
    w = synth.WORKLOADS["llama70b"]
    _request(w, 4, range(4), 384)


def test_rolling_window_write_back_step():
    import torch
    from selective_recompute_cf_amd.rolling import RollingWindow
    w = synth.WORKLOADS["rolling"]
    cfg = w.model
    check = [0, 1, 2, 31]
    keep = Keep(synth.Model(cfg, cache_layers=False), check)
    ctx = context(cfg, max_pos=w.n_total + 4 * w.chunk_len + 1)
    dm = DeviceModel(keep)
    rw = RollingWindow(ctx, dm, w.n_chunks, w.chunk_len, w.n_query, w.rho_num, w.rho_den,
                       lambda j: synth.doc_tokens(j, w.chunk_len, cfg.vocab),
                       lambda r: synth.query_tokens(r, w.n_query, cfg.vocab), mode="doc")
    rw.step()  # step 0: every document standalone; fused K/V and positions written back
    rw.prepare()  # step 1: document 0 leaves, document 20 is prefilled into its slot
    docs = rw.window()
    table = rw.chunk_table(docs)
    deltas = [dst - src for _, src, dst, _ in table]
    assert deltas[:-1] == [-w.chunk_len] * (w.n_chunks - 1) and deltas[-1] == (w.n_chunks - 1) * w.chunk_len
    toks = rw.tokens()
    spans = [i * w.chunk_len for i in range(w.n_chunks + 1)]
    say(f"teacher-forced {w.name} step 1: N={rw.N} L={rw.L} k={rw.k}, re-position offsets {sorted(set(deltas))}")
    torch.cuda.synchronize()
    teacher_forced(ctx, dm, keep, toks, rw.N, rw.k, "doc", spans, rw.k_store, rw.v_store, table, 1, check, 384)


MID = {
    "gqa4-hd128": synth.Workload("mid-5x200+40", synth.TINY.replace(
        name="mid", n_layers=3, d_model=1024, n_q_heads=8, n_kv_heads=2, head_dim=128, d_ffn=2816, vocab=2000,
        rope_theta=5e5, dtype="bf16"), 5, 200, 40, 15, 100),
    "qknorm-hd64": synth.Workload("mid-qk-4x256+64", synth.TINY.replace(
        name="mid-qk", n_layers=3, d_model=512, n_q_heads=8, n_kv_heads=1, head_dim=64, d_ffn=1408, vocab=2000,
        rope_theta=1e6, rms_eps=1e-6, qk_norm=True, dtype="bf16"), 4, 256, 64, 30, 100),
    "tiny-bf16-doc": synth.WORKLOADS["tiny"].replace(model=synth.TINY.replace(dtype="bf16", n_layers=3), mode="doc",
                                                      rho_num=30, rho_den=100),
}


@pytest.mark.parametrize("name", list(MID))
def test_small_shapes_every_layer(name):
    w = MID[name]
    _request(w, w.model.n_layers, range(w.model.n_layers), None)
