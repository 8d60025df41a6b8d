"""GPU parity of one blended layer (cf_blend_layer) against the oracle's layer on the same inputs:
gather + norm + QKV on the selected rows, qk-norm + RoPE, scatter into the cache, sparse-query
causal attention over the whole cache, O projection, SwiGLU MLP, rows written back
(CacheBlend, "Selective Recompute Without Skipping"; QCFuse Eq. 7). Selections: all rows, scattered
rows + a tail, one row, and rows clustered at the start or at the end (which load the attention's
key pieces very unevenly)."""
import numpy as np
import pytest

import oracle
import synth
from selective_recompute_cf_amd.device import DeviceModel
from tests._gpu import compare, context, host, say, torch_dtype

pytestmark = pytest.mark.gpu

SHAPES = {
    # name: model shape (1 layer used), L
    "tiny-f32": (synth.TINY.replace(n_layers=1), 200),
    "tiny-bf16-ragged-ffn": (synth.TINY.replace(n_layers=1, dtype="bf16"), 200),
    "gqa4-hd128-bf16": (synth.TINY.replace(n_layers=1, d_model=1024, n_q_heads=8, n_kv_heads=2, head_dim=128,
                                           d_ffn=2816, dtype="bf16"), 333),
    "gqa8-hd64-bf16": (synth.TINY.replace(n_layers=1, d_model=1024, n_q_heads=16, n_kv_heads=2, head_dim=64,
                                          d_ffn=1536, dtype="bf16"), 257),
    "qknorm-bf16": (synth.TINY.replace(n_layers=1, d_model=512, n_q_heads=4, n_kv_heads=1, head_dim=128,
                                       d_ffn=1408, qk_norm=True, rms_eps=1e-6, dtype="bf16"), 300),
}


class _Host:
    def __init__(self, cfg):
        self.cfg = cfg
        self._w = synth.layer_weights(cfg, 0, 3)
        self.embed = np.zeros((8, cfg.d_model), np.float32)
        self.final_norm = np.ones(cfg.d_model, np.float32)

    def layer(self, l):
        return self._w


def _sel(L, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "all":
        return np.arange(L)
    if kind == "sparse":  # scattered context rows + a contiguous tail (the query rows)
        body = np.sort(rng.choice(L - 16, size=(L - 16) // 6, replace=False))
        return np.concatenate([body, np.arange(L - 16, L)])
    if kind == "one":
        return np.array([L // 2])
    if kind == "early":  # clustered at the start + the tail: one query tile sees many more keys
        return np.concatenate([np.arange((L - 16) // 6), np.arange(L - 16, L)])
    if kind == "late":  # clustered at the end: every query tile sees nearly all keys
        return np.arange(L - L // 5, L)
    raise ValueError(kind)


@pytest.mark.parametrize("shape", list(SHAPES))
@pytest.mark.parametrize("kind", ["all", "sparse", "one", "early", "late"])
def test_blend_layer_matches_oracle(shape, kind):
    import torch
    cfg, L = SHAPES[shape]
    say(f"blend_layer shape={shape} sel={kind} L={L}")
    hostm = _Host(cfg)
    dm = DeviceModel(hostm, with_embed=False)
    ctx = context(cfg, max_pos=4096)
    kvd, d = cfg.kv_dim, cfg.d_model
    h = synth.normal_array([9, 1], (L, d))
    kc = synth.normal_array([9, 2], (L, cfg.n_kv_heads, cfg.head_dim))
    vc = synth.normal_array([9, 3], (L, cfg.n_kv_heads, cfg.head_dim))
    if cfg.dtype == "bf16":
        kc, vc = synth.bf16_round(kc), synth.bf16_round(vc)
    sel = _sel(L, kind, 4)
    dt = torch_dtype(cfg.dtype)
    th = torch.from_numpy(h).cuda()
    tk = torch.from_numpy(kc.reshape(L, kvd)).to(dt).cuda()
    tv = torch.from_numpy(vc.reshape(L, kvd)).to(dt).cuda()
    ts = torch.from_numpy(sel.astype(np.int32)).cuda()
    ws = torch.empty(ctx.blend_layer_workspace_size(L, len(sel)), dtype=torch.uint8, device="cuda")
    ctx.blend_layer(dm.array[0], th, tk, tv, ts, ws)
    torch.cuda.synchronize()

    kref, vref = kc.astype(np.float32).copy(), vc.astype(np.float32).copy()
    href = h.copy()
    href[sel] = oracle.layer_rows(cfg, hostm.layer(0), h[sel], sel, kref, vref, np.float32)
    gh = host(th)
    other = np.setdiff1d(np.arange(L), sel)
    compare("hidden[sel]", gh[sel], href[sel], cfg.dtype)
    np.testing.assert_array_equal(gh[other], h[other])
    gk = host(tk).reshape(L, cfg.n_kv_heads, cfg.head_dim)
    gv = host(tv).reshape(L, cfg.n_kv_heads, cfg.head_dim)
    compare("K[sel]", gk[sel], kref[sel], cfg.dtype)
    compare("V[sel]", gv[sel], vref[sel], cfg.dtype)
    np.testing.assert_array_equal(gk[other], kc[other])
    np.testing.assert_array_equal(gv[other], vc[other])
