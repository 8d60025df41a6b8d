"""Oracle decoder: RMSNorm, RoPE, causal GQA attention, SwiGLU, full prefill.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The decoder is the plain pre-norm Llama/Qwen3 shape that the workloads name (RMSNorm,
RoPE, SwiGLU FFN, grouped-query attention, optional per-head RMS qk-norm). The pages fix
only the parts that matter to blending: QCFuse §2.1.1 Eq. 2 (full prefill materialises
every layer's K/V for the whole context under the current order and positions) and the
per-layer pass of CacheBlend's "Selective Recompute Without Skipping" (projections, attention
over the cache, MLP). Everything here is numpy; matrix products are the only library
primitive used, and no step is fused or reordered.

Conventions: matrices are [out, in] (y = x @ W.T); RoPE rotates the pair (x_j, x_{j+hd/2})
by the angle pos * theta^(-2j/hd); attention lets a query at position p see cache rows t <= p;
query head h reads kv head h // (Hq / Hkv).

Arithmetic: everything runs in ``ft`` (fp32 by default) on the model's stored weights and
embeddings (bf16-valued for bf16 models). With ``bf16_ops=True`` the oracle instead follows the
arithmetic of a BF16 serving stack (QCFuse §4.1.1 serves BF16): every operand of a matrix
product (the normed rows, Q, the softmax weights, the attention output, the SwiGLU activation;
weights and K/V are bf16 already) and every K/V cache entry is rounded to bf16
(round-to-nearest-even) while sums stay fp32. That mode measures how far bf16 arithmetic itself
lands from the fp32 result, which calibrates the tolerance of bf16 comparisons.
"""
from __future__ import annotations

import numpy as np


def bf16_round(x):
    """Nearest bfloat16 value of each fp32 element (ties to even), returned as fp32: add
    0x7FFF plus the lowest kept bit to the fp32 bit pattern and clear the low 16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    keep_lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + keep_lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def rounding(cfg, bf16_ops=None):
    """The rounding applied to matrix-product operands and K/V cache entries: bf16 when
    ``bf16_ops`` is true (and the model is bf16), none otherwise (see above)."""
    use = bool(bf16_ops) and getattr(cfg, "dtype", "f32") == "bf16"
    return bf16_round if use else None


def _r(rnd, x, ft):
    return x if rnd is None else np.asarray(rnd(x), dtype=ft)


def rms_norm(x, gain, eps, ft=np.float32):
    """x / sqrt(mean(x^2) + eps) * gain over the last axis, computed in ``ft``."""
    x = np.asarray(x, dtype=ft)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + ft(eps))) * np.asarray(gain, dtype=ft)


def rope_angles(pos, head_dim, theta):
    """cos and sin of pos * omega_j, omega_j = theta^(-2j/hd), j < hd/2, all in fp64.
    pos: array of (possibly negative) integer offsets. Returns two [len(pos), hd/2] arrays."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    omega = np.power(np.float64(theta), -2.0 * j / np.float64(head_dim))
    ang = np.asarray(pos, dtype=np.float64).reshape(-1, 1) * omega.reshape(1, -1)
    return np.cos(ang), np.sin(ang)


def rope(x, pos, theta, ft=np.float32):
    """Rotate x [n, heads, hd] row i by pos[i]: (x_j, x_{j+hd/2}) ->
    (x_j cos - x_{j+hd/2} sin, x_j sin + x_{j+hd/2} cos). The rotation runs in fp64 and the
    result is returned in ``ft``."""
    x = np.asarray(x)
    n, _, hd = x.shape
    half = hd // 2
    c, s = rope_angles(np.asarray(pos).reshape(n), hd, theta)
    c = c[:, None, :]
    s = s[:, None, :]
    x1 = x[..., :half].astype(np.float64)
    x2 = x[..., half:].astype(np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    out[..., :half] = x1 * c - x2 * s
    out[..., half:] = x1 * s + x2 * c
    return out.astype(ft)


def causal_attention(q, q_pos, k_cache, v_cache, ft=np.float32, rnd=None):
    """Softmax attention of queries q [n, Hq, hd] sitting at absolute positions q_pos [n] over
    the cache rows k_cache/v_cache [L, Hkv, hd]; row t is visible to a query at p iff t <= p.
    Scale 1/sqrt(hd); query head h uses kv head h // (Hq / Hkv). ``rnd`` (if given) rounds the
    unnormalised softmax weights, the operand of the product with V."""
    q = np.asarray(q, dtype=ft)
    kc = np.asarray(k_cache, dtype=ft)
    vc = np.asarray(v_cache, dtype=ft)
    n, hq, hd = q.shape
    hkv = kc.shape[1]
    group = hq // hkv
    q_pos = np.asarray(q_pos).reshape(n)
    visible = np.arange(kc.shape[0])[None, :] <= q_pos[:, None]
    scale = ft(1.0 / np.sqrt(hd))
    out = np.empty((n, hq, hd), dtype=ft)
    for h in range(hq):
        g = h // group
        s = (q[:, h, :] @ kc[:, g, :].T) * scale
        s = np.where(visible, s, ft(-np.inf))
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        out[:, h, :] = (_r(rnd, p, ft) @ vc[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def attention_at(q, q_pos, keys, key_pos, values, ft=np.float32):
    """Softmax attention of queries q [n, Hq, hd] at positions q_pos [n] over a set of cached rows
    given with their own positions: keys/values [m, Hkv, hd] at key_pos [m] (any order, any gaps);
    row t is visible to a query at p iff key_pos[t] <= p. Scale 1/sqrt(hd); query head h reads kv
    head h // (Hq / Hkv). With key_pos = 0..L-1 this is causal_attention."""
    q = np.asarray(q, dtype=ft)
    kc = np.asarray(keys, dtype=ft)
    vc = np.asarray(values, dtype=ft)
    n, hq, hd = q.shape
    group = hq // kc.shape[1]
    visible = np.asarray(key_pos).reshape(1, -1) <= np.asarray(q_pos).reshape(n, 1)
    scale = ft(1.0 / np.sqrt(hd))
    out = np.empty((n, hq, hd), dtype=ft)
    for h in range(hq):
        g = h // group
        s = (q[:, h, :] @ kc[:, g, :].T) * scale
        s = np.where(visible, s, ft(-np.inf))
        p = np.exp(s - s.max(axis=1, keepdims=True))
        out[:, h, :] = (p @ vc[:, g, :]) / p.sum(axis=1, keepdims=True)
    return out


def silu(z):
    return z / (1 + np.exp(-z))


def layer_rows(cfg, w, h_rows, pos, k_cache, v_cache, ft=np.float32, bf16_ops=None):
    """One decoder layer applied to the rows ``h_rows`` [n, d] sitting at positions ``pos``.

    The rows' fresh K and V are written into ``k_cache``/``v_cache`` [L, Hkv, hd] at rows
    ``pos`` *before* attention, so each row attends over the cache as it stands after the
    write (QCFuse §2.1.3 Eq. 7: selected rows read their prefix through the partially fused
    cache; CacheBlend's per-layer pass scatters fresh K/V, then attends). Returns the layer
    output for these rows; other rows are untouched.
    """
    n = h_rows.shape[0]
    hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    eps = cfg.rms_eps
    rnd = rounding(cfg, bf16_ops)
    a = _r(rnd, rms_norm(h_rows, w.attn_norm, eps, ft), ft)
    q = (a @ np.asarray(w.wq, ft).T).reshape(n, hq, hd)
    k = (a @ np.asarray(w.wk, ft).T).reshape(n, hkv, hd)
    v = (a @ np.asarray(w.wv, ft).T).reshape(n, hkv, hd)
    if cfg.qk_norm:
        q = rms_norm(q, w.q_norm, eps, ft)
        k = rms_norm(k, w.k_norm, eps, ft)
    q = rope(q, pos, cfg.rope_theta, ft)
    k = rope(k, pos, cfg.rope_theta, ft)
    k_cache[pos] = _r(rnd, k, ft)
    v_cache[pos] = _r(rnd, v, ft)
    o = causal_attention(_r(rnd, q, ft), pos, k_cache, v_cache, ft, rnd).reshape(n, hq * hd)
    h1 = np.asarray(h_rows, ft) + _r(rnd, o, ft) @ np.asarray(w.wo, ft).T
    b = _r(rnd, rms_norm(h1, w.mlp_norm, eps, ft), ft)
    act = silu(b @ np.asarray(w.w_gate, ft).T) * (b @ np.asarray(w.w_up, ft).T)
    return h1 + _r(rnd, act, ft) @ np.asarray(w.w_down, ft).T


def layer_rows_over(cfg, w, h_rows, pos, keys, key_pos, values, ft=np.float32):
    """One decoder layer applied to the rows ``h_rows`` [n, d] at positions ``pos`` when the cache
    they read is a set of rows with explicit positions (keys/values [m, Hkv, hd] at key_pos [m])
    rather than rows 0..L-1: the rows' fresh K/V join that set at their own positions before the
    attention, as in layer_rows. Returns (layer output [n, d], fresh K, fresh V)."""
    n = h_rows.shape[0]
    hq, hkv, hd = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    eps = cfg.rms_eps
    a = rms_norm(h_rows, w.attn_norm, eps, ft)
    q = (a @ np.asarray(w.wq, ft).T).reshape(n, hq, hd)
    if cfg.qk_norm:
        q = rms_norm(q, w.q_norm, eps, ft)
    q = rope(q, pos, cfg.rope_theta, ft)
    k, v = kv_rows(cfg, w, h_rows, pos, ft)
    ks = np.concatenate([np.asarray(keys, ft), k])
    vs = np.concatenate([np.asarray(values, ft), v])
    kp = np.concatenate([np.asarray(key_pos, np.int64), np.asarray(pos, np.int64)])
    o = attention_at(q, pos, ks, kp, vs, ft).reshape(n, hq * hd)
    h1 = np.asarray(h_rows, ft) + o @ np.asarray(w.wo, ft).T
    b = rms_norm(h1, w.mlp_norm, eps, ft)
    act = silu(b @ np.asarray(w.w_gate, ft).T) * (b @ np.asarray(w.w_up, ft).T)
    return h1 + act @ np.asarray(w.w_down, ft).T, k, v


def k_rows(cfg, w, h_rows, pos, ft=np.float32, bf16_ops=None):
    """Current keys of the given rows: RoPE_pos(knorm(RMSNorm(h) @ Wk^T)) -> [n, Hkv, hd].
    These are the K_i^current of Request Order Matters §2.2 Eq. 1 (kept unrounded: they are
    compared, not stored)."""
    n = h_rows.shape[0]
    a = _r(rounding(cfg, bf16_ops), rms_norm(h_rows, w.attn_norm, cfg.rms_eps, ft), ft)
    k = (a @ np.asarray(w.wk, ft).T).reshape(n, cfg.n_kv_heads, cfg.head_dim)
    if cfg.qk_norm:
        k = rms_norm(k, w.k_norm, cfg.rms_eps, ft)
    return rope(k, pos, cfg.rope_theta, ft)


def kv_rows(cfg, w, h_rows, pos, ft=np.float32):
    """Fresh K and V of the given rows as a layer writes them into its cache (before any storage
    rounding): K = RoPE_pos(knorm(RMSNorm(h) @ Wk^T)), V = RMSNorm(h) @ Wv^T; [n, Hkv, hd] each."""
    n = h_rows.shape[0]
    a = rms_norm(h_rows, w.attn_norm, cfg.rms_eps, ft)
    k = (a @ np.asarray(w.wk, ft).T).reshape(n, cfg.n_kv_heads, cfg.head_dim)
    v = (a @ np.asarray(w.wv, ft).T).reshape(n, cfg.n_kv_heads, cfg.head_dim)
    if cfg.qk_norm:
        k = rms_norm(k, w.k_norm, cfg.rms_eps, ft)
    return rope(k, pos, cfg.rope_theta, ft), v


def full_prefill(model, tokens, ft=np.float32, n_layers=None, bf16_ops=None):
    """QCFuse §2.1.1 Eq. 2: every layer on every token at positions 0..n-1, causal.

    model: object with ``cfg``, ``embed`` [vocab, d], ``final_norm`` [d], ``layer(l)``.
    Returns (K [Ly, n, Hkv, hd], V, final normed hidden [n, d], last hidden before the norm)."""
    cfg = model.cfg
    ly = cfg.n_layers if n_layers is None else n_layers
    tokens = np.asarray(tokens)
    n = len(tokens)
    kc = np.zeros((ly, n, cfg.n_kv_heads, cfg.head_dim), dtype=ft)
    vc = np.zeros_like(kc)
    h = np.asarray(model.embed[tokens], dtype=ft)
    pos = np.arange(n)
    for l in range(ly):
        h = layer_rows(cfg, model.layer(l), h, pos, kc[l], vc[l], ft, bf16_ops)
    return kc, vc, rms_norm(h, model.final_norm, cfg.rms_eps, ft), h


def chunk_prefill(model, chunk, ft=np.float32, n_layers=None, bf16_ops=None):
    """QCFuse §2.1.2 Eq. 3: a chunk's own cache, prefilled standalone at local positions
    0..|c|-1. Returns (K [Ly, |c|, Hkv, hd], V)."""
    kc, vc, _, _ = full_prefill(model, chunk, ft, n_layers, bf16_ops)
    return kc, vc
