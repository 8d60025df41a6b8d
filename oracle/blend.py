"""Oracle blending: position remap + stitch, KV deviation, selection, selective recompute.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings taken where the pages leave a step open (each is listed with its reason in the
design notes of the repository):

* selection layer ``s`` is a 0-based layer index; layers < s are recomputed on every row
  (CacheBlend, "The Chicken-and-Egg Problem": one early layer runs over every row, its tokens
  are ranked by KV deviation, and that set is kept for all later layers; Request Order
  Matters §2.2: one selection at a configured layer, no reranking),
* the deviation is the squared L2 norm of K only, over all kv heads and head dims
  (Request Order Matters §2.2 Eq. 1), accumulated in fp64 and returned as fp32,
* budget k = max(1, floor(rho * N)) for rho > 0 and 0 for rho = 0, in integer arithmetic
  with rho given as a rational (Request Order Matters §2.2 Eq. 2; QCFuse §2.1.3 Eq. 6),
* token top-k orders by (deviation descending, index ascending); NaN counts as +inf and
  -0 equals +0; the output is ascending,
* document-aligned spans (Request Order Matters §2.3): span score is the fp64 sequential
  sum over the span divided by its length (Eq. 3), spans rank by (score desc, span index
  asc), whole spans are taken while they fit and the walk stops at the first that does not,
  and the remainder r is the window [a, a+r) of that span with the largest fp64 total,
  computed as P[a+r] - P[a] over the span's fp64 running sum P; ties take the smallest a,
* the query U follows the context, is never ranked and is recomputed at every layer >= s
  (QCFuse §2.1.1: U is processed online and is not part of the reusable cache),
* at layer s only the selected rows and U replace the stitched cache (QCFuse Eq. 7),
* gradual filtering (CacheBlend, "The Chicken-and-Egg Problem"): the page ranks the later
  layers once by "attention deviation" and once, in its selection function, by a generic
  per-token deviation; the KV deviation of Eq. 1 is taken for both. The recompute count of
  each layer comes from a schedule k_s >= k_{s+1} >= ... (the page narrows r_1 > r_2 > ... toward
  r); the set recomputed at layer l + 1 is the k_{l+1} rows of layer l's set with the largest
  deviation measured at layer l, which is the only layer where all of them have fresh keys.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np

from .model import rms_norm, rope, layer_rows, k_rows, full_prefill, rounding, _r, layer_rows_over


# ------------------------------------------------------------------ budget

def budget(n_ctx: int, rho_num: int, rho_den: int) -> int:
    """Request Order Matters §2.2 Eq. 2: k = max(1, floor(r * N)); k = 0 when r = 0
    (the direct-reuse endpoint of QCFuse §4.1.4). r = rho_num / rho_den, integers only."""
    if rho_num < 0 or rho_den <= 0 or rho_num > rho_den:
        raise ValueError("ratio must be in [0, 1]")
    if rho_num == 0 or n_ctx == 0:
        return 0
    return max(1, (n_ctx * rho_num) // rho_den)


# ------------------------------------------------------------------ position remap + stitch

def reposition(k_rows_at_src, delta: int, theta: float, ft=np.float32):
    """QCFuse Eq. 4 remap Pi_i for RoPE keys: a key encoded at position p moves to p + delta by
    one more rotation by delta (CacheBlend, "Why You Can't Just Concatenate": re-positioned
    by composing rotations). k_rows_at_src: [n, Hkv, hd]."""
    n = k_rows_at_src.shape[0]
    return rope(k_rows_at_src, np.full(n, delta, dtype=np.int64), theta, ft)


def stitch(k_store, v_store, chunk_table, n_ctx, layers: Sequence[int], theta, ft=np.float32,
           k_out=None, v_out=None, n_total: Optional[int] = None, rnd=None):
    """QCFuse Eq. 4: KV^PIC(C) = [Pi_1(KV_1); ...; Pi_m(KV_m)].

    k_store/v_store: [Ly, rows, Hkv, hd]; chunk_table: rows of (store_row, src_pos, dst_pos,
    length): the chunk's cache rows start at ``store_row`` and were encoded at positions
    src_pos.. ; they land at request rows dst_pos.. . Keys are rotated by dst - src, values
    are copied. Returns (K, V) of shape [Ly, n_total, Hkv, hd] (rows >= n_ctx left zero).
    ``rnd`` rounds the rotated keys as they are stored (bf16 caches)."""
    ly, _, hkv, hd = k_store.shape
    n_total = n_ctx if n_total is None else n_total
    if k_out is None:
        k_out = np.zeros((ly, n_total, hkv, hd), dtype=ft)
        v_out = np.zeros_like(k_out)
    for l in layers:
        for (row, src, dst, ln) in chunk_table:
            k_out[l, dst:dst + ln] = _r(rnd, reposition(np.asarray(k_store[l, row:row + ln]), dst - src, theta, ft), ft)
            v_out[l, dst:dst + ln] = np.asarray(v_store[l, row:row + ln], dtype=ft)
    return k_out, v_out


# ------------------------------------------------------------------ deviation

def kv_deviation(k_new, k_ref):
    """Request Order Matters §2.2 Eq. 1: d_i = ||K_i^current - K_i^cached||_2^2 over every kv head
    and head dim, accumulated in fp64, returned as fp32 [n]."""
    a = np.asarray(k_new, dtype=np.float64).reshape(len(k_new), -1)
    b = np.asarray(k_ref, dtype=np.float64).reshape(len(k_ref), -1)
    diff = a - b
    return np.sum(diff * diff, axis=1).astype(np.float32)


# ------------------------------------------------------------------ selection

def _canonical(d):
    d = np.array(d, dtype=np.float32, copy=True)
    d[np.isnan(d)] = np.float32(np.inf)
    d[d == 0] = np.float32(0.0)  # -0 -> +0
    return d


def select_topk(d, k: int) -> np.ndarray:
    """Token top-k (CacheBlend, "Quantifying the Damage": HKVD tokens are the top r% by
    deviation; Request Order Matters §2.2: LMCache picks the k largest d_i). Order:
    deviation descending, lower index first among equals. Output: ascending int32 [k]."""
    d = _canonical(d)
    n = len(d)
    if not 0 <= k <= n:
        raise ValueError("k out of range")
    order = np.argsort(-d, kind="stable")  # stable: equal values keep index order
    return np.sort(order[:k]).astype(np.int32)


def _seq_sum(x) -> float:
    s = 0.0
    for v in x:
        s += float(v)
    return s


def select_doc_spans(d, k: int, bounds) -> np.ndarray:
    """Document-aligned selection (Request Order Matters §2.3 and Eq. 3).

    bounds: strictly increasing span boundaries, bounds[0] = 0, bounds[-1] = len(d).
    1. rho_j = S_j / |S_j| with S_j the fp64 sum of the span in index order.
    2. rank spans by rho_j descending, lower span index first among equals.
    3. walk the ranking taking whole spans while they fit in the remaining budget; stop at
       the first span that does not fit.
    4. if r > 0 tokens remain, take from that span the window [a, a+r) whose fp64 total
       P[a+r] - P[a] (P = the span's running fp64 sum from its start) is largest, smallest a
       first among equals.
    Output: ascending int32 [k]."""
    d = _canonical(d)
    bounds = [int(b) for b in bounds]
    n = len(d)
    if not 0 <= k <= n:
        raise ValueError("k out of range")
    if bounds[0] != 0 or bounds[-1] != n or any(b1 <= b0 for b0, b1 in zip(bounds, bounds[1:])):
        raise ValueError("bad span bounds")
    spans = list(zip(bounds[:-1], bounds[1:]))
    score = [_seq_sum(d[a:b]) / float(b - a) for a, b in spans]
    ranking = sorted(range(len(spans)), key=lambda j: (-score[j], j))
    chosen: List[int] = []
    remaining = k
    for j in ranking:
        if remaining == 0:
            break
        a, b = spans[j]
        if b - a <= remaining:
            chosen.extend(range(a, b))
            remaining -= b - a
            continue
        # first span that does not fit: best window of length `remaining` inside it
        run = [0.0]
        for v in d[a:b]:
            run.append(run[-1] + float(v))
        best_a, best = a, None
        for start in range(0, (b - a) - remaining + 1):
            tot = run[start + remaining] - run[start]
            if best is None or tot > best:
                best, best_a = tot, a + start
        chosen.extend(range(best_a, best_a + remaining))
        remaining = 0
        break
    return np.array(sorted(chosen), dtype=np.int32)


def narrow(prev_set, dev_prev, k: int) -> np.ndarray:
    """Gradual filtering step (CacheBlend, "The Chicken-and-Egg Problem"): keep the k rows of
    ``prev_set`` (ascending positions) whose deviation ``dev_prev`` (one value per row of
    ``prev_set``, same order) is largest; equal deviations keep the lower position. Only rows
    recomputed on the previous layer have a deviation there, so the set can only shrink.
    Output: ascending int32 positions [k]."""
    prev = np.asarray(prev_set, dtype=np.int64)
    if len(dev_prev) != len(prev):
        raise ValueError("one deviation per row of the previous set")
    if not 0 <= k <= len(prev):
        raise ValueError("k out of range")
    return prev[select_topk(dev_prev, k)].astype(np.int32)


def gradual_schedule(n_ctx: int, n_sched: int, first: Tuple[int, int], keep: Tuple[int, int],
                     final: Tuple[int, int]) -> List[int]:
    """Per-layer recompute counts for gradual filtering (CacheBlend, "The Chicken-and-Egg
    Problem"): the first layer takes budget(N, r_1); each later layer keeps max(1,
    floor(k_prev * keep)) of the previous set, as the page's selection function does, but never
    fewer than the target budget(N, r) (the page narrows toward r, it does not undershoot it).
    Ratios are (numerator, denominator) pairs; integer arithmetic only."""
    k = budget(n_ctx, *first)
    floor_k = budget(n_ctx, *final)
    if floor_k > k:
        raise ValueError("the final ratio must not exceed the first")
    kn, kd = keep
    if kn < 0 or kd <= 0 or kn > kd:
        raise ValueError("keep fraction must be in [0, 1]")
    out = []
    for i in range(n_sched):
        out.append(k)
        if k > 0:
            k = max(floor_k, max(1, (k * kn) // kd))
    return out


def loading_ratio(load_ms: float, recompute_ms, floor=(15, 100)) -> Tuple[int, int]:
    """CacheBlend's loading controller ("Hiding Recompute Behind I/O"): recompute is free while a
    layer's recompute takes no longer than loading the next layer's cache, so the controller takes
    the largest ratio r whose per-layer recompute time fits in the per-layer load time, then
    clamps from below: r = max(r, r*), r* = ``floor``. ``recompute_ms`` maps (num, den) ratios to
    measured per-layer times. Returns the chosen (num, den)."""
    fits = [r for r, t in recompute_ms.items() if t <= load_ms]
    best = max(fits, key=lambda r: r[0] / r[1]) if fits else None
    if best is None or best[0] * floor[1] < floor[0] * best[1]:
        return tuple(floor)
    return tuple(best)


def single_window_bounds(n_ctx: int) -> List[int]:
    """Request Order Matters §2.3, single-window: the k-token window of largest total deviation
    anywhere in the context. As one span [0, N), the document-aligned rule takes exactly that
    window (a window of k tokens ranks the same by total or by mean)."""
    return [0, int(n_ctx)]


def fixed_chunk_bounds(n_ctx: int, size: int = 92, offset: int = 46) -> List[int]:
    """Request Order Matters §2.3 and §4.4, fixed-chunk: equal spans of ``size`` tokens (92, the
    median document length there) that cross document boundaries; the page shifts them off the
    documents by an unstated offset (``offset``, half a span by default). Bounds 0, offset,
    offset + size, ..., N (a leading span shorter than ``size`` and a ragged last one)."""
    if size <= 0 or not 0 <= offset < max(size, 1):
        raise ValueError("need size > 0 and 0 <= offset < size")
    b = [0]
    at = offset if offset > 0 else size
    while at < n_ctx:
        b.append(at)
        at += size
    b.append(int(n_ctx))
    return b if n_ctx > 0 else [0, 0]


def select_ranked_spans(n: int, k: int, bounds, order) -> np.ndarray:
    """Request Order Matters §2.3, random-document: document spans taken in a given order
    (the page draws a deterministic random order and ignores the deviation), whole spans while
    they fit; the walk stops at the first span that does not fit and takes its first r tokens
    (no deviation to pick a window by). Output: ascending int32 [k]."""
    bounds = [int(b) for b in bounds]
    order = [int(j) for j in order]
    ns = len(bounds) - 1
    if sorted(order) != list(range(ns)):
        raise ValueError("order must be a permutation of the spans")
    if not 0 <= k <= n or bounds[0] != 0 or bounds[-1] != n:
        raise ValueError("bad arguments")
    chosen, rem = [], k
    for j in order:
        if rem == 0:
            break
        a, b = bounds[j], bounds[j + 1]
        if b - a <= rem:
            chosen.extend(range(a, b))
            rem -= b - a
        else:
            chosen.extend(range(a, a + rem))
            rem = 0
    return np.array(sorted(chosen), dtype=np.int32)


def select_span_heads(n: int, k: int, bounds) -> np.ndarray:
    """EPIC's LegoLink as Request Order Matters §3 describes it: a fixed set of initial tokens of
    every reusable chunk. At an equal budget the k tokens are shared evenly (water-filling):
    T is the smallest head length with sum_j min(len_j, T) >= k, chunk j gives its first
    min(len_j, T) tokens, and the excess is taken back one token each from the last chunks whose
    head is T long. Output: ascending int32 [k]."""
    bounds = [int(b) for b in bounds]
    lens = [b - a for a, b in zip(bounds[:-1], bounds[1:])]
    if not 0 <= k <= n or bounds[0] != 0 or bounds[-1] != n:
        raise ValueError("bad arguments")
    T = 0
    while sum(min(x, T) for x in lens) < k:
        T += 1
    heads = [min(x, T) for x in lens]
    excess = sum(heads) - k
    for j in reversed(range(len(lens))):
        if excess == 0:
            break
        if heads[j] == T and T > 0:
            heads[j] -= 1
            excess -= 1
    chosen = [i for j, t in enumerate(heads) for i in range(bounds[j], bounds[j] + t)]
    return np.array(chosen, dtype=np.int32)


def selection_stats(sel, d) -> Tuple[int, float]:
    """Request Order Matters Table 2: how many separate contiguous regions the selection covers
    (segments) and the share of the total selection-layer deviation its tokens carry (captured
    deviation, fp64 sums)."""
    sel = sorted(int(i) for i in sel)
    segments = sum(1 for i, x in enumerate(sel) if i == 0 or x != sel[i - 1] + 1)
    d = _canonical(d).astype(np.float64)
    total = float(np.sum(d))
    return segments, (float(np.sum(d[sel])) / total if total > 0 else 0.0)


# ------------------------------------------------------------------ query-aware scores

def query_attention_mass(cfg, q, q_pos, k_cache, n_ctx: int, ft=np.float32, rnd=None) -> np.ndarray:
    """QCFuse §3.2.1, Attn^l(Q_U, K_C)_t: the attention weight that the query rows put on context
    position t, summed over query rows and heads. Each row's weights are its softmax over every
    cache row it sees (t <= its position, scale 1/sqrt(hd), query head h on kv head h // (Hq /
    Hkv)), so a row's weights sum to 1 over context and query rows together; only the context
    columns t < n_ctx are returned (fp64 sums)."""
    q = np.asarray(q, dtype=ft)
    kc = np.asarray(k_cache, dtype=ft)
    n, hq, hd = q.shape
    group = hq // kc.shape[1]
    visible = np.arange(kc.shape[0])[None, :] <= np.asarray(q_pos).reshape(n)[:, None]
    mass = np.zeros(n_ctx, dtype=np.float64)
    for h in range(hq):
        s = (q[:, h, :] @ kc[:, h // group, :].T) * ft(1.0 / np.sqrt(hd))
        s = np.where(visible, s, ft(-np.inf))
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        mass += p[:, :n_ctx].astype(np.float64).sum(axis=0)
    return mass


def query_scores(model, tokens, n_ctx, k_stitched, v_stitched, layer_set, ft=np.float32, bf16_ops=None,
                 return_cache=False):
    """Query-aware importance (QCFuse §3.2.1 Eq. 9-10; Eq. 20 for a layer subset, the ProphetKV-style
    full view with full-context probing): the query rows U run through the layers with the whole
    stitched cache as their prefix, which they only read (no context entry is refreshed; their
    own K/V go to rows n_ctx.. as usual), and I(t) sums the attention mass of Attn^l over the
    layers in ``layer_set``. Returns fp32 [n_ctx]. k_stitched/v_stitched: [Ly, L, Hkv, hd] with
    every layer stitched; copies are used."""
    cfg = model.cfg
    tokens = np.asarray(tokens)
    L, N = len(tokens), int(n_ctx)
    layers = sorted(set(int(l) for l in layer_set))
    kc = np.array(k_stitched, dtype=ft, copy=True)
    vc = np.array(v_stitched, dtype=ft, copy=True)
    rnd = rounding(cfg, bf16_ops)
    h = np.asarray(model.embed[tokens[N:]], dtype=ft)
    pos = np.arange(N, L)
    score = np.zeros(N, dtype=np.float64)
    for l in range(max(layers) + 1 if layers else 0):
        w = model.layer(l)
        if l in layers:  # the layer's query states, as layer_rows forms them, against the cache they see
            a = _r(rnd, rms_norm(h, w.attn_norm, cfg.rms_eps, ft), ft)
            n = len(pos)
            q = (a @ np.asarray(w.wq, ft).T).reshape(n, cfg.n_q_heads, cfg.head_dim)
            k = k_rows(cfg, w, h, pos, ft, bf16_ops)
            if cfg.qk_norm:
                q = rms_norm(q, w.q_norm, cfg.rms_eps, ft)
            q = _r(rnd, rope(q, pos, cfg.rope_theta, ft), ft)
            seen = kc[l].copy()
            seen[pos] = _r(rnd, k, ft)
            score += query_attention_mass(cfg, q, pos, seen, N, ft)
        h = layer_rows(cfg, w, h, pos, kc[l], vc[l], ft, bf16_ops)
    if return_cache:
        return score.astype(np.float32), kc, vc
    return score.astype(np.float32)


# ------------------------------------------------------------------ chunk-anchor query probing

def anchor_count(chunk_len: int, ra_num: int, ra_den: int) -> int:
    """QCFuse §3.3.1 Eq. 14: ceil(r_a |c_i|) anchors per chunk, r_a = ra_num / ra_den (integers)."""
    if ra_num < 0 or ra_den <= 0 or ra_num > ra_den or chunk_len < 0:
        raise ValueError("bad anchor ratio or chunk length")
    return (chunk_len * ra_num + ra_den - 1) // ra_den


def key_norms(k_chunk) -> np.ndarray:
    """Knorm's score (QCFuse §3.3.1): the squared L2 norm of each token's key-cache tensor, over
    every layer, kv head and head dim of the stored PIC keys. k_chunk: [Ly, n, Hkv, hd]. fp64 sums,
    returned as fp64 [n] (ranking by the norm or by its square is the same)."""
    k = np.asarray(k_chunk, dtype=np.float64)
    return np.sum(k * k, axis=(0, 2, 3))


def select_anchors(chunk_len: int, ra_num: int, ra_den: int, rule: str = "sink", scores=None) -> np.ndarray:
    """QCFuse §3.3.1 Eq. 14: A_i = TopK(G_i, ceil(r_a |c_i|)), chunk-local positions ascending.
    rule "sink": G_i(r) = -r (the tokens at the start of the chunk); "knorm": G_i(r) = the key
    norm score of position r (largest kept); "knorm_low": G_i(r) = minus that score (smallest kept).
    Equal scores keep the lower position."""
    n_a = anchor_count(chunk_len, ra_num, ra_den)
    if rule == "sink":
        g = -np.arange(chunk_len, dtype=np.float64)
    elif rule in ("knorm", "knorm_low"):
        g = np.asarray(scores, dtype=np.float64)
        if len(g) != chunk_len:
            raise ValueError("one score per chunk position")
        g = g if rule == "knorm" else -g
    else:
        raise ValueError("unknown anchor rule " + str(rule))
    order = np.argsort(-g, kind="stable")  # stable: equal scores keep the lower position first
    return np.sort(order[:n_a]).astype(np.int32)


def anchored_query_scores(model, tokens, n_ctx, k_stitched, v_stitched, anchors, layer_set, ft=np.float32,
                          return_cache=False):
    """Anchor-conditioned query probing and critical-layer scoring (QCFuse §3.3.2 Eq. 15-17, §3.4
    Eq. 18-20). ``anchors``: ascending request positions of the chunk anchors (A_i of each chunk at
    its request offset, Eq. 15). The query rows U (positions N..L-1) run through the layers with
    only the anchor rows of the stitched cache as their prefix, each anchor at its original request
    position (Eq. 16-17: the anchor KV are the re-positioned PIC entries). At each layer l of
    ``layer_set`` the anchor-conditioned query states score every original context position t
    against the full stitched context keys (Eq. 18, Eq. 20): the softmax weight of a query row on
    row t among all context rows and the query rows up to itself, summed over query rows and heads
    (the weights of the full-view probe, query_scores, read the same way). Returns fp32 [n_ctx]."""
    cfg = model.cfg
    tokens = np.asarray(tokens)
    L, N = len(tokens), int(n_ctx)
    anchors = np.asarray(anchors, dtype=np.int64)
    if len(anchors) and (np.any(np.diff(anchors) <= 0) or anchors[0] < 0 or anchors[-1] >= N):
        raise ValueError("anchors must be strictly increasing context positions")
    layers = sorted(set(int(l) for l in layer_set))
    h = np.asarray(model.embed[tokens[N:]], dtype=ft)
    pos = np.arange(N, L)
    score = np.zeros(N, dtype=np.float64)
    kc = np.array(k_stitched, dtype=ft, copy=True)
    for l in range(max(layers) + 1 if layers else 0):
        w = model.layer(l)
        h_next, k_new, v_new = layer_rows_over(cfg, w, h, pos, kc[l][anchors], anchors, v_stitched[l][anchors], ft)
        if l in layers:  # Eq. 18: the probe's query states against the full context keys of this layer
            a = rms_norm(h, w.attn_norm, cfg.rms_eps, ft)
            q = (a @ np.asarray(w.wq, ft).T).reshape(len(pos), cfg.n_q_heads, cfg.head_dim)
            if cfg.qk_norm:
                q = rms_norm(q, w.q_norm, cfg.rms_eps, ft)
            q = rope(q, pos, cfg.rope_theta, ft)
            kc[l][pos] = k_new
            score += query_attention_mass(cfg, q, pos, kc[l], N, ft)
        h = h_next
    if return_cache:
        return score.astype(np.float32), kc
    return score.astype(np.float32)


# ------------------------------------------------------------------ blended prefill

@dataclasses.dataclass
class BlendResult:
    k: np.ndarray        # fused K [Ly, L, Hkv, hd]
    v: np.ndarray        # fused V
    out: np.ndarray      # RMSNorm(h) of the query rows [U, d]
    sel: np.ndarray      # selected context positions, ascending [k]
    dev: np.ndarray      # deviation at the selection layer [N] (empty for full prefill)
    hidden: np.ndarray   # residual stream [L, d] after the last layer
    sets: Optional[List[np.ndarray]] = None        # gradual: the recompute set of layers s..Ly-1
    layer_devs: Optional[List[np.ndarray]] = None  # gradual: deviation over the set, layers s+1..Ly-2


def blend_prefill(model, tokens, n_ctx, k_store, v_store, chunk_table, sel_layer: int, k: int,
                  mode: str = "token", span_bounds=None, ft=np.float32, n_layers=None,
                  bf16_ops=None, k_sched: Optional[Sequence[int]] = None) -> BlendResult:
    """Blended prefill of one request: context C (n_ctx rows) followed by the query U.

    1. Stitch: layers s..Ly-1 of the request cache are the remapped chunk caches (QCFuse Eq. 4).
    2. h = embedding of every token.
    3. Layers l < s: ordinary prefill of all rows (their K/V overwrite the cache).
    4. Layer s: current keys of the context rows, deviation against the stitched keys
       (Request Order Matters Eq. 1), then the recompute set P (top-k or document spans).
    5. sel = P followed by the query rows N..L-1; layers l >= s run only on ``sel``: fresh
       K/V are scattered into the cache at sel, the selected rows attend over the fused cache
       and only their hidden rows change (CacheBlend "Selective Recompute Without Skipping";
       QCFuse Eq. 7).
    6. Output: the fused K/V of every layer and RMSNorm of the query rows.

    With ``k_sched`` (token mode; Ly - s counts, k_sched[0] = k, non-increasing) the set narrows
    layer by layer (gradual filtering, CacheBlend "The Chicken-and-Egg Problem"): at each layer
    l < Ly - 1 the deviation of the current set's fresh keys against the stitched keys they are
    about to replace is measured (at layer s it is the step-4 deviation), and layer l + 1
    recomputes the k_sched[l + 1 - s] rows of that set with the largest deviation (``narrow``).

    mode "all" is ordinary full prefill of every row at every layer (QCFuse Eq. 2)."""
    cfg = model.cfg
    ly = cfg.n_layers if n_layers is None else n_layers
    tokens = np.asarray(tokens)
    L = len(tokens)
    N = int(n_ctx)
    hkv, hd = cfg.n_kv_heads, cfg.head_dim
    kc = np.zeros((ly, L, hkv, hd), dtype=ft)
    vc = np.zeros_like(kc)
    h = np.asarray(model.embed[tokens], dtype=ft)
    pos_all = np.arange(L)
    rnd = rounding(cfg, bf16_ops)
    if mode == "all":
        for l in range(ly):
            h = layer_rows(cfg, model.layer(l), h, pos_all, kc[l], vc[l], ft, bf16_ops)
        out = rms_norm(h[N:], model.final_norm, cfg.rms_eps, ft)
        return BlendResult(kc, vc, out, np.arange(N, dtype=np.int32), np.zeros(0, np.float32), h)

    s = int(sel_layer)
    if not 0 <= s < ly:
        raise ValueError("selection layer out of range")
    stitch(k_store, v_store, chunk_table, N, range(s, ly), cfg.rope_theta, ft, kc, vc, rnd=rnd)
    for l in range(s):
        h = layer_rows(cfg, model.layer(l), h, pos_all, kc[l], vc[l], ft, bf16_ops)

    w_s = model.layer(s)
    if N > 0:
        k_cur = k_rows(cfg, w_s, h[:N], np.arange(N), ft, bf16_ops)
        dev = kv_deviation(k_cur, kc[s, :N])
    else:
        dev = np.zeros(0, np.float32)
    if mode == "token":
        P = select_topk(dev, k)
    elif mode == "doc":
        P = select_doc_spans(dev, k, span_bounds)
    elif mode == "ranked":  # span_bounds = (bounds, order)
        P = select_ranked_spans(N, k, span_bounds[0], span_bounds[1])
    elif mode == "heads":
        P = select_span_heads(N, k, span_bounds)
    elif mode == "given":  # span_bounds = the recompute set (e.g. the top of query_scores)
        P = np.asarray(sorted(int(i) for i in span_bounds), dtype=np.int32)
        if len(P) != k or len(set(P.tolist())) != k or (k and not 0 <= P[0] <= P[-1] < N):
            raise ValueError("the given set must hold k distinct context positions")
    else:
        raise ValueError("unknown mode " + str(mode))
    if k_sched is None:
        sel = np.concatenate([P.astype(np.int64), np.arange(N, L)])
        for l in range(s, ly):
            w = w_s if l == s else model.layer(l)
            if len(sel):
                h[sel] = layer_rows(cfg, w, h[sel], sel, kc[l], vc[l], ft, bf16_ops)
        out = rms_norm(h[N:], model.final_norm, cfg.rms_eps, ft)
        return BlendResult(kc, vc, out, P, dev, h)

    sched = [int(x) for x in k_sched]
    if mode != "token":
        raise ValueError("gradual filtering ranks single tokens")
    if len(sched) != ly - s or sched[0] != k or any(b > a for a, b in zip(sched, sched[1:])) or sched[-1] < 0:
        raise ValueError("k_sched needs Ly - s non-increasing counts starting at k")
    cur = P
    sets, layer_devs = [P], []
    d_cur = None
    for l in range(s, ly):
        w = w_s if l == s else model.layer(l)
        if l > s:
            cur = narrow(cur, d_cur, sched[l - s])
            sets.append(cur)
        if l + 1 < ly:  # deviation over this layer's set, before its keys replace the stitched ones
            if l == s:
                d_cur = dev[cur]
            else:
                d_cur = kv_deviation(k_rows(cfg, w, h[cur], cur, ft, bf16_ops), kc[l, cur])
                layer_devs.append(d_cur)
        sel = np.concatenate([cur.astype(np.int64), np.arange(N, L)])
        if len(sel):
            h[sel] = layer_rows(cfg, w, h[sel], sel, kc[l], vc[l], ft, bf16_ops)
    out = rms_norm(h[N:], model.final_norm, cfg.rms_eps, ft)
    return BlendResult(kc, vc, out, P, dev, h, sets, layer_devs)


def direct_reuse(model, tokens, n_ctx, k_store, v_store, chunk_table, ft=np.float32, n_layers=None,
                 bf16_ops=None):
    """The rho = 0 endpoint written from its own definition (QCFuse §2.1.2): the context cache is
    the stitched chunk caches at every layer, untouched; only the query rows are computed,
    attending over that cache. Returns (K, V, normed query hidden)."""
    cfg = model.cfg
    ly = cfg.n_layers if n_layers is None else n_layers
    tokens = np.asarray(tokens)
    L, N = len(tokens), int(n_ctx)
    kc, vc = stitch(k_store, v_store, chunk_table, N, range(ly), cfg.rope_theta, ft, n_total=L,
                    rnd=rounding(cfg, bf16_ops))
    hq = np.asarray(model.embed[tokens[N:]], dtype=ft)
    pos = np.arange(N, L)
    for l in range(ly):
        hq = layer_rows(cfg, model.layer(l), hq, pos, kc[l], vc[l], ft, bf16_ops)
    return kc, vc, rms_norm(hq, model.final_norm, cfg.rms_eps, ft)


# ------------------------------------------------------------------ rolling window

class RollingWindow:
    """Rolling agent window (Request Order Matters §2.1 and §4.1): a window of ``n_docs``
    documents; each step evicts the oldest, appends a new document and asks a fresh query.
    The store persists across steps: a new document gets a standalone prefill at position 0;
    in write-back mode every document's fused K/V and its new base position are written back
    after the step (§5: each call both consumes and updates the cache state), in pristine
    mode the store keeps the standalone caches."""

    def __init__(self, model, n_docs, doc_len, n_query, rho_num, rho_den, mode="doc",
                 sel_layer=1, write_back=True, ft=np.float32, n_layers=None, doc_tokens=None,
                 query_tokens=None):
        self.model = model
        self.n_docs, self.doc_len, self.n_query = n_docs, doc_len, n_query
        self.rho = (rho_num, rho_den)
        self.mode, self.s, self.write_back = mode, sel_layer, write_back
        self.ft = ft
        self.n_layers = model.cfg.n_layers if n_layers is None else n_layers
        self.doc_tokens = doc_tokens
        self.query_tokens = query_tokens
        self.store = {}   # doc id -> [K (Ly, len, Hkv, hd), V, base position]
        self.t = 0

    def window(self, t):
        return list(range(t, t + self.n_docs))

    def _ensure(self, j):
        if j not in self.store:
            toks = self.doc_tokens(j)
            kc, vc = chunk_prefill_for(self.model, toks, self.ft, self.n_layers)
            self.store[j] = [kc, vc, 0]

    def step(self):
        t = self.t
        docs = self.window(t)
        for j in list(self.store):
            if j not in docs:
                del self.store[j]
        for j in docs:
            self._ensure(j)
        toks = np.concatenate([self.doc_tokens(j) for j in docs] + [self.query_tokens(t)]).astype(np.int32)
        N = self.n_docs * self.doc_len
        k_store = np.concatenate([self.store[j][0] for j in docs], axis=1)
        v_store = np.concatenate([self.store[j][1] for j in docs], axis=1)
        table = [(i * self.doc_len, self.store[j][2], i * self.doc_len, self.doc_len)
                 for i, j in enumerate(docs)]
        k = budget(N, *self.rho)
        bounds = [i * self.doc_len for i in range(self.n_docs + 1)]
        res = blend_prefill(self.model, toks, N, k_store, v_store, table, self.s, k, self.mode,
                            bounds, self.ft, self.n_layers)
        if self.write_back:
            for i, j in enumerate(docs):
                a = i * self.doc_len
                self.store[j] = [res.k[:, a:a + self.doc_len].copy(), res.v[:, a:a + self.doc_len].copy(), a]
        self.t += 1
        return res, toks, table


def chunk_prefill_for(model, toks, ft, n_layers):
    kc, vc, _, _ = full_prefill(model, toks, ft, n_layers)
    return kc, vc
