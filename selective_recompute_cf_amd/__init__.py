"""Python binding of libcf (blended prefill on AMD MI355X).

Argument marshalling only: every call forwards device pointers of torch tensors and torch's
current HIP stream to the C entry points declared in include/cf.h, and every step of the
path runs in libcf's HIP kernels. The shared library must be built first
(``python -m selective_recompute_cf_amd.build``); without it every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcf.so")

CF_OK, CF_EINVAL, CF_ESHAPE, CF_EDTYPE, CF_EUNSUPPORTED, CF_EWORKSPACE, CF_EHIP = range(7)
CF_NOALLOC_SCRATCH_BYTES = 4 << 20  # include/cf.h: the fixed scratch of cf_topk_select_noalloc
CF_F32, CF_BF16 = 0, 1
CF_SEL_TOKEN_TOPK, CF_SEL_DOC_SPANS, CF_SEL_ALL, CF_SEL_RANKED_SPANS, CF_SEL_SPAN_HEADS, CF_SEL_GIVEN = range(6)
ANCHOR_RULES = {"sink": 0, "knorm": 1, "knorm_low": 2}
MODES = {"token": CF_SEL_TOKEN_TOPK, "doc": CF_SEL_DOC_SPANS, "all": CF_SEL_ALL, "ranked": CF_SEL_RANKED_SPANS,
         "heads": CF_SEL_SPAN_HEADS, "given": CF_SEL_GIVEN}
EXPORTS = ["cf_ctx_create", "cf_ctx_destroy", "cf_last_error", "cf_version", "cf_rope_reposition",
           "cf_kv_deviation", "cf_topk_workspace_size", "cf_topk_workspace_min_size", "cf_topk_select",
           "cf_topk_select_noalloc",
           "cf_blend_layer_workspace_size", "cf_blend_layer", "cf_blend_prefill_workspace_size",
           "cf_blend_prefill", "cf_blend_prefill_gradual_workspace_size", "cf_blend_prefill_gradual",
           "cf_blend_prefill_streamed_workspace_size", "cf_blend_prefill_streamed", "cf_query_scores_workspace_size",
           "cf_query_scores", "cf_selection_deviation_workspace_size", "cf_selection_deviation",
           "cf_budget", "cf_gradual_schedule", "cf_loading_ratio", "cf_single_window_bounds",
           "cf_fixed_chunk_bounds", "cf_selection_stats", "cf_key_norms", "cf_anchor_positions",
           "cf_query_scores_anchored_workspace_size", "cf_query_scores_anchored",
           "cf_profile_enable", "cf_profile_report", "cf_mfma_loop", "cf_copy_loop"]


class CfError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libcf status {status}: {msg}")
        self.status = status


class ModelCfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "d_ffn", "vocab", "qk_norm")] + \
               [("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "w_gate", "w_up", "w_down", "q_norm", "k_norm")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libcf.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m selective_recompute_cf_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "cf_ctx_create": (i32, [ctypes.POINTER(ModelCfg), i32, i32, ctypes.POINTER(vp)]),
        "cf_ctx_destroy": (None, [vp]),
        "cf_last_error": (ctypes.c_char_p, []),
        "cf_version": (ctypes.c_char_p, []),
        "cf_profile_enable": (i32, [i32]),
        "cf_profile_report": (ctypes.c_char_p, []),
        "cf_mfma_loop": (i32, [i32, i32, i32, vp, ctypes.POINTER(ctypes.c_double), vp]),
        "cf_copy_loop": (i32, [i32, vp, vp, i64, vp]),
        "cf_rope_reposition": (i32, [vp, vp, vp, i64, i32, vp, vp, i64, i32, vp, i32, i32, i32, vp]),
        "cf_kv_deviation": (i32, [vp, i32, i64, vp, i32, i64, vp, i32, i32, vp]),
        "cf_topk_workspace_size": (sz, [i32, i32]),
        "cf_topk_workspace_min_size": (sz, [i32, i32]),
        "cf_topk_select": (i32, [vp, i32, i32, i32, vp, i32, vp, vp, sz, vp]),
        "cf_topk_select_noalloc": (i32, [vp, i32, i32, i32, vp, i32, vp, vp]),
        "cf_blend_layer_workspace_size": (sz, [vp, i32, i32]),
        "cf_blend_layer": (i32, [vp, ctypes.POINTER(LayerWeights), vp, vp, vp, vp, i32, i32, vp, sz, vp]),
        "cf_blend_prefill_workspace_size": (sz, [vp, i32, i32, i32, i32]),
        "cf_blend_prefill": (i32, [vp, ctypes.POINTER(LayerWeights), vp, vp, vp, i32, i32, vp, vp, i64, i32, vp,
                                   i32, i32, i32, i32, vp, i32, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "cf_blend_prefill_gradual_workspace_size": (sz, [vp, i32, i32, i32, vp]),
        "cf_blend_prefill_streamed_workspace_size": (sz, [vp, i32, i32, i32, i32, i32]),
        "cf_query_scores_workspace_size": (sz, [vp, i32, i32]),
        "cf_query_scores": (i32, [vp, ctypes.POINTER(LayerWeights), vp, vp, i32, i32, vp, vp, i64, vp, i32, vp, vp, sz,
                                  vp]),
        "cf_blend_prefill_streamed": (i32, [vp, ctypes.POINTER(LayerWeights), vp, vp, vp, i32, i32, vp, vp, i64, i32,
                                            vp, i32, i32, i32, i32, vp, i32, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "cf_blend_prefill_gradual": (i32, [vp, ctypes.POINTER(LayerWeights), vp, vp, vp, i32, i32, vp, vp, i64, i32,
                                           vp, i32, i32, vp, vp, vp, i64, vp, vp, vp, vp, sz, vp]),
        "cf_selection_deviation_workspace_size": (sz, [vp, i32]),
        "cf_selection_deviation": (i32, [vp, ctypes.POINTER(LayerWeights), vp, i32, vp, vp, vp, sz, vp]),
        "cf_budget": (i32, [i32, i32, i32, ctypes.POINTER(i32)]),
        "cf_gradual_schedule": (i32, [i32, i32, i32, i32, i32, i32, i32, i32, vp]),
        "cf_loading_ratio": (i32, [ctypes.c_double, vp, vp, i32, i32, i32, ctypes.POINTER(i32),
                                   ctypes.POINTER(i32)]),
        "cf_single_window_bounds": (i32, [i32, vp, i32, ctypes.POINTER(i32)]),
        "cf_fixed_chunk_bounds": (i32, [i32, i32, i32, vp, i32, ctypes.POINTER(i32)]),
        "cf_selection_stats": (i32, [vp, i32, vp, i32, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_double)]),
        "cf_key_norms": (i32, [vp, vp, i64, i32, i32, i32, vp, vp]),
        "cf_anchor_positions": (i32, [i32, vp, i32, i32, i32, vp, i32, vp, i32, ctypes.POINTER(i32)]),
        "cf_query_scores_anchored_workspace_size": (sz, [vp, i32, i32, i32]),
        "cf_query_scores_anchored": (i32, [vp, ctypes.POINTER(LayerWeights), vp, vp, i32, i32, vp, vp, i64, vp, i32,
                                           vp, i32, vp, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != CF_OK:
        raise CfError(status, lib().cf_last_error().decode())


def version() -> str:
    return lib().cf_version().decode()


def profile_enable(on: bool = True):
    """Bracket every libcf kernel launch with HIP events (see cf_profile_enable)."""
    _check(lib().cf_profile_enable(1 if on else 0))


def mfma_loop(out, blocks_per_cu: int, iters: int) -> float:
    """Enqueue the matrix-core loop (cf_mfma_loop) on the current stream; returns its flop count."""
    fl = ctypes.c_double(0.0)
    _check(lib().cf_mfma_loop(out.device.index or 0, blocks_per_cu, iters, _ptr(out), ctypes.byref(fl),
                              _stream(out.device)))
    return fl.value


def copy_loop(src, dst):
    """Enqueue the streaming copy (cf_copy_loop) of src's bytes into dst on the current stream."""
    _check(lib().cf_copy_loop(src.device.index or 0, _ptr(src), _ptr(dst), src.numel() * src.element_size(),
                              _stream(src.device)))


def profile_report() -> dict:
    """{kernel name: (launches, total ms)} since the previous report (waits for the events)."""
    import json
    return {k: (int(v[0]), float(v[1])) for k, v in json.loads(lib().cf_profile_report().decode()).items()}


# ----------------------------------------------------------------------------- torch plumbing

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device=None) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _host_i32(rows: Optional[Iterable[Iterable[int]]]):
    if rows is None:
        return None, 0
    flat: List[int] = [int(v) for r in rows for v in (r if isinstance(r, (list, tuple)) else [r])]
    arr = (ctypes.c_int32 * max(1, len(flat)))(*flat)
    return arr, len(flat)


def _span_arg(mode: str, span_bounds):
    """Host span array and span count: the bounds, and for "ranked" (span_bounds = (bounds,
    order)) the order after them."""
    if span_bounds is None:
        return None, 0
    if mode == "ranked":
        bounds, order = span_bounds
        arr, _ = _host_i32(list(bounds) + list(order))
        return arr, len(bounds) - 1
    arr, nb = _host_i32(span_bounds)
    return arr, max(0, nb - 1)


def _room(t, n: int, name: str, dtype=None):
    """Raise CF_EDTYPE unless t (when given) has the dtype, CF_EINVAL unless its storage holds n elements from its
    data pointer on. The library reads and writes through raw pointers and cannot see allocation
    sizes, so this is where a short or mistyped buffer is caught before any kernel runs."""
    if t is None or n <= 0:
        return
    if dtype is not None and t.dtype != dtype:
        raise CfError(CF_EDTYPE, f"{name}: dtype {t.dtype}, expected {dtype}")
    avail = t.untyped_storage().nbytes() // t.element_size() - t.storage_offset()
    if n > avail:
        raise CfError(CF_EINVAL, f"{name}: needs {n} elements from its start, has {avail}")


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return CF_BF16
    if t.dtype == torch.float32:
        return CF_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


class Context:
    """A cf_ctx: model shape + RoPE tables on one device."""

    def __init__(self, n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab, qk_norm,
                 rope_theta, rms_eps, dtype: str, max_pos: int, device: int = 0):
        self.cfg = ModelCfg(n_layers, d_model, n_q_heads, n_kv_heads, head_dim, d_ffn, vocab, int(bool(qk_norm)),
                            float(rope_theta), float(rms_eps), CF_BF16 if dtype == "bf16" else CF_F32)
        self.dtype = dtype
        self.device = device
        self.max_pos = max_pos
        h = ctypes.c_void_p()
        _check(lib().cf_ctx_create(ctypes.byref(self.cfg), max_pos, device, ctypes.byref(h)))
        self.handle = h

    @classmethod
    def from_model_cfg(cls, m, max_pos: int, device: int = 0, dtype: Optional[str] = None):
        return cls(m.n_layers, m.d_model, m.n_q_heads, m.n_kv_heads, m.head_dim, m.d_ffn, m.vocab, m.qk_norm,
                   m.rope_theta, m.rms_eps, dtype or m.dtype, max_pos, device)

    def close(self):
        if getattr(self, "handle", None) and self.handle.value:
            lib().cf_ctx_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def kv_dim(self) -> int:
        return self.cfg.n_kv_heads * self.cfg.head_dim

    def _tdt(self):
        torch = _torch()
        return torch.bfloat16 if self.cfg.dtype == CF_BF16 else torch.float32

    def _room_prefill(self, tokens, N, U, embed, final_norm, k_store, v_store, sls, sr, k_out, v_out, ols,
                      out_hidden):
        """Sizes and dtypes of the buffers every prefill call shares."""
        torch = _torch()
        Ly, kvd, d, dt = self.cfg.n_layers, self.kv_dim, self.cfg.d_model, self._tdt()
        _room(tokens, N + U, "tokens", torch.int32)
        _room(embed, self.cfg.vocab * d, "embed", dt)
        _room(final_norm, d, "final_norm", torch.float32)
        if sr > 0:
            _room(k_store, (Ly - 1) * sls + sr * kvd, "k_store", dt)
            _room(v_store, (Ly - 1) * sls + sr * kvd, "v_store", dt)
        _room(k_out, (Ly - 1) * ols + (N + U) * kvd, "k_out", dt)
        _room(v_out, (Ly - 1) * ols + (N + U) * kvd, "v_out", dt)
        _room(out_hidden, U * d, "out_hidden", torch.float32)

    # ------------------------------------------------------------------ entry points
    def rope_reposition(self, k_store, v_store, k_blend, v_blend, chunk_tab: Sequence[Sequence[int]],
                        layer_begin: int, layer_end: int, store_rows: Optional[int] = None,
                        blend_rows: Optional[int] = None, store_layer_stride: Optional[int] = None,
                        blend_layer_stride: Optional[int] = None):
        """Tensors [Ly, rows, kvd] (or any layout with the given strides, in elements)."""
        tab, nflat = _host_i32(chunk_tab)
        sr = store_rows if store_rows is not None else k_store.shape[-2]
        br = blend_rows if blend_rows is not None else k_blend.shape[-2]
        sls = store_layer_stride if store_layer_stride is not None else sr * self.kv_dim
        bls = blend_layer_stride if blend_layer_stride is not None else br * self.kv_dim
        if layer_end > layer_begin:
            for t, nm in ((k_store, "k_store"), (v_store, "v_store")):
                _room(t, (layer_end - 1) * sls + sr * self.kv_dim, nm, self._tdt())
            for t, nm in ((k_blend, "k_blend"), (v_blend, "v_blend")):
                _room(t, (layer_end - 1) * bls + br * self.kv_dim, nm, self._tdt())
        _check(lib().cf_rope_reposition(self.handle, _ptr(k_store), _ptr(v_store), sls, sr, _ptr(k_blend),
                                        _ptr(v_blend), bls, br, tab, nflat // 4, layer_begin, layer_end,
                                        _stream(k_blend.device)))

    def blend_layer_workspace_size(self, L: int, n_sel: int) -> int:
        return int(lib().cf_blend_layer_workspace_size(self.handle, L, n_sel))

    def blend_layer(self, weights: LayerWeights, hidden, k_cache, v_cache, sel, ws):
        torch = _torch()
        n_sel = 0 if sel is None else int(sel.numel())
        L = hidden.shape[0]
        _room(hidden, L * self.cfg.d_model, "hidden", torch.float32)
        _room(k_cache, L * self.kv_dim, "k_cache", self._tdt())
        _room(v_cache, L * self.kv_dim, "v_cache", self._tdt())
        _room(sel, n_sel, "sel", torch.int32)
        _check(lib().cf_blend_layer(self.handle, ctypes.byref(weights), _ptr(hidden), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(sel), n_sel, hidden.shape[0], _ptr(ws), 0 if ws is None else ws.numel(),
                                    _stream(hidden.device)))

    def selection_deviation_workspace_size(self, N: int) -> int:
        return int(lib().cf_selection_deviation_workspace_size(self.handle, N))

    def selection_deviation(self, weights: LayerWeights, hidden, N: int, k_ref, dev, ws):
        """cf_selection_deviation: dev[i] (fp32 [N]) = squared distance between the current keys of
        hidden rows 0..N-1 (fp32 [>= N, d]) and the stitched keys k_ref ([>= N, kvd])."""
        torch = _torch()
        _room(hidden, N * self.cfg.d_model, "hidden", torch.float32)
        _room(k_ref, N * self.kv_dim, "k_ref", self._tdt())
        _room(dev, N, "dev", torch.float32)
        _check(lib().cf_selection_deviation(self.handle, ctypes.byref(weights), _ptr(hidden), N, _ptr(k_ref),
                                            _ptr(dev), _ptr(ws), 0 if ws is None else ws.numel(),
                                            _stream(hidden.device)))

    def blend_prefill_workspace_size(self, N: int, U: int, k: int, mode: str) -> int:
        return int(lib().cf_blend_prefill_workspace_size(self.handle, N, U, k, MODES[mode]))

    def blend_prefill(self, layers, embed, final_norm, tokens, N: int, U: int, k_store, v_store,
                      chunk_tab, sel_layer: int, k: int, mode: str, span_bounds, k_out, v_out, out_hidden,
                      ws, out_sel=None, out_dev=None, store_rows: Optional[int] = None,
                      store_layer_stride: Optional[int] = None, out_layer_stride: Optional[int] = None):
        """layers: a ctypes array of LayerWeights (see ``layer_array``)."""
        tab, nflat = _host_i32(chunk_tab)
        spans, ns = _span_arg(mode, span_bounds)
        sr = store_rows if store_rows is not None else (0 if k_store is None else k_store.shape[-2])
        sls = store_layer_stride if store_layer_stride is not None else sr * self.kv_dim
        ols = out_layer_stride if out_layer_stride is not None else (N + U) * self.kv_dim
        self._room_prefill(tokens, N, U, embed, final_norm, k_store, v_store, sls, sr, k_out, v_out, ols, out_hidden)
        if mode != "all":
            _room(out_sel, k, "out_sel", _torch().int32)
            _room(out_dev, N, "out_dev", _torch().float32)
        _check(lib().cf_blend_prefill(self.handle, layers, _ptr(embed), _ptr(final_norm), _ptr(tokens), N, U,
                                      _ptr(k_store), _ptr(v_store), sls, sr, tab, nflat // 4, sel_layer, k,
                                      MODES[mode], spans, ns, _ptr(k_out), _ptr(v_out), ols,
                                      _ptr(out_hidden), _ptr(out_sel), _ptr(out_dev), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(tokens.device)))


    def query_scores_workspace_size(self, N: int, U: int) -> int:
        return int(lib().cf_query_scores_workspace_size(self.handle, N, U))

    def query_scores(self, layers, embed, tokens, N: int, U: int, k_cache, v_cache, layer_set: Sequence[int], scores,
                     ws, out_layer_stride: Optional[int] = None):
        """cf_query_scores: scores (fp32 [N]) = the query rows' attention mass on each context position,
        summed over the layers in layer_set; k_cache/v_cache hold the stitched cache of every layer."""
        lset, nset = _host_i32(list(layer_set))
        ols = out_layer_stride if out_layer_stride is not None else (N + U) * self.kv_dim
        torch = _torch()
        ext = (self.cfg.n_layers - 1) * ols + (N + U) * self.kv_dim
        _room(tokens, N + U, "tokens", torch.int32)
        _room(embed, self.cfg.vocab * self.cfg.d_model, "embed", self._tdt())
        _room(k_cache, ext, "k_cache", self._tdt())
        _room(v_cache, ext, "v_cache", self._tdt())
        _room(scores, N, "scores", torch.float32)
        _check(lib().cf_query_scores(self.handle, layers, _ptr(embed), _ptr(tokens), N, U, _ptr(k_cache),
                                     _ptr(v_cache), ols, lset, nset, _ptr(scores), _ptr(ws),
                                     0 if ws is None else ws.numel(), _stream(tokens.device)))

    def key_norms(self, k_store, norms, layer_begin: int = 0, layer_end: Optional[int] = None,
                  store_rows: Optional[int] = None, store_layer_stride: Optional[int] = None):
        """cf_key_norms: norms (fp32 [store_rows]) = squared key norm of each store row over the layers."""
        le = self.cfg.n_layers if layer_end is None else layer_end
        sr = store_rows if store_rows is not None else k_store.shape[-2]
        sls = store_layer_stride if store_layer_stride is not None else sr * self.kv_dim
        if sr > 0 and le > layer_begin:
            _room(k_store, (le - 1) * sls + sr * self.kv_dim, "k_store", self._tdt())
            _room(norms, sr, "norms", _torch().float32)
        _check(lib().cf_key_norms(self.handle, _ptr(k_store), sls, sr, layer_begin, le, _ptr(norms),
                                  _stream(norms.device)))

    def query_scores_anchored_workspace_size(self, N: int, U: int, n_anchors: int) -> int:
        return int(lib().cf_query_scores_anchored_workspace_size(self.handle, N, U, n_anchors))

    def query_scores_anchored(self, layers, embed, tokens, N: int, U: int, k_cache, v_cache, anchors,
                              layer_set: Sequence[int], scores, ws, out_layer_stride: Optional[int] = None):
        """cf_query_scores_anchored: the query rows probe only the anchor rows (device int32 tensor of
        ascending context positions) of the stitched cache; scores as in query_scores."""
        torch = _torch()
        lset, nset = _host_i32(list(layer_set))
        ols = out_layer_stride if out_layer_stride is not None else (N + U) * self.kv_dim
        ext = (self.cfg.n_layers - 1) * ols + (N + U) * self.kv_dim
        n_a = 0 if anchors is None else int(anchors.numel())
        _room(tokens, N + U, "tokens", torch.int32)
        _room(embed, self.cfg.vocab * self.cfg.d_model, "embed", self._tdt())
        _room(k_cache, ext, "k_cache", self._tdt())
        _room(v_cache, ext, "v_cache", self._tdt())
        _room(anchors, n_a, "anchors", torch.int32)
        _room(scores, N, "scores", torch.float32)
        _check(lib().cf_query_scores_anchored(self.handle, layers, _ptr(embed), _ptr(tokens), N, U, _ptr(k_cache),
                                              _ptr(v_cache), ols, _ptr(anchors) if n_a else None, n_a, lset, nset,
                                              _ptr(scores), _ptr(ws), 0 if ws is None else ws.numel(),
                                              _stream(tokens.device)))

    def blend_prefill_streamed_workspace_size(self, N: int, U: int, k: int, mode: str, store_rows: int) -> int:
        return int(lib().cf_blend_prefill_streamed_workspace_size(self.handle, N, U, k, MODES[mode], store_rows))

    def blend_prefill_streamed(self, layers, embed, final_norm, tokens, N: int, U: int, k_store, v_store,
                               chunk_tab, sel_layer: int, k: int, mode: str, span_bounds, k_out, v_out, out_hidden,
                               ws, out_sel=None, out_dev=None, store_rows: Optional[int] = None,
                               store_layer_stride: Optional[int] = None, out_layer_stride: Optional[int] = None):
        """cf_blend_prefill_streamed: k_store/v_store are pinned host tensors (pin_memory=True)."""
        tab, nflat = _host_i32(chunk_tab)
        spans, ns = _span_arg(mode, span_bounds)
        sr = store_rows if store_rows is not None else (0 if k_store is None else k_store.shape[-2])
        sls = store_layer_stride if store_layer_stride is not None else sr * self.kv_dim
        ols = out_layer_stride if out_layer_stride is not None else (N + U) * self.kv_dim
        self._room_prefill(tokens, N, U, embed, final_norm, k_store, v_store, sls, sr, k_out, v_out, ols, out_hidden)
        if mode != "all":
            _room(out_sel, k, "out_sel", _torch().int32)
            _room(out_dev, N, "out_dev", _torch().float32)
        _check(lib().cf_blend_prefill_streamed(self.handle, layers, _ptr(embed), _ptr(final_norm), _ptr(tokens), N, U,
                                               _ptr(k_store), _ptr(v_store), sls, sr, tab, nflat // 4, sel_layer, k,
                                               MODES[mode], spans, ns, _ptr(k_out), _ptr(v_out), ols,
                                               _ptr(out_hidden), _ptr(out_sel), _ptr(out_dev), _ptr(ws),
                                               0 if ws is None else ws.numel(), _stream(tokens.device)))

    def blend_prefill_gradual_workspace_size(self, N: int, U: int, sel_layer: int, k_sched: Sequence[int]) -> int:
        sched, _ = _host_i32(k_sched)
        return int(lib().cf_blend_prefill_gradual_workspace_size(self.handle, N, U, sel_layer, sched))

    def blend_prefill_gradual(self, layers, embed, final_norm, tokens, N: int, U: int, k_store, v_store,
                              chunk_tab, sel_layer: int, k_sched: Sequence[int], k_out, v_out, out_hidden, ws,
                              out_sets=None, out_devs=None, store_rows: Optional[int] = None,
                              store_layer_stride: Optional[int] = None, out_layer_stride: Optional[int] = None):
        """cf_blend_prefill_gradual: k_sched holds n_layers - sel_layer per-layer counts."""
        if len(k_sched) != self.cfg.n_layers - sel_layer:
            raise ValueError("k_sched needs one count per layer from sel_layer on")
        tab, nflat = _host_i32(chunk_tab)
        sched, _ = _host_i32(k_sched)
        sr = store_rows if store_rows is not None else (0 if k_store is None else k_store.shape[-2])
        sls = store_layer_stride if store_layer_stride is not None else sr * self.kv_dim
        ols = out_layer_stride if out_layer_stride is not None else (N + U) * self.kv_dim
        self._room_prefill(tokens, N, U, embed, final_norm, k_store, v_store, sls, sr, k_out, v_out, ols, out_hidden)
        ks = [int(x) for x in k_sched]
        _room(out_sets, sum(ks), "out_sets", _torch().int32)
        _room(out_devs, N + sum(ks[1:-1]), "out_devs", _torch().float32)
        _check(lib().cf_blend_prefill_gradual(self.handle, layers, _ptr(embed), _ptr(final_norm), _ptr(tokens), N, U,
                                              _ptr(k_store), _ptr(v_store), sls, sr, tab, nflat // 4, sel_layer, sched,
                                              _ptr(k_out), _ptr(v_out), ols, _ptr(out_hidden), _ptr(out_sets),
                                              _ptr(out_devs), _ptr(ws), 0 if ws is None else ws.numel(),
                                              _stream(tokens.device)))


def layer_struct(t: dict) -> LayerWeights:
    """LayerWeights from a dict of device tensors (keys as in cf_layer_weights)."""
    return LayerWeights(*[_ptr(t.get(n)) for n, _ in LayerWeights._fields_])


def layer_array(layers: Sequence[dict]):
    arr = (LayerWeights * len(layers))()
    for i, t in enumerate(layers):
        arr[i] = layer_struct(t)
    return arr


def kv_deviation(k_new, k_ref, dev, kv_dim: Optional[int] = None):
    """dev[i] = sum_c (k_new[i, c] - k_ref[i, c])^2; 2-D tensors [n, >= kv_dim]."""
    n = k_new.shape[0]
    kvd = kv_dim if kv_dim is not None else k_new.shape[1]
    if n > 0:
        _room(k_new, (n - 1) * k_new.stride(0) + kvd, "k_new")
        _room(k_ref, (n - 1) * k_ref.stride(0) + kvd, "k_ref")
        _room(dev, n, "dev", _torch().float32)
    _check(lib().cf_kv_deviation(_ptr(k_new), _dtype_code(k_new), k_new.stride(0), _ptr(k_ref), _dtype_code(k_ref),
                                 k_ref.stride(0), _ptr(dev), n, kvd, _stream(dev.device)))


def topk_workspace_size(n: int, mode: str) -> int:
    return int(lib().cf_topk_workspace_size(n, MODES[mode]))


def topk_workspace_min_size(n: int, mode: str) -> int:
    """cf_topk_workspace_min_size: the least workspace cf_topk_select runs with (token mode then keeps
    fewer undecided keys in its candidate list and may read the values twice more; same result)."""
    return int(lib().cf_topk_workspace_min_size(n, MODES[mode]))


def topk_select(dev, k: int, out_idx, mode: str = "token", span_bounds=None, ws=None):
    spans, ns = _span_arg(mode, span_bounds)
    _room(out_idx, k, "out_idx", _torch().int32)
    _check(lib().cf_topk_select(_ptr(dev), dev.numel(), k, MODES[mode], spans, ns, _ptr(out_idx),
                                _ptr(ws), 0 if ws is None else ws.numel(), _stream(dev.device)))


def topk_select_noalloc(dev, k: int, out_idx, mode: str = "token", span_bounds=None):
    """cf_topk_select_noalloc: cf_topk_select without a workspace (the library's fixed scratch)."""
    spans, ns = _span_arg(mode, span_bounds)
    _room(out_idx, k, "out_idx", _torch().int32)
    _check(lib().cf_topk_select_noalloc(_ptr(dev), dev.numel(), k, MODES[mode], spans, ns, _ptr(out_idx),
                                        _stream(dev.device)))


def budget(n_ctx: int, rho_num: int, rho_den: int) -> int:
    """cf_budget: k = max(1, floor(rho * N)) for rho > 0, 0 for rho = 0 (integer arithmetic)."""
    k = ctypes.c_int32(0)
    _check(lib().cf_budget(int(n_ctx), int(rho_num), int(rho_den), ctypes.byref(k)))
    return int(k.value)


def gradual_schedule(n_ctx: int, n_sched: int, first=(20, 100), keep=(9, 10), final=(15, 100)) -> List[int]:
    """cf_gradual_schedule: per-layer recompute counts for cf_blend_prefill_gradual. Ratios are
    (numerator, denominator) integer pairs."""
    out = (ctypes.c_int32 * max(1, int(n_sched)))()
    _check(lib().cf_gradual_schedule(int(n_ctx), int(n_sched), int(first[0]), int(first[1]), int(keep[0]),
                                     int(keep[1]), int(final[0]), int(final[1]), out))
    return [int(out[i]) for i in range(int(n_sched))]


def loading_controller(load_ms: float, recompute_ms: dict, floor=(15, 100)):
    """cf_loading_ratio: the largest candidate ratio whose per-layer recompute time fits inside the
    per-layer load time, clamped from below at ``floor``. recompute_ms: {(num, den): ms}. Returns
    (num, den)."""
    items = list(recompute_ms.items())
    n = len(items)
    rat, ms = _host_i32([[int(a), int(b)] for (a, b), _ in items])
    tms = (ctypes.c_double * max(1, n))(*[float(t) for _, t in items])
    a, b = ctypes.c_int32(0), ctypes.c_int32(1)
    _check(lib().cf_loading_ratio(float(load_ms), rat, tms, n, int(floor[0]), int(floor[1]), ctypes.byref(a),
                                  ctypes.byref(b)))
    return int(a.value), int(b.value)


def _bounds_call(fn, *args) -> List[int]:
    nb = ctypes.c_int32(0)
    cap = 64
    while True:
        out = (ctypes.c_int32 * cap)()
        st = fn(*args, out, cap, ctypes.byref(nb))
        if st == CF_OK:
            return [int(out[i]) for i in range(nb.value)]
        if nb.value <= cap:
            _check(st)
        cap = int(nb.value)


def single_window_bounds(n_ctx: int) -> List[int]:
    """cf_single_window_bounds: the one span [0, n_ctx)."""
    return _bounds_call(lib().cf_single_window_bounds, int(n_ctx))


def fixed_chunk_bounds(n_ctx: int, size: int = 92, offset: int = 46) -> List[int]:
    """cf_fixed_chunk_bounds: spans of `size` tokens shifted by `offset`: 0, offset, offset + size, ...,
    n_ctx."""
    return _bounds_call(lib().cf_fixed_chunk_bounds, int(n_ctx), int(size), int(offset))


def selection_stats(sel: Sequence[int], dev) -> tuple:
    """cf_selection_stats: (segments, captured deviation) of a selection. dev: host array-like of the
    selection-layer deviation."""
    import numpy as np
    s = np.ascontiguousarray(np.asarray(sel, dtype=np.int32).ravel())
    d = np.ascontiguousarray(np.asarray(dev, dtype=np.float32).ravel())
    seg, cap = ctypes.c_int32(0), ctypes.c_double(0.0)
    _check(lib().cf_selection_stats(s.ctypes.data if s.size else None, int(s.size),
                                    d.ctypes.data if d.size else None, int(d.size), ctypes.byref(seg),
                                    ctypes.byref(cap)))
    return int(seg.value), float(cap.value)


def anchor_positions(rule: str, chunk_tab, ratio=(1, 10), scores=None, store_rows: int = 0) -> List[int]:
    """cf_anchor_positions: request positions of the chunk anchors (QCFuse Eq. 14-15), ascending.
    rule "sink", "knorm" or "knorm_low"; scores: host fp32 array-like of per-store-row key norms."""
    import numpy as np
    tab, nflat = _host_i32(chunk_tab)
    sc = None if scores is None else np.ascontiguousarray(np.asarray(scores, dtype=np.float32).ravel())
    sr = int(store_rows) if sc is None else max(int(store_rows), int(sc.size))
    nb = ctypes.c_int32(0)
    cap = 64
    while True:
        out = (ctypes.c_int32 * cap)()
        st = lib().cf_anchor_positions(ANCHOR_RULES[rule], tab, nflat // 4, int(ratio[0]), int(ratio[1]),
                                       None if sc is None else sc.ctypes.data, sr, out, cap, ctypes.byref(nb))
        if st == CF_OK:
            return [int(out[i]) for i in range(nb.value)]
        if nb.value <= cap:
            _check(st)
        cap = int(nb.value)
