"""Algorithmic work model of the blended-prefill path: the bytes each HBM-bound step must move
and the flops each matrix step must compute, per call, for one request. These are the
numerators of the roofline fractions (padding, re-reads and scratch traffic excluded).

Peaks are MI355X's published figures: HBM3E 8 TB/s; dense bf16 MFMA 2.5 PFLOP/s; fp32
vector 157.3 TFLOP/s.
"""
from __future__ import annotations

import dataclasses
from typing import Dict

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3


def kv_bytes_per_layer(L: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V of one layer for L tokens (CacheBlend blog, "Hiding Recompute Behind I/O")."""
    return 2 * L * kv_heads * head_dim * elem_bytes


@dataclasses.dataclass
class Shape:
    n_layers: int
    d: int
    hq: int
    hkv: int
    hd: int
    F: int
    eb: int  # bytes per stored element (2 for bf16)

    @property
    def qd(self) -> int:
        return self.hq * self.hd

    @property
    def kvd(self) -> int:
        return self.hkv * self.hd


def shape_of(cfg) -> Shape:
    return Shape(cfg.n_layers, cfg.d_model, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.d_ffn,
                 2 if cfg.dtype == "bf16" else 4)


def layer_gemm_flops(s: Shape, n: int) -> Dict[str, int]:
    """2 * M * N * K for the four projections of one layer on n rows."""
    return {
        "gemm/qkv": 2 * n * (s.qd + 2 * s.kvd) * s.d,
        "gemm/o": 2 * n * s.d * s.qd,
        "gemm/gate_up": 2 * n * 2 * s.F * s.d,
        "gemm/down": 2 * n * s.d * s.F,
    }


def layer_gemm_bytes(s: Shape, n: int) -> Dict[str, int]:
    """Least HBM traffic of the four projections on n rows: weights and bf16 inputs read once,
    outputs written once (fp32 for the projections feeding fp32 steps, bf16 for the SwiGLU
    activations)."""
    return {
        "bytes:gemm/qkv": s.eb * (s.qd + 2 * s.kvd) * s.d + s.eb * n * s.d + 4 * n * (s.qd + 2 * s.kvd),
        "bytes:gemm/o": s.eb * s.d * s.qd + s.eb * n * s.qd + 4 * n * s.d,
        "bytes:gemm/gate_up": s.eb * 2 * s.F * s.d + s.eb * n * s.d + s.eb * n * s.F,
        "bytes:gemm/down": s.eb * s.d * s.F + s.eb * n * s.F + 4 * n * s.d,
    }


def attention_flops(s: Shape, positions) -> int:
    """QK^T and PV of every selected row over its visible keys: 4 * Hq * hd * sum_j (p_j + 1)."""
    return 4 * s.hq * s.hd * sum(int(p) + 1 for p in positions)


def blend_step_work(s: Shape, N: int, U: int, k: int, sel_layer: int = 1, sel_positions=None) -> Dict[str, float]:
    """Algorithmic flops (MFMA steps) and bytes (HBM steps) of one blended prefill call.

    sel_positions: the selected context positions (for attention work); if None they are
    taken as evenly spread over [0, N)."""
    L = N + U
    n_sel = k + U
    if sel_positions is None:
        sel_positions = [int((i + 0.5) * N / k) for i in range(k)] if k else []
    sel_all = list(sel_positions) + list(range(N, L))
    w: Dict[str, float] = {}

    def add(key, v):
        w[key] = w.get(key, 0) + v

    for l in range(s.n_layers):
        n = L if l < sel_layer else n_sel
        for key, f in layer_gemm_flops(s, n).items():
            add(key, f)
        for key, f in layer_gemm_bytes(s, n).items():
            add(key, f)
        add("attention", attention_flops(s, range(L)) if l < sel_layer else attention_flops(s, sel_all))
    add("gemm/k_sel", 2 * N * s.kvd * s.d)
    add("bytes:gemm/k_sel", s.eb * s.kvd * s.d + s.eb * N * s.d + 4 * N * s.kvd)
    # HBM-bound steps (bytes)
    add("reposition", (s.n_layers - sel_layer) * 4 * N * s.kvd * s.eb)     # read K,V; write K,V
    # deviation of the N context keys (H2), as the method needs it with the key projection fused:
    # read the stitched keys, write one fp32 per row (the fresh keys never need to reach HBM)
    add("h2_deviation", N * s.kvd * s.eb + 4 * N)
    # gather + norm + K/V scatter of the recomputed rows (H4/H6): the fp32 residual rows read once
    # and the K/V rows written once per layer; the selection layer's norm of the N context rows and
    # the final norm of the U query rows
    for l in range(s.n_layers):
        n = L if l < sel_layer else n_sel
        add("h4h6_rows", n * s.d * 4 + 2 * n * s.kvd * s.eb)
    add("h4h6_rows", 4 * N * s.d + 2 * 4 * U * s.d)
    # what the current, unfused row kernels move (not algorithmic): the fp32 projection outputs and
    # split-K partial sums round-trip through memory
    add("unfused:deviation", 4 * N * s.kvd + s.eb * N * s.kvd + 4 * N)
    for l in range(s.n_layers):
        n = L if l < sel_layer else n_sel
        add("unfused:qkv_post", 4 * n * (s.qd + 2 * s.kvd) + s.eb * n * (s.qd + 2 * s.kvd))
        add("unfused:rows", 2 * n * s.d * (12 + s.eb))
    add("unfused:rows", 4 * N * s.d + s.eb * N * s.d + 2 * 4 * U * s.d)
    add("topk_token", 4 * N + 4 * k)
    add("embed", L * s.d * (s.eb + 4))
    return w


def full_step_work(s: Shape, L: int) -> Dict[str, float]:
    w: Dict[str, float] = {}
    for l in range(s.n_layers):
        for key, f in layer_gemm_flops(s, L).items():
            w[key] = w.get(key, 0) + f
        w["attention"] = w.get("attention", 0) + attention_flops(s, range(L))
    return w


def gemm_flops(work: Dict[str, float]) -> float:
    return sum(v for key, v in work.items() if key.startswith("gemm/"))


def gemm_bytes(work: Dict[str, float]) -> float:
    return sum(v for key, v in work.items() if key.startswith("bytes:gemm/"))
