"""Seeded synthetic inputs for blended prefill: model shapes, random-init weights, token streams.

This module holds no step of the method. It only draws the numbers that both the CPU
oracle and the GPU path consume, so that the two sides see identical inputs:

* decoder shapes (layers, width, heads, FFN, RoPE base, vocabulary),
* weights: every linear matrix and the embedding are N(0, 0.02) fp32 draws, rounded to
  bf16 (round-to-nearest-even, by bit arithmetic) for bf16 models; norm gains are 1,
* uniform-random token ids for chunks, queries and rolling-window documents,
* the workload tables (chunk count and length, query length, recompute ratio as a
  rational number, selection layer, selection mode).

Seeds: tensor ``t`` of layer ``l`` is drawn from ``SeedSequence([model_seed, l, t])``;
chunk ``i`` from ``[data_seed, 1000 + i]``, query ``r`` from ``[data_seed, 2000 + r]``,
rolling document ``j`` from ``[data_seed, 3000 + j]``.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional

import numpy as np

MODEL_SEED = 0
DATA_SEED = 1

# tensor ids inside a layer (the third SeedSequence word)
T_WQ, T_WK, T_WV, T_WO, T_WGATE, T_WUP, T_WDOWN = range(7)
# pseudo-layer ids for the per-model tensors
L_EMBED = 1_000_000
L_LMHEAD = 1_000_001


@dataclasses.dataclass(frozen=True)
class ModelCfg:
    name: str
    n_layers: int
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    rope_theta: float
    rms_eps: float
    qk_norm: bool
    dtype: str  # "f32" or "bf16": storage type of matrices, embedding and K/V cache

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def replace(self, **kw) -> "ModelCfg":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    model: ModelCfg
    n_chunks: int
    chunk_len: int
    n_query: int
    rho_num: int  # recompute ratio rho = rho_num / rho_den (a rational, never a float)
    rho_den: int
    sel_layer: int = 1
    mode: str = "token"  # "token" (top-k) or "doc" (document-aligned spans)
    steps: int = 1  # rolling-window steps (1 = a single request)

    @property
    def n_ctx(self) -> int:
        return self.n_chunks * self.chunk_len

    @property
    def n_total(self) -> int:
        return self.n_ctx + self.n_query

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY = ModelCfg("tiny-2L-d256", 2, 256, 4, 2, 64, 688, 1000, 1.0e4, 1e-5, False, "f32")
LLAMA3_8B = ModelCfg("llama-3-8b-shape", 32, 4096, 32, 8, 128, 14336, 128256, 5.0e5, 1e-5, False, "bf16")
QWEN3_8B = ModelCfg("qwen3-8b-shape", 36, 4096, 32, 8, 128, 12288, 151936, 1.0e6, 1e-6, True, "bf16")
LLAMA3_70B = ModelCfg("llama-3-70b-shape", 80, 8192, 64, 8, 128, 28672, 128256, 5.0e5, 1e-5, False, "bf16")

WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny-4x128+32-rho15", TINY, 4, 128, 32, 15, 100),
    "llama8b": Workload("llama3-8b-6x512+64-rho15", LLAMA3_8B, 6, 512, 64, 15, 100),
    "qwen8b": Workload("qwen3-8b-10x1024+128-rho30", QWEN3_8B, 10, 1024, 128, 30, 100),
    "rolling": Workload("rolling-llama3-8b-20x512+64-rho5", LLAMA3_8B, 20, 512, 64, 5, 100,
                        mode="doc", steps=50),
    "llama70b": Workload("llama3-70b-16x1024+256-rho10", LLAMA3_70B, 16, 1024, 256, 10, 100),
}


# ---------------------------------------------------------------- bf16 helpers (bit arithmetic)

def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32 holding bf16 values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000))
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of fp32 values that are already bf16-representable (uint16 array)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------- weights

def _normal(seed_words: List[int], shape, scale: float = 0.02) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(seed_words))
    x = rng.standard_normal(shape, dtype=np.float32)
    x *= np.float32(scale)
    return x


def _storage_round(cfg: ModelCfg, x: np.ndarray) -> np.ndarray:
    return bf16_round(x) if cfg.dtype == "bf16" else x


@dataclasses.dataclass
class LayerWeights:
    """One decoder layer. Matrices are [out, in] row-major fp32 arrays holding the values the
    GPU receives (bf16-representable for bf16 models); gains are fp32."""
    attn_norm: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    mlp_norm: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray
    q_norm: Optional[np.ndarray]
    k_norm: Optional[np.ndarray]

    def matrices(self):
        return dict(wq=self.wq, wk=self.wk, wv=self.wv, wo=self.wo,
                    w_gate=self.w_gate, w_up=self.w_up, w_down=self.w_down)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def layer_weights(cfg: ModelCfg, layer: int, model_seed: int = MODEL_SEED,
                  pool: Optional[ThreadPoolExecutor] = None) -> LayerWeights:
    d, qd, kvd, f = cfg.d_model, cfg.q_dim, cfg.kv_dim, cfg.d_ffn
    specs = [(T_WQ, (qd, d)), (T_WK, (kvd, d)), (T_WV, (kvd, d)), (T_WO, (d, qd)),
             (T_WGATE, (f, d)), (T_WUP, (f, d)), (T_WDOWN, (d, f))]

    def one(spec):
        t, shape = spec
        return _storage_round(cfg, _normal([model_seed, layer, t], shape))

    if pool is None:
        with ThreadPoolExecutor(_workers()) as p:
            mats = list(p.map(one, specs))
    else:
        mats = list(pool.map(one, specs))
    ones_d = np.ones(d, np.float32)
    ones_hd = np.ones(cfg.head_dim, np.float32) if cfg.qk_norm else None
    return LayerWeights(ones_d, mats[0], mats[1], mats[2], mats[3], ones_d.copy(),
                        mats[4], mats[5], mats[6], ones_hd, None if ones_hd is None else ones_hd.copy())


def embedding(cfg: ModelCfg, model_seed: int = MODEL_SEED) -> np.ndarray:
    """[vocab, d] embedding table, drawn in row blocks so several threads can fill it."""
    v, d = cfg.vocab, cfg.d_model
    out = np.empty((v, d), np.float32)
    block = 8192
    starts = list(range(0, v, block))

    def one(b0):
        rows = min(block, v - b0)
        out[b0:b0 + rows] = _storage_round(cfg, _normal([model_seed, L_EMBED, b0 // block], (rows, d)))

    with ThreadPoolExecutor(_workers()) as p:
        list(p.map(one, starts))
    return out


def final_norm(cfg: ModelCfg) -> np.ndarray:
    return np.ones(cfg.d_model, np.float32)


class Model:
    """Lazily generated random-init decoder (layer weights are produced on demand)."""

    def __init__(self, cfg: ModelCfg, model_seed: int = MODEL_SEED, cache_layers: bool = True):
        self.cfg = cfg
        self.seed = model_seed
        self._cache: Dict[int, LayerWeights] = {}
        self._cache_layers = cache_layers
        self._embed: Optional[np.ndarray] = None
        self.final_norm = final_norm(cfg)

    @property
    def embed(self) -> np.ndarray:
        if self._embed is None:
            self._embed = embedding(self.cfg, self.seed)
        return self._embed

    def layer(self, l: int) -> LayerWeights:
        if l in self._cache:
            return self._cache[l]
        w = layer_weights(self.cfg, l, self.seed)
        if self._cache_layers:
            self._cache[l] = w
        return w


# ---------------------------------------------------------------- token streams

def _tokens(words: List[int], n: int, vocab: int) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(words))
    return rng.integers(0, vocab, size=n, dtype=np.int64).astype(np.int32)


def chunk_tokens(i: int, n: int, vocab: int, data_seed: int = DATA_SEED) -> np.ndarray:
    return _tokens([data_seed, 1000 + i], n, vocab)


def query_tokens(r: int, n: int, vocab: int, data_seed: int = DATA_SEED) -> np.ndarray:
    return _tokens([data_seed, 2000 + r], n, vocab)


def doc_tokens(j: int, n: int, vocab: int, data_seed: int = DATA_SEED) -> np.ndarray:
    return _tokens([data_seed, 3000 + j], n, vocab)


def request_tokens(w: Workload, query_id: int = 0, data_seed: int = DATA_SEED):
    """Chunks in index order followed by the query: (chunks list, query, all tokens)."""
    v = w.model.vocab
    chunks = [chunk_tokens(i, w.chunk_len, v, data_seed) for i in range(w.n_chunks)]
    q = query_tokens(query_id, w.n_query, v, data_seed)
    return chunks, q, np.concatenate(chunks + [q]).astype(np.int32)


def uniform_array(words: List[int], shape, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    """Generic seeded fp32 uniform array for kernel-level tests."""
    rng = np.random.default_rng(np.random.SeedSequence(words))
    return rng.uniform(lo, hi, size=shape).astype(np.float32)


def normal_array(words: List[int], shape, scale: float = 1.0) -> np.ndarray:
    return _normal(words, shape, scale)
