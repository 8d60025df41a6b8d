"""Rolling agent window on the GPU (Request Order Matters §2.1 and §4.1): a window of ``n_docs``
documents of ``doc_len`` tokens; each step evicts the oldest document, appends a new one and asks
a fresh query of ``n_query`` tokens, which is answered with one blended prefill over the window.

The chunk store persists across steps in HBM: document j lives in store slot j mod n_docs, as the
K/V of its tokens at base position base[j]. A document that enters the window gets a standalone
prefill at position 0 (written straight into its slot). In write-back mode (the paper's §5: each
call both consumes and updates the cache state) every document's fused K/V and its position in
this step's window become its stored cache and base position after the step, so the next step
re-positions it by -doc_len; in pristine mode the store keeps the standalone caches.

Every step is made of the library's calls only: ``blend_prefill`` (standalone prefill of arriving
documents in "all" mode, then the blended prefill of the window) and ``rope_reposition`` with a
zero offset for the write-back copy (a rotation by 0 reproduces bf16 values exactly)."""
from __future__ import annotations

from typing import Callable, Dict, List, Optional

import numpy as np

from . import Context, budget


class RollingWindow:
    def __init__(self, ctx: Context, dm, n_docs: int, doc_len: int, n_query: int, rho_num: int, rho_den: int,
                 doc_tokens: Callable[[int], np.ndarray], query_tokens: Callable[[int], np.ndarray],
                 mode: str = "doc", sel_layer: int = 1, write_back: bool = True):
        import torch
        self.torch = torch
        self.ctx, self.dm = ctx, dm
        self.n_docs, self.doc_len, self.n_query = n_docs, doc_len, n_query
        self.rho = (rho_num, rho_den)
        self.mode, self.s, self.write_back = mode, sel_layer, write_back
        self.doc_tokens, self.query_tokens = doc_tokens, query_tokens
        cfg = ctx.cfg
        self.Ly, self.kvd = cfg.n_layers, ctx.kv_dim
        self.N = n_docs * doc_len
        self.L = self.N + n_query
        dt = torch.bfloat16 if ctx.dtype == "bf16" else torch.float32
        dev = torch.device("cuda", ctx.device)
        # store: [Ly][n_docs slots x doc_len rows][kvd]; fused output of the current step: [Ly][L][kvd]
        self.k_store = torch.zeros(self.Ly, self.N, self.kvd, dtype=dt, device=dev)
        self.v_store = torch.zeros_like(self.k_store)
        self.k_out = torch.zeros(self.Ly, self.L, self.kvd, dtype=dt, device=dev)
        self.v_out = torch.zeros_like(self.k_out)
        self.out = torch.zeros(max(n_query, 1), cfg.d_model, dtype=torch.float32, device=dev)
        self.k = budget(self.N, rho_num, rho_den)
        self.sel = torch.zeros(max(self.k, 1), dtype=torch.int32, device=dev)
        self.dev = torch.zeros(self.N, dtype=torch.float32, device=dev)
        ws = max(ctx.blend_prefill_workspace_size(self.N, n_query, self.k, mode),
                 ctx.blend_prefill_workspace_size(doc_len, 0, doc_len, "all"))
        self.ws = torch.empty(ws, dtype=torch.uint8, device=dev)
        self.base: Dict[int, int] = {}  # doc id -> base position of its stored K/V
        self.t = 0

    def slot(self, j: int) -> int:
        return j % self.n_docs

    def window(self, t: Optional[int] = None) -> List[int]:
        t = self.t if t is None else t
        return list(range(t, t + self.n_docs))

    def _prefill_doc(self, j: int):
        """Standalone prefill of document j at position 0 into its store slot."""
        torch = self.torch
        toks = torch.from_numpy(np.ascontiguousarray(self.doc_tokens(j), np.int32)).to(self.k_store.device)
        r0 = self.slot(j) * self.doc_len
        self.ctx.blend_prefill(self.dm.array, self.dm.embed, self.dm.final_norm, toks, self.doc_len, 0, None, None,
                               None, 0, 0, "all", None, self.k_store[:, r0:], self.v_store[:, r0:], None, self.ws,
                               out_layer_stride=self.N * self.kvd)
        self.base[j] = 0

    def chunk_table(self, docs: List[int]):
        return [(self.slot(j) * self.doc_len, self.base[j], i * self.doc_len, self.doc_len)
                for i, j in enumerate(docs)]

    def store_state(self, docs: Optional[List[int]] = None):
        """Host copy of the store as the next step will read it: per window document (K, V, base)."""
        docs = self.window() if docs is None else docs
        ks, vs = self.k_store.float().cpu().numpy(), self.v_store.float().cpu().numpy()
        out = []
        for j in docs:
            if j not in self.base:
                out.append(None)
                continue
            r0 = self.slot(j) * self.doc_len
            out.append((ks[:, r0:r0 + self.doc_len], vs[:, r0:r0 + self.doc_len], self.base[j]))
        return out

    def tokens(self, t: Optional[int] = None) -> np.ndarray:
        t = self.t if t is None else t
        return np.concatenate([self.doc_tokens(j) for j in self.window(t)] + [self.query_tokens(t)]).astype(np.int32)

    def prepare(self):
        """Evict documents that left the window and prefill the ones that entered (outside the
        timed step, as on the paper's arrival path)."""
        docs = self.window()
        for j in list(self.base):
            if j not in docs:
                del self.base[j]
        for j in docs:
            if j not in self.base:
                self._prefill_doc(j)

    def step(self):
        """One query over the current window; returns (selected rows, chunk table used)."""
        torch = self.torch
        self.prepare()
        docs = self.window()
        table = self.chunk_table(docs)
        toks = torch.from_numpy(self.tokens()).to(self.k_store.device)
        spans = [i * self.doc_len for i in range(self.n_docs + 1)]
        self.ctx.blend_prefill(self.dm.array, self.dm.embed, self.dm.final_norm, toks, self.N, self.n_query,
                               self.k_store, self.v_store, table, self.s, self.k, self.mode, spans, self.k_out,
                               self.v_out, self.out if self.n_query else None, self.ws,
                               out_sel=self.sel if self.k else None, out_dev=self.dev)
        if self.write_back:
            # fused rows of window position i -> the document's slot, unrotated; its base becomes i * doc_len
            back = [(i * self.doc_len, self.slot(j) * self.doc_len, self.slot(j) * self.doc_len, self.doc_len)
                    for i, j in enumerate(docs)]
            self.ctx.rope_reposition(self.k_out, self.v_out, self.k_store, self.v_store, back, 0, self.Ly)
            for i, j in enumerate(docs):
                self.base[j] = i * self.doc_len
        self.t += 1
        return table
