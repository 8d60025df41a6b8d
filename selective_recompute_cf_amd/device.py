"""Device-memory plumbing: upload host weight arrays as torch tensors and build the
cf_layer_weights array that libcf reads. No compute happens here."""
from __future__ import annotations

from typing import Callable, List, Optional

import numpy as np

from . import layer_array

MATS = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
GAINS = ("attn_norm", "mlp_norm", "q_norm", "k_norm")


def to_device(a: np.ndarray, dtype: str, device="cuda"):
    """Upload an fp32 array. For "bf16" the values must already be bf16-representable (their
    low 16 bits zero); the upper halves are sent as raw bf16 bits."""
    import torch
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        hi = (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        return torch.from_numpy(hi.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


class DeviceModel:
    """A decoder's weights resident on one GPU.

    ``host`` is any object with ``cfg`` (shape fields and ``dtype``), ``layer(l)`` returning
    per-layer arrays named as in cf_layer_weights ([out, in] matrices, fp32 gains), ``embed``
    [vocab, d] and ``final_norm`` [d]. ``on_layer(l)`` is called after layer l is on the device."""

    def __init__(self, host, device="cuda", n_layers: Optional[int] = None, with_embed: bool = True,
                 on_layer: Optional[Callable[[int], None]] = None):
        import torch
        self.cfg = host.cfg
        self.dtype = host.cfg.dtype
        self.n_layers = host.cfg.n_layers if n_layers is None else n_layers
        self.layers: List[dict] = []
        for l in range(self.n_layers):
            w = host.layer(l)
            t = {n: to_device(getattr(w, n), self.dtype, device) for n in MATS}
            for n in GAINS:
                g = getattr(w, n, None)
                if g is not None:
                    t[n] = torch.from_numpy(np.ascontiguousarray(g, np.float32)).to(device)
            self.layers.append(t)
            if on_layer is not None:
                on_layer(l)
        self.embed = to_device(host.embed, self.dtype, device) if with_embed else None
        self.final_norm = torch.from_numpy(np.ascontiguousarray(host.final_norm, np.float32)).to(device)
        self.array = layer_array(self.layers)

    def weight_bytes(self) -> int:
        return sum(t.numel() * t.element_size() for layer in self.layers for t in layer.values())
