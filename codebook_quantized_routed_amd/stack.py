"""A residual chain of routed layers: h <- h + MoE_l(RMSNorm(h)) for l = 0 .. L-1.

"Red Lite dev16 — complete full-attention parity", section "Pinned full-attention graph"
(the block composition: post-attention RMSNorm, the full-width top-10 routed MoE plus
shared expert, then the residual) and section "Scope boundary" (the 48-layer scheduler
is the next gate): in the field model the routed MoE runs after the post-attention
RMSNorm and its output is added to the residual stream; the model stacks 48 layers.  Attention and the rest of the block
are not part of this path, so the chain here is the MoE part of each block alone.

This module only sequences calls of the C ABI (every step runs in the library's
kernels): per layer, ``moe_rmsnorm`` then either the one-launch decode
(``moe_layer_decode_q``, one token) or ``moe_route_group`` -> ``moe_expert_ffn_q`` ->
``moe_accumulate`` (many tokens), with the residual stream as the accumulator; or, for
one token, every layer in one launch (``moe_stack_decode_q``), which gives the same bits
as the per-layer sequence.
Routing logits are inputs, one [T][E] array per layer (the router network is not part
of the path).
"""
from __future__ import annotations

from . import (DeviceLayer, accumulate, check_decode, decode_error, decode_workspace_bytes, expert_ffn_q,
               layer_decode_q, rmsnorm, route_group, stack_decode_q, stack_layers, stack_prepare,
               stack_workspace_bytes, work_ints, workspace_bytes)

RMS_EPS = 1e-6


def stack_formats(n_layers: int = 48) -> list:
    """Format of each layer of the field-model stack (1 = IQ2_XS-like, 2 = IQ1_M-like):
    IQ2_XS-like where l mod 4 == 0 and l <= 40 (11 of 48 layers), IQ1_M-like elsewhere.
    The pages give the counts (11 and 37) and that layer 0 is IQ2_XS and layer 6 IQ1_M,
    not the full map; this is the reading used here."""
    return [1 if (l % 4 == 0 and l <= 40) else 2 for l in range(n_layers)]


class LayerStack:
    """Device layers of a chain plus the per-call buffers for batches of T tokens.

    ``layers``: DeviceLayer objects (same hidden, inter, n_experts, has_shared).
    ``k``: routed experts per token.  Buffers are allocated on first use for a given T
    and reused, so a step can be captured in a graph.
    """

    def __init__(self, layers, k: int, eps: float = RMS_EPS):
        import torch
        if not layers:
            raise ValueError("empty stack")
        d0 = layers[0].desc
        for l in layers:
            d = l.desc
            if (d.hidden, d.inter, d.n_experts, d.has_shared) != (d0.hidden, d0.inter, d0.n_experts, d0.has_shared):
                raise ValueError("all layers of a stack share one shape")
        self.layers = layers
        self.k = k
        self.eps = eps
        self.H, self.I, self.E, self.shared = d0.hidden, d0.inter, d0.n_experts, d0.has_shared
        self.kp = k + self.shared
        self.n_ids = self.E + self.shared
        self.device = layers[0].tensors[0].device
        self._bufs = {}
        self._torch = torch
        self._stack = None

    def buffers(self, T: int) -> dict:
        if T in self._bufs:
            return self._bufs[T]
        torch, dev = self._torch, self.device
        i32 = dict(dtype=torch.int32, device=dev)
        kp, H, I = self.kp, self.H, self.I
        b = dict(x=torch.zeros((T, H), dtype=torch.float32, device=dev),
                 ids=torch.zeros((T, kp), **i32), w=torch.zeros((T, kp), dtype=torch.float32, device=dev),
                 counts=torch.zeros(self.n_ids, **i32), offsets=torch.zeros(self.n_ids + 1, **i32),
                 ss=torch.zeros(T * kp, **i32), sp=torch.zeros(T * kp, **i32),
                 work=torch.zeros(work_ints(T, kp, self.n_ids), **i32))
        if T == 1:
            b["ws"] = torch.zeros(decode_workspace_bytes(kp, I) // 4, dtype=torch.int32, device=dev)
        else:
            b["y"] = torch.zeros((T * kp, H), dtype=torch.float32, device=dev)
            b["ws"] = torch.zeros(workspace_bytes(T, kp, H, I) // 4, dtype=torch.int32, device=dev)
        self._bufs[T] = b
        return b

    def layer(self, l: int, h, logits, stream=None) -> None:
        """h [T][H] (in/out) <- h + MoE_l(RMSNorm(h)), routed by logits [T][E]."""
        T = h.shape[0]
        b = self.buffers(T)
        L = self.layers[l].desc
        rmsnorm(h, T, self.H, self.eps, b["x"], stream)
        if T == 1:
            layer_decode_q(L, logits, b["x"], self.k, self.shared, b["ids"], b["w"], b["counts"], b["offsets"],
                           b["ss"], b["sp"], b["work"], h, b["ws"], stream)
        else:
            route_group(logits, T, self.E, self.k, self.shared, b["ids"], b["w"], b["counts"], b["offsets"],
                        b["ss"], b["sp"], b["work"], stream)
            expert_ffn_q(L, b["x"], T, self.kp, b["ss"], b["work"], b["y"], b["ws"], stream)
            accumulate(b["y"], b["w"], b["ids"], b["sp"], T, self.kp, self.H, h, stream)

    def step(self, h, logits_per_layer, stream=None) -> None:
        """All layers in order: logits_per_layer[l] routes layer l."""
        for l in range(len(self.layers)):
            self.layer(l, h, logits_per_layer[l], stream)

    def stack_buffers(self) -> dict:
        """Buffers of the one-launch decode of every layer: the host layer array, the
        prepared workspace, and each layer's selection (ids, w [L][kprime])."""
        if self._stack is None:
            torch, dev = self._torch, self.device
            n = len(self.layers)
            arr = stack_layers([l.desc for l in self.layers])
            ws = torch.zeros(stack_workspace_bytes(n, self.kp, self.H, self.I) // 4, dtype=torch.int32, device=dev)
            stack_prepare(arr, ws)
            self._stack = dict(layers=arr, ws=ws, ids=torch.zeros((n, self.kp), dtype=torch.int32, device=dev),
                               w=torch.zeros((n, self.kp), dtype=torch.float32, device=dev))
        return self._stack

    def decode(self, h_in, h_out, logits_per_layer, stream=None) -> None:
        """One token through every layer in one launch: h_out [1][H] <- the chain applied
        to h_in [1][H] (h_in is not written; the two must not overlap)."""
        b = self.stack_buffers()
        stack_decode_q(b["layers"], logits_per_layer, h_in, h_out, self.k, self.shared, self.eps, b["ids"], b["w"],
                       b["ws"], stream)


    def decode_error(self, T: int = 1) -> int:
        """Status word of the one-launch per-layer decode's workspace (T = 1 calls of
        ``layer``); nonzero after a timed-out wait.  Synchronises the device."""
        b = self._bufs.get(T)
        return 0 if b is None or T != 1 else decode_error(b["ws"])

    def stack_error(self) -> int:
        """Status word of the one-launch stack decode's workspace.  Synchronises."""
        return 0 if self._stack is None else decode_error(self._stack["ws"])

    def check(self) -> None:
        """Raises if a one-launch call (per layer or whole stack) reported a timed-out
        wait.  Call it after the stream has run the calls (it synchronises)."""
        if self._stack is not None:
            check_decode(self._stack["ws"])
        if 1 in self._bufs:
            check_decode(self._bufs[1]["ws"])


def device_stack(formats, banks_by_format: dict, grids, hidden: int = 2048, inter: int = 512, n_experts: int = 512,
                 has_shared: int = 1, device="cuda") -> list:
    """DeviceLayer per entry of ``formats``, each its own device copy of the banks of its
    format (``banks_by_format[qtype]``)."""
    return [DeviceLayer(hidden, inter, n_experts, has_shared, banks_by_format[f], grids, device) for f in formats]
