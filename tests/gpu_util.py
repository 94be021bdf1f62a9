"""Helpers shared by the GPU parity tests: device copies of seeded inputs, one call of
the whole layer through the C ABI, and the tolerance checks.  Every input comes from
``synth``; every expected value from ``oracle``."""
from __future__ import annotations

import sys

import numpy as np
import torch

import codebook_quantized_routed_amd as moe
import oracle as O
import synth

# Outputs: max |error| <= REL_TOL * ||reference row||_2, per output row.
REL_TOL = 2e-5


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def device_grids(c2: np.ndarray, c1: np.ndarray) -> torch.Tensor:
    g = torch.empty(moe.grids_bytes(), dtype=torch.uint8, device="cuda")
    moe.grids_expand(dev(c2.view(np.int16)), dev(c1.view(np.int16)), g)
    return g


def device_layer(layer: synth.Layer, grids: torch.Tensor) -> moe.DeviceLayer:
    return moe.DeviceLayer(layer.hidden, layer.inter, layer.n_experts, layer.has_shared, layer.banks, grids)


class Run:
    """Device buffers for one layer call and its numpy results."""

    def __init__(self, T, E, k, add_shared, H, I):
        kp = k + int(bool(add_shared))
        n_ids = E + int(bool(add_shared))
        i32 = dict(dtype=torch.int32, device="cuda")
        self.T, self.E, self.k, self.kp, self.H, self.I, self.add_shared = T, E, k, kp, H, I, int(bool(add_shared))
        self.ids = torch.zeros((T, kp), **i32)
        self.w = torch.zeros((T, kp), dtype=torch.float32, device="cuda")
        self.counts = torch.zeros(n_ids, **i32)
        self.offsets = torch.zeros(n_ids + 1, **i32)
        self.sorted_slot = torch.zeros(T * kp, **i32)
        self.slot_pos = torch.zeros(T * kp, **i32)
        self.work = torch.zeros(moe.work_ints(T, kp, n_ids), **i32)
        self.y = torch.zeros((T * kp, H), dtype=torch.float32, device="cuda")
        nws = moe.workspace_bytes(T, kp, H, I)
        self.ws = torch.zeros(max(nws // 4, 4), dtype=torch.float32, device="cuda")

    def route(self, logits_dev=None, ids=None, w=None):
        if logits_dev is None:
            self.ids[:, : self.k] = dev(ids)
            self.w[:, : self.k] = dev(w)
        moe.route_group(logits_dev, self.T, self.E, self.k, self.add_shared, self.ids, self.w, self.counts,
                        self.offsets, self.sorted_slot, self.slot_pos, self.work)

    def ffn(self, dl: moe.DeviceLayer, x_dev):
        moe.expert_ffn_q(dl.desc, x_dev, self.T, self.kp, self.sorted_slot, self.work, self.y, self.ws)

    def gateup(self, dl: moe.DeviceLayer, x_dev, h):
        moe.expert_gateup_q(dl.desc, x_dev, self.T, self.kp, self.sorted_slot, self.work, h)

    def down_accumulate(self, dl: moe.DeviceLayer, h, acc_dev):
        moe.expert_down_accumulate_q(dl.desc, h, self.T, self.kp, self.ids, self.w, self.slot_pos, acc_dev)

    def accumulate(self, acc_dev):
        moe.accumulate(self.y, self.w, self.ids, self.slot_pos, self.T, self.kp, self.H, acc_dev)

    def host(self):
        torch.cuda.synchronize()
        return {k: getattr(self, k).cpu().numpy() for k in
                ("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos", "work", "y")}


def run_layer(dl, x, k, add_shared, logits=None, ids=None, w=None, acc=None, decode=False):
    """Route, FFN and accumulate on the GPU.  Default: moe_expert_ffn_q (y in sorted
    order) then moe_accumulate.  decode=True: moe_expert_gateup_q then the fused
    moe_expert_down_accumulate_q (no y)."""
    T, H = x.shape
    r = Run(T, dl.desc.n_experts, k, add_shared, H, dl.desc.inter)
    r.route(None if logits is None else dev(logits), ids, w)
    acc_d = torch.zeros((T, H), dtype=torch.float32, device="cuda") if acc is None else dev(acc.astype(np.float32))
    if decode:
        h = torch.zeros((T * r.kp, dl.desc.inter), dtype=torch.float32, device="cuda")
        r.gateup(dl, dev(x), h)
        r.down_accumulate(dl, h, acc_d)
    else:
        r.ffn(dl, dev(x))
        r.accumulate(acc_d)
    out = r.host()
    out["acc"] = acc_d.cpu().numpy()
    return out


def y_in_slot_order(res) -> np.ndarray:
    """GPU y is in sorted order; slot s lives at row slot_pos[s]."""
    return res["y"][res["slot_pos"]]


def assert_rows_close(got: np.ndarray, ref: np.ndarray, what: str, rel: float = REL_TOL):
    got = np.atleast_2d(got).astype(np.float64)
    ref = np.atleast_2d(ref).astype(np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    err = np.abs(got - ref).max(axis=1)
    norm = np.linalg.norm(ref, axis=1)
    worst = float((err / np.maximum(norm, 1e-30)).max())
    log(f"  {what}: rows={len(ref)} worst max|err|/||ref||2 = {worst:.3e} (bound {rel:g})")
    assert np.all(err <= rel * norm), f"{what}: worst relative error {worst:.3e} > {rel}"
    return worst
