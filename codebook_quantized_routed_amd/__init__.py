"""Routed top-k MoE expert layer on codebook-quantized experts, for MI355X (gfx950).

A thin ctypes binding of ``libmoe.so`` (declared in include/moe.h).  Every function
here only marshals arguments: torch tensors are passed as device pointers and torch's
current HIP stream as the stream, and all the work runs in the library's kernels.  The
library must be built (``python codebook_quantized_routed_amd/_build.py``); importing
this package without it raises.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

IQ2XS_LIKE = 1
IQ1M_LIKE = 2
IQ1S_LIKE = 4  # repacked into IQ1M_LIKE banks when a layer is loaded
MAX_BANKS = 4
MAX_K = 16
MAX_IDS = 1024
MATVEC_MAX_TOKENS = 0  # above SMALL_BATCH_TOKENS: every expert with a token runs on the matrix cores
SMALL_BATCH_TOKENS = 16  # calls of at most this many tokens run every expert on the mat-vec kernels


def matvec_max_tokens(T: int) -> int:
    """Experts with at most this many of a call's T tokens run on the mat-vec kernels
    (m(T) in include/moe.h)."""
    return T if T <= SMALL_BATCH_TOKENS else MATVEC_MAX_TOKENS
MFMA_TILE_TOKENS = 16  # tokens per matrix-core tile (MOE_MFMA_TILE_TOKENS)
DECODE_SYNC_BYTES = 4352  # synchronisation words at the start of a decode workspace (MOE_DECODE_SYNC_BYTES)
DECODE_STATIC_BYTES = 73984  # the static per-device workspace of layer_decode_q_static
DECODE_ERROR_OFFSET = 128  # byte offset of the uint32 status word in it (MOE_DECODE_ERROR_OFFSET)
MAX_STACK_LAYERS = 256  # MOE_MAX_STACK_LAYERS

STATUS = {0: "MOE_OK", -1: "MOE_E_NULL", -2: "MOE_E_SHAPE", -3: "MOE_E_QTYPE", -4: "MOE_E_ALIGN",
          -5: "MOE_E_WORKSPACE", -6: "MOE_E_HIP"}

EXPORTS = ["moe_abi_version", "moe_status_string", "moe_last_hip_error", "moe_last_hip_error_string", "moe_grids_bytes", "moe_grids_expand", "moe_work_ints", "moe_workspace_bytes",
           "moe_route_group", "moe_expert_ffn_q", "moe_expert_gateup_q", "moe_expert_down_q",
           "moe_expert_down_accumulate_q", "moe_decode_workspace_bytes", "moe_layer_decode_q", "moe_layer_decode_q_static", "moe_accumulate",
           "moe_dequant_f32", "moe_rmsnorm", "moe_stack_workspace_bytes", "moe_stack_table_bytes", "moe_stack_table",
           "moe_stack_decode_q", "moe_router_logits", "moe_shared_weight", "moe_repack_iq1s"]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


class Bank(C.Structure):
    _fields_ = [("qtype", C.c_int32), ("first_expert", C.c_int32), ("n_experts", C.c_int32),
                ("reserved", C.c_int32), ("gate", C.c_void_p * 3), ("up", C.c_void_p * 3), ("down", C.c_void_p * 3)]


class Layer(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("inter", C.c_int32), ("n_experts", C.c_int32), ("has_shared", C.c_int32),
                ("n_banks", C.c_int32), ("reserved", C.c_int32), ("banks", Bank * MAX_BANKS), ("grids", C.c_void_p)]


def _load():
    # torch ships its own HIP runtime with the same soname as /opt/rocm's.  Loading torch
    # first makes libmoe bind to that already-mapped runtime; loading libmoe first would
    # map a second runtime next to torch's, and the two do not share devices.
    import torch  # noqa: F401

    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python codebook_quantized_routed_amd/_build.py`")
    L = C.CDLL(LIB_PATH)
    P, i32, sz = C.c_void_p, C.c_int32, C.c_size_t
    sig = {
        "moe_abi_version": (i32, []),
        "moe_status_string": (C.c_char_p, [C.c_int]),
        "moe_last_hip_error": (i32, []),
        "moe_last_hip_error_string": (C.c_char_p, []),
        "moe_grids_bytes": (sz, []),
        "moe_grids_expand": (C.c_int, [P, P, P, P]),
        "moe_work_ints": (i32, [i32, i32, i32]),
        "moe_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "moe_route_group": (C.c_int, [P, i32, i32, i32, i32, P, P, P, P, P, P, P, P]),
        "moe_expert_ffn_q": (C.c_int, [P, P, i32, i32, P, P, P, P, sz, P]),
        "moe_expert_gateup_q": (C.c_int, [P, P, i32, i32, P, P, P, P]),
        "moe_expert_down_q": (C.c_int, [P, P, i32, i32, P, P, P]),
        "moe_expert_down_accumulate_q": (C.c_int, [P, P, i32, i32, P, P, P, P, P]),
        "moe_decode_workspace_bytes": (sz, [i32, i32]),
        "moe_layer_decode_q": (C.c_int, [P, P, P, i32, i32, P, P, P, P, P, P, P, P, P, sz, P]),
        "moe_layer_decode_q_static": (C.c_int, [P, P, P, i32, i32, P, P, P, P, P, P, P, P, P, P]),
        "moe_accumulate": (C.c_int, [P, P, P, P, i32, i32, i32, P, P]),
        "moe_dequant_f32": (C.c_int, [i32, i32, i32, P, P, P, P, P, P]),
        "moe_rmsnorm": (C.c_int, [P, i32, i32, C.c_float, P, P]),
        "moe_stack_workspace_bytes": (sz, [i32, i32, i32, i32]),
        "moe_stack_table_bytes": (sz, [i32]),
        "moe_stack_table": (C.c_int, [P, i32, P, sz]),
        "moe_stack_decode_q": (C.c_int, [P, i32, P, P, P, i32, i32, C.c_float, P, P, P, sz, P]),
        "moe_router_logits": (C.c_int, [P, P, P, i32, i32, i32, P, P, P]),
        "moe_shared_weight": (C.c_int, [P, i32, i32, P, P]),
        "moe_repack_iq1s": (C.c_int, [P, P, P, i32, i32, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


lib = _load()


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn, st):
    if st != 0:
        msg = lib.moe_status_string(st).decode()
        if st == -6:
            msg += f": hipError {lib.moe_last_hip_error()} {lib.moe_last_hip_error_string().decode()}"
        raise MoeError(fn, st, msg)


def abi_version() -> int:
    return lib.moe_abi_version()


def grids_bytes() -> int:
    return lib.moe_grids_bytes()


def workspace_bytes(T: int, kprime: int, hidden: int, inter: int) -> int:
    return lib.moe_workspace_bytes(T, kprime, hidden, inter)


def grids_expand(compact_iq2, compact_iq1, grids, stream=None):
    _check("moe_grids_expand", lib.moe_grids_expand(_ptr(compact_iq2), _ptr(compact_iq1), _ptr(grids),
                                                    _stream(stream)))


def work_ints(T: int, kprime: int, n_ids: int) -> int:
    """Length (int32 elements) of the work list route_group writes."""
    return lib.moe_work_ints(T, kprime, n_ids)


def route_group(logits, T, E, k, add_shared, ids, w, counts, offsets, sorted_slot, slot_pos, work, stream=None):
    _check("moe_route_group", lib.moe_route_group(_ptr(logits), T, E, k, int(add_shared), _ptr(ids), _ptr(w),
                                                  _ptr(counts), _ptr(offsets), _ptr(sorted_slot), _ptr(slot_pos),
                                                  _ptr(work), _stream(stream)))


def expert_ffn_q(layer: Layer, x, T, kprime, sorted_slot, work, y, ws, stream=None):
    _check("moe_expert_ffn_q", lib.moe_expert_ffn_q(C.byref(layer), _ptr(x), T, kprime, _ptr(sorted_slot),
                                                    _ptr(work), _ptr(y), _ptr(ws), ws.numel() * ws.element_size(),
                                                    _stream(stream)))


def expert_gateup_q(layer: Layer, x, T, kprime, sorted_slot, work, h, stream=None):
    _check("moe_expert_gateup_q", lib.moe_expert_gateup_q(C.byref(layer), _ptr(x), T, kprime, _ptr(sorted_slot),
                                                          _ptr(work), _ptr(h), _stream(stream)))


def expert_down_q(layer: Layer, h, T, kprime, work, y, stream=None):
    _check("moe_expert_down_q", lib.moe_expert_down_q(C.byref(layer), _ptr(h), T, kprime, _ptr(work), _ptr(y),
                                                      _stream(stream)))


def expert_down_accumulate_q(layer: Layer, h, T, kprime, ids, w, slot_pos, acc, stream=None):
    _check("moe_expert_down_accumulate_q",
           lib.moe_expert_down_accumulate_q(C.byref(layer), _ptr(h), T, kprime, _ptr(ids), _ptr(w), _ptr(slot_pos),
                                            _ptr(acc), _stream(stream)))


def decode_workspace_bytes(kprime: int, inter: int) -> int:
    return lib.moe_decode_workspace_bytes(kprime, inter)


def layer_decode_q(layer: Layer, logits, x, k, add_shared, ids, w, counts, offsets, sorted_slot, slot_pos, work, acc,
                   ws, stream=None):
    """One decode step (one token) of the layer in one launch; ws: decode_workspace_bytes
    bytes, zero before the first call (reused as is by later calls)."""
    nbytes = ws.numel() * ws.element_size()
    _check("moe_layer_decode_q",
           lib.moe_layer_decode_q(C.byref(layer), _ptr(logits), _ptr(x), k, add_shared, _ptr(ids), _ptr(w),
                                  _ptr(counts), _ptr(offsets), _ptr(sorted_slot), _ptr(slot_pos), _ptr(work),
                                  _ptr(acc), _ptr(ws), nbytes, _stream(stream)))


def layer_decode_q_static(layer: Layer, logits, x, k, add_shared, ids, w, counts, offsets, sorted_slot, slot_pos, work,
                          acc, status, stream=None):
    """layer_decode_q with the library's static per-device workspace: the call allocates
    no device memory.  status: one 32-bit word (device) that receives the call's status
    word (nonzero: a wait timed out and the results are undefined)."""
    _check("moe_layer_decode_q_static",
           lib.moe_layer_decode_q_static(C.byref(layer), _ptr(logits), _ptr(x), k, add_shared, _ptr(ids), _ptr(w),
                                         _ptr(counts), _ptr(offsets), _ptr(sorted_slot), _ptr(slot_pos), _ptr(work),
                                         _ptr(acc), _ptr(status), _stream(stream)))


def decode_error(ws) -> int:
    """The status word of a one-launch decode workspace (moe_layer_decode_q,
    moe_stack_decode_q): nonzero when a wait of an earlier call timed out, which leaves
    that call's results undefined.  Waits for the device to finish its queued work."""
    import torch
    torch.cuda.synchronize(ws.device)
    return int(ws.view(torch.uint8)[DECODE_ERROR_OFFSET:DECODE_ERROR_OFFSET + 4].view(torch.int32).item())


def check_decode(ws) -> None:
    """Raises when the workspace's status word reports a timed-out wait."""
    err = decode_error(ws)
    if err:
        raise RuntimeError(f"one-launch decode: a wait for another workgroup's values timed out (status {err}); "
                           "the results are undefined and the workspace must be zeroed before reuse")


def accumulate(y, w, ids, slot_pos, T, kprime, hidden, acc, stream=None):
    _check("moe_accumulate", lib.moe_accumulate(_ptr(y), _ptr(w), _ptr(ids), _ptr(slot_pos), T, kprime, hidden,
                                                _ptr(acc), _stream(stream)))


def dequant_f32(qtype, rows, cols, s0, s1, s2, grids, out, stream=None):
    _check("moe_dequant_f32", lib.moe_dequant_f32(qtype, rows, cols, _ptr(s0), _ptr(s1), _ptr(s2), _ptr(grids),
                                                  _ptr(out), _stream(stream)))


def rmsnorm(h, T, hidden, eps, x, stream=None):
    _check("moe_rmsnorm", lib.moe_rmsnorm(_ptr(h), T, hidden, eps, _ptr(x), _stream(stream)))


def router_logits(x, wr, T, hidden, E, logits, wsg=None, shared_w=None, stream=None):
    """logits [T][E] = x [T][hidden] wr[E][hidden]^T; with wsg, shared_w [T] = sigmoid(x . wsg)."""
    _check("moe_router_logits", lib.moe_router_logits(_ptr(x), _ptr(wr), _ptr(wsg), T, hidden, E, _ptr(logits),
                                                      _ptr(shared_w), _stream(stream)))


def shared_weight(shared_w, T, kprime, w, stream=None):
    """w[t][kprime - 1] = shared_w[t] (the gated shared expert's weight)."""
    _check("moe_shared_weight", lib.moe_shared_weight(_ptr(shared_w), T, kprime, _ptr(w), _stream(stream)))


def repack_iq1s(ql, qh, d, rows, cols, ql_out, qh_out, sd_out, stream=None):
    """IQ1_S-like streams of rows x cols -> the IQ1_M-like layout (same weights, exactly)."""
    _check("moe_repack_iq1s", lib.moe_repack_iq1s(_ptr(ql), _ptr(qh), _ptr(d), rows, cols, _ptr(ql_out), _ptr(qh_out),
                                                  _ptr(sd_out), _stream(stream)))


def stack_workspace_bytes(n_layers: int, kprime: int, hidden: int, inter: int) -> int:
    return lib.moe_stack_workspace_bytes(n_layers, kprime, hidden, inter)


def stack_table_bytes(n_layers: int) -> int:
    return lib.moe_stack_table_bytes(n_layers)


def stack_layers(layers) -> C.Array:
    """A host array of the ``Layer`` descriptors of a chain, in order."""
    arr = (Layer * len(layers))()
    for i, L in enumerate(layers):
        arr[i] = L
    return arr


def stack_prepare(layer_array, ws):
    """Set-up of a stack decode workspace (blocking): zeroes it and copies the layers'
    table in after the synchronisation words.  ``layer_array`` from ``stack_layers``."""
    import torch
    n = len(layer_array)
    nbytes = stack_table_bytes(n)
    host = (C.c_uint8 * nbytes)()
    _check("moe_stack_table", lib.moe_stack_table(layer_array, n, host, nbytes))
    ws8 = ws.view(torch.uint8)
    ws8.zero_()
    ws8[DECODE_SYNC_BYTES:DECODE_SYNC_BYTES + nbytes].copy_(torch.frombuffer(host, dtype=torch.uint8))
    torch.cuda.synchronize(ws.device)


def stack_decode_q(layer_array, logits, h_in, h_out, k, add_shared, eps, ids, w, ws, stream=None):
    """One decode step of the chain h <- h + MoE_l(RMSNorm(h)) over every layer, one launch;
    ``ws`` prepared by ``stack_prepare`` with the same layers."""
    nbytes = ws.numel() * ws.element_size()
    _check("moe_stack_decode_q",
           lib.moe_stack_decode_q(layer_array, len(layer_array), _ptr(logits), _ptr(h_in), _ptr(h_out), k,
                                  int(add_shared), eps, _ptr(ids), _ptr(w), _ptr(ws), nbytes, _stream(stream)))


# ----------------------------------------------------------------------------- device data

class DeviceLayer:
    """A routed layer resident in device memory.

    ``banks`` is a sequence of objects with ``qtype``, ``first``, ``n`` and ``gate``,
    ``up``, ``down`` (each three host byte arrays [n][stream bytes]).  The streams are
    copied once to device tensors; ``self.desc`` is the ``moe_layer`` for the calls.
    """

    def __init__(self, hidden, inter, n_experts, has_shared, banks, grids, device="cuda"):
        import torch
        if len(banks) > MAX_BANKS:
            raise ValueError("too many banks")
        self.tensors = []
        d = Layer()
        d.hidden, d.inter, d.n_experts, d.has_shared = hidden, inter, n_experts, int(has_shared)
        d.n_banks = len(banks)
        d.grids = grids.data_ptr()
        self.grids = grids
        self.bytes = 0
        for i, b in enumerate(banks):
            bd = d.banks[i]
            # IQ1_S-like banks are repacked on the device into the IQ1_M-like layout
            bd.qtype = IQ1M_LIKE if b.qtype == IQ1S_LIKE else b.qtype
            bd.first_expert, bd.n_experts = b.first, b.n
            for name in ("gate", "up", "down"):
                arr = getattr(bd, name)
                streams = [torch.from_numpy(host.reshape(-1)).to(device) for host in getattr(b, name)]
                if b.qtype == IQ1S_LIKE:
                    rows, cols = (inter, hidden) if name != "down" else (hidden, inter)
                    n_rows = b.n * rows
                    out = [streams[0], torch.empty(n_rows * cols // 16, dtype=torch.uint8, device=device),
                           torch.empty(n_rows * cols // 256 * 8, dtype=torch.uint8, device=device)]
                    repack_iq1s(streams[0], streams[1], streams[2], n_rows, cols, out[0], out[1], out[2])
                    torch.cuda.synchronize(out[0].device)
                    streams = out
                for j, t in enumerate(streams):
                    self.tensors.append(t)
                    self.bytes += t.numel()
                    arr[j] = t.data_ptr()
        self.desc = d

    def copy(self) -> "DeviceLayer":
        """Another resident copy of the same layer: the same bytes in new device buffers
        (a device-to-device copy of every stream)."""
        other = DeviceLayer.__new__(DeviceLayer)
        other.grids, other.bytes = self.grids, self.bytes
        other.tensors = [t.clone() for t in self.tensors]
        d = Layer()
        C.memmove(C.addressof(d), C.addressof(self.desc), C.sizeof(Layer))
        remap = {t.data_ptr(): c.data_ptr() for t, c in zip(self.tensors, other.tensors)}
        for i in range(d.n_banks):
            for name in ("gate", "up", "down"):
                arr = getattr(d.banks[i], name)
                for j in range(3):
                    arr[j] = remap[arr[j]]
        other.desc = d
        return other

    def __del__(self):
        self.tensors = []
