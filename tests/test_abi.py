"""The C-ABI library loads, exports every function include/moe.h declares, and rejects
bad arguments on the host before anything is enqueued (CPU only: every call here fails
validation, so no HIP call is made)."""
import ctypes as C
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

moe = pytest.importorskip("codebook_quantized_routed_amd")
lib = moe.lib

A = 0x10000          # an aligned fake device address: never dereferenced, validation fails first
MIS = 0x10004        # misaligned


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src))
    return names


def test_exports_every_declared_function():
    names = declared_functions()
    assert "moe_route_group" in names and "moe_expert_ffn_q" in names and "moe_accumulate" in names
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert set(moe.EXPORTS) == names


def test_binding_constants_match_header():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    defs = dict(re.findall(r"#define (MOE_[A-Z0-9_]+) (\d+)", src))
    assert int(defs["MOE_ABI_VERSION"]) == moe.abi_version()
    assert int(defs["MOE_MAX_BANKS"]) == moe.MAX_BANKS
    assert int(defs["MOE_MAX_K"]) == moe.MAX_K
    assert int(defs["MOE_MAX_IDS"]) == moe.MAX_IDS
    assert int(defs["MOE_MATVEC_MAX_TOKENS"]) == moe.MATVEC_MAX_TOKENS
    assert int(defs["MOE_SMALL_BATCH_TOKENS"]) == moe.SMALL_BATCH_TOKENS
    assert int(defs["MOE_MFMA_TILE_TOKENS"]) == moe.MFMA_TILE_TOKENS
    assert int(defs["MOE_DECODE_SYNC_BYTES"]) == moe.DECODE_SYNC_BYTES
    assert int(defs["MOE_DECODE_ERROR_OFFSET"]) == moe.DECODE_ERROR_OFFSET
    assert int(defs["MOE_DECODE_STATIC_BYTES"]) == moe.DECODE_STATIC_BYTES
    # the static workspace holds the largest valid call: 16 routed + 1 shared slots at inter 512
    assert moe.decode_workspace_bytes(17, 512) == moe.DECODE_STATIC_BYTES
    assert moe.DECODE_STATIC_BYTES % 16 == 0
    assert int(defs["MOE_MAX_STACK_LAYERS"]) == moe.MAX_STACK_LAYERS
    assert int(defs["MOE_Q_IQ1S_LIKE"]) == moe.IQ1S_LIKE
    assert moe.decode_workspace_bytes(11, 512) - 11 * 512 * 8 == moe.DECODE_SYNC_BYTES


def test_version_strings_sizes():
    assert moe.abi_version() == 11
    for st in moe.STATUS:
        assert lib.moe_status_string(st)
    assert moe.grids_bytes() >= 512 * 8 + 2048 * 8
    assert moe.workspace_bytes(1, 11, 2048, 512) == 11 * 512 * 4
    # the work list: n_ids + 1 records, then room for the matrix-core tiles
    assert moe.work_ints(1, 11, 513) == 4 * 514                       # one token: no expert above 1 slot
    assert moe.work_ints(16, 11, 513) == 4 * 514                      # small batch: every expert on the mat-vec path
    n17 = min(513, 17 * 11 // (moe.MATVEC_MAX_TOKENS + 1))
    assert moe.work_ints(17, 11, 513) == 4 * (514 + n17 + (17 * 11 + 15) // 16)
    n_wide = min(513, 256 * 10 // (moe.MATVEC_MAX_TOKENS + 1))
    assert moe.work_ints(256, 10, 512) == 4 * (513 + min(512, n_wide) + (2560 + 15) // 16)
    assert moe.work_ints(0, 11, 513) == 0
    assert moe.workspace_bytes(0, 11, 2048, 512) == 0
    assert moe.workspace_bytes(1, 11, 2048, 300) == 0


def rg(**kw):
    a = dict(logits=A, T=1, E=512, k=10, add_shared=1, ids=A, w=A, counts=A, offsets=A, ss=A, sp=A, act=A)
    a.update(kw)
    return lib.moe_route_group(a["logits"], a["T"], a["E"], a["k"], a["add_shared"], a["ids"], a["w"], a["counts"],
                               a["offsets"], a["ss"], a["sp"], a["act"], None)


def test_route_group_rejects():
    assert rg(ids=None) == -1
    assert rg(act=None) == -1
    assert rg(k=0) == -2
    assert rg(k=17) == -2
    assert rg(E=8, k=9) == -2
    assert rg(T=0) == -2
    assert rg(E=1024, add_shared=1) == -2
    assert rg(add_shared=2) == -2
    assert rg(w=MIS) == -4
    assert rg(logits=MIS) == -4


def layer(**kw):
    d = moe.Layer()
    d.hidden, d.inter, d.n_experts, d.has_shared, d.n_banks = 2048, 512, 512, 1, 1
    d.grids = A
    b = d.banks[0]
    b.qtype, b.first_expert, b.n_experts = 1, 0, 513
    for name in ("gate", "up", "down"):
        arr = getattr(b, name)
        for j in range(3):
            arr[j] = A
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def ffn(d, ws_bytes=1 << 30, **kw):
    a = dict(x=A, T=1, kp=11, ss=A, work=A, y=A, ws=A)
    a.update(kw)
    return lib.moe_expert_ffn_q(C.byref(d), a["x"], a["T"], a["kp"], a["ss"], a["work"], a["y"], a["ws"],
                                ws_bytes, None)


def test_expert_ffn_rejects():
    assert lib.moe_expert_ffn_q(None, A, 1, 11, A, A, A, A, 1 << 30, None) == -1
    assert lib.moe_expert_gateup_q(C.byref(layer()), A, 1, 11, A, None, A, None) == -1
    assert lib.moe_expert_down_q(C.byref(layer()), A, 1, 11, A, MIS, None) == -4
    assert lib.moe_expert_down_accumulate_q(C.byref(layer()), A, 1, 0, A, A, A, A, None) == -2
    assert ffn(layer(), x=None) == -1
    assert ffn(layer(grids=None)) == -1
    assert ffn(layer(hidden=300)) == -2
    for bad in (768, 1536, 4096, 128):              # widths other than 256, 512, 1024, 2048
        assert ffn(layer(hidden=bad)) == -2
        assert ffn(layer(inter=bad)) == -2
    assert ffn(layer(inter=4096)) == -2
    assert ffn(layer(n_banks=0)) == -2
    assert ffn(layer(n_experts=600)) == -2          # banks no longer cover E + shared
    assert ffn(layer(), T=0) == -2
    assert ffn(layer(), kp=18) == -2
    assert ffn(layer(), ws_bytes=100) == -5
    assert ffn(layer(), y=MIS) == -4
    assert ffn(layer(grids=MIS)) == -4
    d = layer()
    d.banks[0].qtype = 3
    assert ffn(d) == -3
    d = layer()
    d.banks[0].up[1] = None
    assert ffn(d) == -1
    d = layer()
    d.banks[0].down[2] = MIS
    assert ffn(d) == -4
    d = layer()
    d.banks[0].first_expert = 1
    assert ffn(d) == -2


def test_other_rejects():
    assert lib.moe_accumulate(None, A, A, A, 1, 11, 2048, A, None) == -1
    assert lib.moe_accumulate(A, A, A, A, 1, 11, 2000, A, None) == -2
    assert lib.moe_accumulate(A, A, A, A, 1, 18, 2048, A, None) == -2
    assert lib.moe_accumulate(A, A, A, MIS, 1, 11, 2048, A, None) == -4
    assert lib.moe_dequant_f32(3, 8, 256, A, A, A, A, A, None) == -3
    assert lib.moe_dequant_f32(1, 8, 100, A, A, A, A, A, None) == -2
    assert lib.moe_dequant_f32(1, 7, 256, A, A, A, A, A, None) == -2
    assert lib.moe_dequant_f32(1, 8, 256, A, A, None, A, A, None) == -1
    assert lib.moe_dequant_f32(1, 8, 256, A, A, A, A, MIS, None) == -4
    assert lib.moe_rmsnorm(None, 1, 2048, 1e-6, A, None) == -1
    assert lib.moe_rmsnorm(A, 0, 2048, 1e-6, A, None) == -2
    assert lib.moe_rmsnorm(A, 1, 2048, float("nan"), A, None) == -2
    assert lib.moe_grids_expand(A, None, A, None) == -1
    assert lib.moe_grids_expand(A, A, MIS, None) == -4


def test_layer_decode_rejects():
    d = layer()
    ws_need = moe.decode_workspace_bytes(11, 512)
    assert ws_need == 4352 + 11 * 512 * 8

    def call(d=d, logits=A, x=A, k=10, add_shared=1, ws=A, ws_bytes=ws_need, acc=A):
        return lib.moe_layer_decode_q(C.byref(d), logits, x, k, add_shared, A, A, A, A, A, A, A, acc, ws, ws_bytes,
                                      None)
    assert lib.moe_layer_decode_q(None, A, A, 10, 1, A, A, A, A, A, A, A, A, A, ws_need, None) == -1
    assert call(x=None) == -1
    assert call(ws=None) == -1
    assert call(logits=MIS) == -4
    assert call(acc=MIS) == -4
    assert call(k=0) == -2
    assert call(k=17) == -2
    assert call(add_shared=0) == -2                     # must match the layer's shared expert
    assert call(d=layer(hidden=1024, n_experts=512)) == -2
    assert call(d=layer(inter=1024)) == -2
    assert call(ws_bytes=ws_need - 4) == -5


def test_layer_decode_static_rejects():
    """The no-allocation variant validates its arguments before any HIP call."""
    d = layer()

    def call(d=d, logits=A, x=A, k=10, add_shared=1, acc=A, status=A):
        return lib.moe_layer_decode_q_static(C.byref(d), logits, x, k, add_shared, A, A, A, A, A, A, A, acc, status,
                                             None)
    assert lib.moe_layer_decode_q_static(None, A, A, 10, 1, A, A, A, A, A, A, A, A, A, None) == -1
    assert call(x=None) == -1
    assert call(status=None) == -1
    assert call(status=MIS) == -4
    assert call(logits=MIS) == -4
    assert call(acc=MIS) == -4
    assert call(k=0) == -2
    assert call(k=17) == -2
    assert call(add_shared=0) == -2
    assert call(d=layer(hidden=1024, n_experts=512)) == -2
    assert call(d=layer(inter=1024)) == -2


def test_stack_table_and_rejects():
    n = 3
    arr = moe.stack_layers([layer(), layer(), layer()])
    tb = moe.stack_table_bytes(n)
    assert tb > 0 and tb % n == 0 and moe.stack_table_bytes(0) == 0 and moe.stack_table_bytes(257) == 0
    # sync words, the table (rounded up to 256 bytes), then per layer h and residual pairs
    ws_need = moe.stack_workspace_bytes(n, 11, 2048, 512)
    assert ws_need == (4352 + tb + 255) // 256 * 256 + n * (11 * 512 + 2048) * 8
    assert moe.stack_workspace_bytes(0, 11, 2048, 512) == 0
    assert moe.stack_workspace_bytes(3, 18, 2048, 512) == 0
    host = (C.c_uint8 * tb)()
    assert lib.moe_stack_table(arr, n, host, tb) == 0
    assert any(host)                                    # the table holds the layers' pointers
    assert lib.moe_stack_table(arr, n, host, tb - 1) == -2
    assert lib.moe_stack_table(arr, n, None, tb) == -1
    assert lib.moe_stack_table(None, n, host, tb) == -1
    assert lib.moe_stack_table(arr, 0, host, tb) == -2
    for bad, code in ((layer(inter=256), -2),              # layers of different shapes
                      (layer(grids=A + 256), -2),          # another grid table
                      (layer(hidden=1024), -2),
                      (layer(grids=None), -1),
                      (layer(n_experts=600), -2)):
        assert lib.moe_stack_table(moe.stack_layers([layer(), bad]), 2, host, tb) == code

    H = 2048 * 4

    def call(arr=arr, n=n, logits=A, h_in=A, h_out=A + H, k=10, add_shared=1, eps=1e-6, ids=A, w=A, ws=A,
             ws_bytes=ws_need):
        return lib.moe_stack_decode_q(arr, n, logits, h_in, h_out, k, add_shared, eps, ids, w, ws, ws_bytes, None)
    assert call(logits=None) == -1
    assert call(h_in=None) == -1
    assert call(ws=None) == -1
    assert call(ids=None) == -1                         # ids and w: both or neither
    assert call(w=None) == -1
    assert call(h_out=MIS) == -4
    assert call(h_out=A) == -2                          # input and output overlap
    assert call(h_out=A + H - 16) == -2
    assert call(k=0) == -2
    assert call(add_shared=0) == -2
    assert call(eps=float("nan")) == -2
    assert call(n=0) == -2
    assert call(ws_bytes=ws_need - 8) == -5
    assert call(arr=moe.stack_layers([layer(), layer(inter=256), layer()])) == -2


def test_router_rejects():
    def call(x=A, wr=A, wsg=A, T=1, H=2048, E=512, lg=A, sw=A):
        return lib.moe_router_logits(x, wr, wsg, T, H, E, lg, sw, None)
    assert call(x=None) == -1
    assert call(lg=None) == -1
    assert call(wsg=None) == -1                         # gate vector and gate output: both or neither
    assert call(sw=None) == -1
    assert call(wr=MIS) == -4
    assert call(T=0) == -2
    assert call(H=300) == -2
    assert call(E=0) == -2
    assert call(E=1025) == -2
    assert lib.moe_shared_weight(None, 1, 11, A, None) == -1
    assert lib.moe_shared_weight(A, 1, 1, A, None) == -2
    assert lib.moe_shared_weight(A, 0, 11, A, None) == -2
    assert lib.moe_shared_weight(A, 1, 11, MIS, None) == -4


def test_repack_rejects():
    def call(ql=A, qh=A, d=A, rows=8, cols=256, o0=A, o1=A, o2=A):
        return lib.moe_repack_iq1s(ql, qh, d, rows, cols, o0, o1, o2, None)
    assert call(ql=None) == -1
    assert call(o2=None) == -1
    assert call(qh=MIS) == -4
    assert call(o1=MIS) == -4
    assert call(rows=0) == -2
    assert call(cols=300) == -2
    assert call(cols=0) == -2
    assert call(rows=1 << 30, cols=2048) == -2        # 2^33 super-blocks


# The HIP runtime functions the library may call: kernel registration and launch, error
# queries, the device id and attributes, and the static workspace's symbol lookup.
# Nothing that copies, synchronises with the host, allocates, frees or sets memory.
ALLOWED_HIP_IMPORTS = {
    "__hipPopCallConfiguration", "__hipPushCallConfiguration", "__hipRegisterFatBinary",
    "__hipRegisterFunction", "__hipRegisterVar", "__hipUnregisterFatBinary",
    "hipLaunchKernel", "hipGetLastError", "hipGetErrorString", "hipGetDevice",
    "hipDeviceGetAttribute", "hipGetSymbolAddress",
}


def test_library_imports_no_copy_sync_or_alloc():
    """Every entry point only enqueues kernels: the library's dynamic imports hold no
    memcpy, memset, synchronisation, allocation or host-registration function, so no
    call can copy to or from the host, wait for the device or allocate (the analogue
    of the pages' zero-bytes-read check during the routed layer)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm (binutils) not installed")
    out = subprocess.run([nm, "-D", "--undefined-only", moe.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    hip = {line.split()[-1].split("@")[0] for line in out.splitlines() if "hip" in line.lower()}
    assert "hipLaunchKernel" in hip
    assert hip <= ALLOWED_HIP_IMPORTS, sorted(hip - ALLOWED_HIP_IMPORTS)
    for bad in ("Memcpy", "Memset", "Malloc", "Free", "Synchronize", "HostRegister", "HostAlloc"):
        assert not any(bad.lower() in s.lower() for s in hip), bad


def test_forced_hip_error_reports_moe_e_hip():
    """A launch the runtime refuses returns MOE_E_HIP, and the thread's last HIP error
    and its text are readable.  Forced from the host: a child process in which no GPU
    is visible, so the launch fails before any kernel could touch the (fake) pointers.
    Skipped where this process sees a GPU."""
    import subprocess
    import sys
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible; the forced error runs on CPU-only machines")
    code = (
        "import ctypes as C\n"
        "import codebook_quantized_routed_amd as moe\n"
        "A = C.c_void_p(1 << 20)\n"
        "st = moe.lib.moe_accumulate(A, A, A, A, 1, 11, 2048, A, None)\n"
        "print(st, moe.lib.moe_last_hip_error(), moe.lib.moe_last_hip_error_string().decode())\n"
    )
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1", CUDA_VISIBLE_DEVICES="-1",
               PYTHONPATH=ROOT + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    st, err, msg = r.stdout.strip().splitlines()[-1].split(" ", 2)
    assert int(st) == -6                                   # MOE_E_HIP
    assert int(err) != 0 and msg                           # the hipError_t and its text
    assert lib.moe_status_string(-6)
