"""The no-allocation layer decode (moe_layer_decode_q_static) against moe_layer_decode_q.

Both run the one-launch decode kernel; the static variant keeps its workspace in the
library's per-device array instead of a caller buffer.  Every output (routing arrays
and the accumulator) must be the same bits as the workspace entry point's on the same
inputs, over consecutive calls of different sizes that share the one static array:
the field shape, then a smaller layer (fewer slots, narrower inter), then the field
shape again with an explicit selection.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

try:
    import codebook_quantized_routed_amd as moe  # noqa: E402
except ImportError:
    if torch.cuda.device_count() > 0:
        raise                      # on a GPU machine a missing library is an error
    pytest.skip("HIP library not built (CPU-only machine)", allow_module_level=True)
import synth  # noqa: E402
from gpu_util import Run, dev, device_grids, device_layer, log  # noqa: E402

IQ2, IQ1 = synth.QTYPE_IQ2XS, synth.QTYPE_IQ1M

# name: (banks, inter, E, shared, k)
SHAPES = {
    "field_iq2_top10_shared": ([(IQ2, 512)], 512, 512, 1, 10),   # kprime 11, inter 512
    "small_iq1_i256_top4": ([(IQ1, 16)], 256, 16, 1, 4),          # kprime 5, inter 256
}
H = 2048
KEYS = ("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos", "work")


@pytest.fixture(scope="module")
def grids(grids_compact):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return device_grids(*grids_compact)


def one_call(dl, name, call, logits, sel, static):
    """One decode of token x with acc0 added in; returns the routing arrays and acc."""
    banks, I, E, shared, k = SHAPES[name]
    x = synth.activations(1, H, tag=f"NA/{name}/{call}/x")
    acc0 = synth.activations(1, H, tag=f"NA/{name}/{call}/acc")
    r = Run(1, E, k, shared, H, I)
    if sel is not None:
        r.ids[:, :k] = dev(sel[0])
        r.w[:, :k] = dev(sel[1])
    acc = dev(acc0.astype(np.float32))
    lg = None if logits is None else dev(logits)
    if static:
        status = torch.full((4,), -1, dtype=torch.int32, device="cuda")
        moe.layer_decode_q_static(dl.desc, lg, dev(x), k, shared, r.ids, r.w, r.counts, r.offsets, r.sorted_slot,
                                  r.slot_pos, r.work, acc, status)
        err = int(status[0].item())
    else:
        ws = torch.zeros(moe.decode_workspace_bytes(k + shared, I) // 4, dtype=torch.int32, device="cuda")
        moe.layer_decode_q(dl.desc, lg, dev(x), k, shared, r.ids, r.w, r.counts, r.offsets, r.sorted_slot,
                           r.slot_pos, r.work, acc, ws)
        err = moe.decode_error(ws)
    out = r.host()
    out["acc"] = acc.cpu().numpy()
    return out, err


def test_static_decode_matches_workspace_decode(grids):
    layers = {}
    for name, (banks, I, E, shared, k) in SHAPES.items():
        sl = synth.make_layer(banks, hidden=H, inter=I, n_experts=E, has_shared=shared, tag=f"NA/{name}")
        layers[name] = device_layer(sl, grids)
    # the field shape, a smaller call, then the field shape with an explicit selection
    plan = [("field_iq2_top10_shared", "logits"), ("small_iq1_i256_top4", "logits"),
            ("field_iq2_top10_shared", "explicit")]
    for call, (name, mode) in enumerate(plan):
        banks, I, E, shared, k = SHAPES[name]
        need = moe.decode_workspace_bytes(k + shared, I)
        assert need <= moe.DECODE_STATIC_BYTES
        log(f"static decode call {call}: {name} ({mode}), workspace {need} of {moe.DECODE_STATIC_BYTES} bytes")
        if mode == "logits":
            logits, sel = synth.logits(1, E, tag=f"NA/{name}/{call}/l"), None
        else:
            ids = np.argsort(synth.u64(3, f"NA/{name}/ids", E), kind="stable")[:k].astype(np.int32)[None, :]
            wts = synth.uniform(3, f"NA/{name}/w", k).astype(np.float32)[None, :]
            logits, sel = None, (ids, wts)
        ref, ref_err = one_call(layers[name], name, call, logits, sel, static=False)
        got, got_err = one_call(layers[name], name, call, logits, sel, static=True)
        assert ref_err == 0 and got_err == 0, (ref_err, got_err)
        for key in KEYS:
            np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
        assert np.array_equal(got["acc"].view(np.uint32), ref["acc"].view(np.uint32)), "acc bits"
        assert np.abs(got["acc"]).max() > 0
