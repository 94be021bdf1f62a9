"""Guard words around every output and workspace: no entry point writes outside the
buffers it is given, or into its inputs.

Each output (and workspace) sits between two 4 KiB guard bands of a fixed byte pattern
in one device allocation; after each call the bands must be unchanged.  Inputs are
compared with copies taken before the calls.  Covered: routing and grouping, the FFN
calls (mat-vec tokens, the 2-8 token matrix-core decode gate/up, 16-token tiles),
down + accumulate, accumulate, RMSNorm, the router projection, the one-launch layer
decode and its static-workspace variant, and the one-launch stack decode, at 1, 7 and
40 tokens on a mixed-format layer with a shared expert.
"""
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
from gpu_util import dev, device_grids, device_layer, log  # noqa: E402

IQ2, IQ1 = synth.QTYPE_IQ2XS, synth.QTYPE_IQ1M
H, I, E, K = 2048, 512, 64, 6
PAD = 4096
PATTERN = 0xA5


class Guarded:
    """A device buffer of n elements between two PAD-byte guard bands."""

    def __init__(self, n, dtype, fill=0):
        esz = torch.empty(0, dtype=dtype).element_size()
        self.nbytes = max(int(n), 1) * esz
        self.raw = torch.full((2 * PAD + self.nbytes,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[PAD:PAD + self.nbytes].view(dtype)
        self.t.fill_(fill)

    def check(self, what):
        torch.cuda.synchronize()
        lo, hi = self.raw[:PAD], self.raw[PAD + self.nbytes:]
        assert bool((lo == PATTERN).all()), f"{what}: write below the buffer"
        assert bool((hi == PATTERN).all()), f"{what}: write past the end of the buffer"


@pytest.fixture(scope="module")
def layer(grids_compact):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    grids = device_grids(*grids_compact)
    sl = synth.make_layer([(IQ2, 32), (IQ1, 32)], hidden=H, inter=I, n_experts=E, has_shared=1, tag="G/layer")
    return grids, device_layer(sl, grids)


def routed(T, kp):
    n_ids = E + 1
    return {"ids": Guarded(T * kp, torch.int32), "w": Guarded(T * kp, torch.float32),
            "counts": Guarded(n_ids, torch.int32), "offsets": Guarded(n_ids + 1, torch.int32),
            "sorted_slot": Guarded(T * kp, torch.int32), "slot_pos": Guarded(T * kp, torch.int32),
            "work": Guarded(moe.work_ints(T, kp, n_ids), torch.int32)}


def check_all(bufs, what):
    for name, g in bufs.items():
        g.check(f"{what}: {name}")


@pytest.mark.parametrize("T", [1, 7, 40])
def test_guards_split_calls(layer, T):
    grids, dl = layer
    kp = K + 1
    log(f"guards: split calls, T={T}")
    x = dev(synth.activations(T, H, tag=f"G/{T}/x"))
    lg = dev(synth.logits(T, E, tag=f"G/{T}/l"))
    x0, lg0 = x.clone(), lg.clone()
    r = routed(T, kp)
    moe.route_group(lg, T, E, K, 1, *(r[k].t for k in ("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos",
                                                          "work")))
    check_all(r, "route_group")
    y = Guarded(T * kp * H, torch.float32)
    ws = Guarded(moe.workspace_bytes(T, kp, H, I) // 4, torch.float32)
    moe.expert_ffn_q(dl.desc, x, T, kp, r["sorted_slot"].t, r["work"].t, y.t, ws.t)
    y.check("expert_ffn_q: y")
    ws.check("expert_ffn_q: ws")
    h = Guarded(T * kp * I, torch.float32)
    moe.expert_gateup_q(dl.desc, x, T, kp, r["sorted_slot"].t, r["work"].t, h.t)
    h.check("expert_gateup_q: h")
    y2 = Guarded(T * kp * H, torch.float32)
    moe.expert_down_q(dl.desc, h.t, T, kp, r["work"].t, y2.t)
    y2.check("expert_down_q: y")
    acc = Guarded(T * H, torch.float32)
    moe.expert_down_accumulate_q(dl.desc, h.t, T, kp, r["ids"].t, r["w"].t, r["slot_pos"].t, acc.t)
    acc.check("expert_down_accumulate_q: acc")
    acc2 = Guarded(T * H, torch.float32)
    moe.accumulate(y.t, r["w"].t, r["ids"].t, r["slot_pos"].t, T, kp, H, acc2.t)
    acc2.check("accumulate: acc")
    xn = Guarded(T * H, torch.float32)
    moe.rmsnorm(acc2.t, T, H, 1e-6, xn.t)
    xn.check("rmsnorm: x")
    wr = dev(synth.activations(E, H, tag="G/wr"))
    wsg = dev(synth.activations(1, H, tag="G/wsg"))
    logits = Guarded(T * E, torch.float32)
    sw = Guarded(T, torch.float32)
    moe.router_logits(x, wr, T, H, E, logits.t, wsg=wsg, shared_w=sw.t)
    logits.check("router_logits: logits")
    sw.check("router_logits: shared_w")
    # inputs intact; the outputs were written
    assert torch.equal(x, x0) and torch.equal(lg, lg0)
    assert int(torch.count_nonzero(acc.t)) > 0 and int(torch.count_nonzero(logits.t)) > 0


def test_guards_one_launch_layer(layer):
    grids, dl = layer
    kp = K + 1
    log("guards: one-launch layer decode and its static variant")
    x = dev(synth.activations(1, H, tag="G/d/x"))
    lg = dev(synth.logits(1, E, tag="G/d/l"))
    x0, lg0 = x.clone(), lg.clone()
    outs = []
    for static in (False, True):
        r = routed(1, kp)
        acc = Guarded(H, torch.float32)
        args = [r[k].t for k in ("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos", "work")]
        if static:
            status = Guarded(4, torch.int32, fill=-1)
            moe.layer_decode_q_static(dl.desc, lg, x, K, 1, *args, acc.t, status.t)
            status.check("layer_decode_q_static: status")
            assert int(status.t[0].item()) == 0
        else:
            ws = Guarded(moe.decode_workspace_bytes(kp, I) // 4, torch.int32)
            moe.layer_decode_q(dl.desc, lg, x, K, 1, *args, acc.t, ws.t)
            ws.check("layer_decode_q: ws")
            assert moe.decode_error(ws.t) == 0
        check_all(r, "layer decode")
        acc.check("layer decode: acc")
        outs.append(acc.t.clone())
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(x, x0) and torch.equal(lg, lg0)


def test_guards_one_launch_stack(layer):
    grids, dl = layer
    kp = K + 1
    n = 2
    log("guards: one-launch stack decode, 2 layers")
    arr = moe.stack_layers([dl.desc, dl.desc])
    ws = Guarded(moe.stack_workspace_bytes(n, kp, H, I) // 4, torch.int32)
    moe.stack_prepare(arr, ws.t)
    h_in = dev(synth.activations(1, H, tag="G/s/h"))
    lg = dev(synth.logits(n, E, tag="G/s/l"))
    h0, lg0 = h_in.clone(), lg.clone()
    h_out = Guarded(H, torch.float32)
    ids = Guarded(n * kp, torch.int32)
    w = Guarded(n * kp, torch.float32)
    moe.stack_decode_q(arr, lg, h_in, h_out.t, K, 1, 1e-6, ids.t, w.t, ws.t)
    h_out.check("stack_decode_q: h_out")
    ids.check("stack_decode_q: ids")
    w.check("stack_decode_q: w")
    ws.check("stack_decode_q: ws")
    assert moe.decode_error(ws.t) == 0
    assert torch.equal(h_in, h0) and torch.equal(lg, lg0)
    assert bool(torch.isfinite(h_out.t).all())
