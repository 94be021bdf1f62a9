"""GPU parity of the router projection (moe_router_logits) and of the gated shared expert
(moe_shared_weight), through the C ABI, against the oracle:

- logits within fp32 rounding of the exact dot products: |gpu - exact| <= 64 * 2^-24 *
  sum_c |x_c w_c| (each GPU dot takes at most 8 fused multiply-adds per lane and six
  levels of a sum tree: well under 64 roundings of terms bounded by that sum);
- the gate within the same bound scaled by the sigmoid's slope (<= 1/4), plus the
  rounding of the sigmoid itself;
- a token's logits are the same bits whatever the batch and its position in it;
- ragged shapes: token counts that are not a multiple of the 8-token chunk, row counts
  that are not a multiple of the 8-row workgroup, a single row, the widest E;
- a gated layer end to end: the routing decision is taken on the GPU's logits by both
  sides (the selection is bit-exact), the shared expert weighted by the GPU's gate.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

try:
    import codebook_quantized_routed_amd as moe  # noqa: E402
except ImportError:
    if torch.cuda.device_count() > 0:
        raise
    pytest.skip("HIP library not built (CPU-only machine)", allow_module_level=True)
import oracle as O  # noqa: E402
import synth  # noqa: E402
from gpu_util import REL_TOL, Run, assert_rows_close, dev, device_grids, device_layer, log  # noqa: E402

BOUND = 64 * 2.0 ** -24


def gpu_router(x, wr, wsg=None):
    T, H = x.shape
    E = wr.shape[0]
    lg = torch.full((T, E), float("nan"), dtype=torch.float32, device="cuda")
    sw = None if wsg is None else torch.full((T,), float("nan"), dtype=torch.float32, device="cuda")
    moe.router_logits(dev(x), dev(wr), T, H, E, lg, None if wsg is None else dev(wsg), sw)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), None if sw is None else sw.cpu().numpy()


CASES = [(1, 2048, 512, True), (8, 2048, 512, True), (37, 2048, 512, True), (3, 256, 16, False),
         (5, 512, 13, True), (2, 1024, 1, True), (9, 2048, 1024, False)]


@pytest.mark.parametrize("T,H,E,gate", CASES)
def test_router_matches_oracle(T, H, E, gate):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    log(f"router T={T} H={H} E={E} gate={gate}")
    x = synth.activations(T, H, tag=f"router-test/{T}/{H}/x")
    wr = synth.router_weights(E, H, tag=f"router-test/{E}/{H}/w")
    wsg = synth.shared_gate_weights(H, tag=f"router-test/{H}/g") if gate else None
    lg, sw = gpu_router(x, wr, wsg)
    l64, s64 = O.router_f64(x, wr, wsg)
    scale = O.dot_abs(x, wr)
    err = np.abs(lg.astype(np.float64) - l64)
    worst = float((err / scale).max())
    log(f"  logits: worst |err| / sum|x w| = {worst:.3e} (bound {BOUND:.3e})")
    assert np.all(err <= BOUND * scale), worst
    if gate:
        gscale = O.dot_abs(x, wsg.reshape(1, H))[:, 0]
        np.testing.assert_array_less(np.abs(sw.astype(np.float64) - s64), 0.25 * BOUND * gscale + 2.0 ** -23)
        assert np.all((sw > 0) & (sw < 1))


def test_router_logits_independent_of_batch():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T, H, E = 21, 2048, 512
    x = synth.activations(T, H, tag="router-test/batch/x")
    wr = synth.router_weights(E, H, tag="router-test/batch/w")
    wsg = synth.shared_gate_weights(H, tag="router-test/batch/g")
    full, sw_full = gpu_router(x, wr, wsg)
    perm = np.random.default_rng(2).permutation(T)
    shuffled, sw_sh = gpu_router(x[perm], wr, wsg)
    assert np.array_equal(shuffled.view(np.uint32), full[perm].view(np.uint32))
    assert np.array_equal(sw_sh.view(np.uint32), sw_full[perm].view(np.uint32))
    for t in (0, 7, 8, 20):
        one, s1 = gpu_router(x[t:t + 1], wr, wsg)
        assert np.array_equal(one[0].view(np.uint32), full[t].view(np.uint32)), t
        assert s1[0].view(np.uint32) == sw_full[t].view(np.uint32)


@pytest.fixture(scope="module")
def gated_layer(grids_compact):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    grids = device_grids(*grids_compact)
    sl = synth.make_layer([(1, 32), (2, 32)], hidden=2048, inter=512, n_experts=64, has_shared=1,
                          tag="router-test/layer")
    return sl, O.ExpertTable(sl), device_layer(sl, grids)


def test_gated_layer_end_to_end(gated_layer, ogrids):
    """x -> router (logits, gate) -> route_group -> shared_weight -> FFN -> accumulate."""
    sl, tab, dl = gated_layer
    T, H, E, k = 6, 2048, 64, 4
    x = synth.activations(T, H, tag="router-test/e2e/x")
    wr = synth.router_weights(E, H, tag="router-test/e2e/w")
    wsg = synth.shared_gate_weights(H, tag="router-test/e2e/g")
    xd = dev(x)
    lg = torch.zeros((T, E), dtype=torch.float32, device="cuda")
    sw = torch.zeros(T, dtype=torch.float32, device="cuda")
    moe.router_logits(xd, dev(wr), T, H, E, lg, dev(wsg), sw)
    r = Run(T, E, k, 1, H, dl.desc.inter)
    r.route(lg)
    moe.shared_weight(sw, T, k + 1, r.w)
    r.ffn(dl, xd)
    acc = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    r.accumulate(acc)
    got = r.host()
    lg_h, sw_h = lg.cpu().numpy(), sw.cpu().numpy()
    ref = O.moe_layer(tab, ogrids, x, k, True, logits=lg_h)
    np.testing.assert_array_equal(got["ids"], ref["ids"])
    np.testing.assert_array_equal(got["w"][:, :k], ref["w"][:, :k])
    np.testing.assert_array_equal(got["w"][:, k], sw_h)
    w_ref = ref["w"].copy()
    w_ref[:, k] = sw_h
    acc_ref = O.accumulate(ref["y"], w_ref, ref["ids"], np.zeros((T, H), np.float32))
    assert_rows_close(acc.cpu().numpy(), acc_ref, "gated layer acc", REL_TOL)
