"""GPU parity of the residual chain of routed layers, h <- h + MoE_l(RMSNorm(h)), through
the C ABI (codebook_quantized_routed_amd.stack): the first 8 layers of the 48-layer
format map (2 IQ2_XS-like, 6 IQ1_M-like), field-shape layers.

Every layer is checked against the oracle fed the GPU's own input to that layer, so the
check covers each layer without compounding errors over the chain: routing ids
bit-exact, outputs within 3e-5 of the layer's MoE output norm per row (the 2e-5 bound
on the layer output, plus one rounding of the residual's own magnitude).

The one-launch decode of the whole chain (moe_stack_decode_q) computes each layer with
the arithmetic of moe_rmsnorm + moe_layer_decode_q, so it is checked bit for bit
against that per-layer chain (itself checked against the oracle above), ids and
weights of every layer included.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

try:
    import codebook_quantized_routed_amd as moe  # noqa: E402
    from codebook_quantized_routed_amd import stack as S  # noqa: E402
except ImportError:
    if torch.cuda.device_count() > 0:
        raise
    pytest.skip("HIP library not built (CPU-only machine)", allow_module_level=True)
import oracle as O  # noqa: E402
import synth  # noqa: E402
from gpu_util import dev, device_grids, log  # noqa: E402

N_LAYERS = 8
K = 10
TOL = 3e-5


@pytest.fixture(scope="module")
def chain(grids_compact):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    O.set_threads(8)
    grids = device_grids(*grids_compact)
    host = {qt: synth.make_layer([(qt, 512)], has_shared=1, tag=f"stack-test/q{qt}") for qt in (1, 2)}
    formats = S.stack_formats(48)[:N_LAYERS]
    layers = S.device_stack(formats, {qt: host[qt].banks for qt in host}, grids)
    tabs = {qt: O.ExpertTable(host[qt]) for qt in host}
    yield formats, S.LayerStack(layers, K), tabs
    O.set_threads(1)


def check_layer(tab, g, hin, hout, lg, ids_gpu, what):
    """hin, hout [n][H]; lg [n][E]; ids_gpu [n][kp]: rows are independent tokens."""
    x = O.rmsnorm(hin)
    r = O.moe_layer(tab, g, x, K, True, logits=lg, acc=hin)
    np.testing.assert_array_equal(ids_gpu, r["ids"], err_msg=what)
    for t in range(hin.shape[0]):
        scale = np.linalg.norm(r["acc"][t].astype(np.float64) - hin[t])
        err = np.abs(hout[t].astype(np.float64) - r["acc"][t]).max()
        assert err <= TOL * scale, f"{what} row {t}: {err:.3e} > {TOL} * {scale:.3e}"


def test_stack_formats_map():
    f = S.stack_formats(48)
    assert len(f) == 48 and f.count(1) == 11 and f.count(2) == 37
    assert f[0] == 1 and f[6] == 2


def test_stack_decode_every_layer(chain, ogrids):
    formats, st, tabs = chain
    h = dev(synth.activations(1, 2048, tag="stack-test/dec/h"))
    lg = synth.logits(N_LAYERS, 512, tag="stack-test/dec/l").reshape(N_LAYERS, 1, 512)
    for l in range(N_LAYERS):
        log(f"stack decode layer {l} (format {formats[l]})")
        hin = h.cpu().numpy().copy()
        st.layer(l, h, dev(lg[l]))
        torch.cuda.synchronize()
        check_layer(tabs[formats[l]], ogrids, hin, h.cpu().numpy(), lg[l], st.buffers(1)["ids"].cpu().numpy(),
                    f"decode layer {l}")


def test_stack_prefill_sampled(chain, ogrids):
    """40 tokens: experts with several tokens go to the matrix cores; sampled rows checked
    at every layer (tokens do not mix in the chain)."""
    formats, st, tabs = chain
    T = 40
    rows = [0, 13, 39]
    h = dev(synth.activations(T, 2048, tag="stack-test/pre/h"))
    lg = synth.logits(N_LAYERS * T, 512, tag="stack-test/pre/l").reshape(N_LAYERS, T, 512)
    for l in range(N_LAYERS):
        log(f"stack prefill layer {l} (format {formats[l]})")
        hin = h.cpu().numpy()[rows].copy()
        st.layer(l, h, dev(lg[l]))
        torch.cuda.synchronize()
        ids = st.buffers(T)["ids"].cpu().numpy()[rows]
        check_layer(tabs[formats[l]], ogrids, hin, h.cpu().numpy()[rows], lg[l][rows], ids, f"prefill layer {l}")


def test_stack_decode_graph_replays(chain):
    """A captured decode step (all layers), replayed several times with eager work and
    synchronisations in between, gives the eager result bit for bit every time."""
    formats, st, tabs = chain
    h0 = dev(synth.activations(1, 2048, tag="stack-test/graph/h"))
    lg = dev(synth.logits(N_LAYERS, 512, tag="stack-test/graph/l").reshape(N_LAYERS, 1, 512))
    h = h0.clone()
    st.step(h, lg)
    torch.cuda.synchronize()
    want = h.cpu().numpy().copy()
    hg = h0.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            st.step(hg, lg)
    torch.cuda.synchronize()
    for rep in range(3):
        hg.copy_(h0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(hg.cpu().numpy().view(np.uint32), want.view(np.uint32)), f"replay {rep}"
        other = h0.clone()  # eager work between replays
        st.layer(0, other, lg[0])
        torch.cuda.synchronize()


def bits(t):
    return t.cpu().numpy().view(np.uint32)


def chain_reference(st, h0, lg):
    """The per-layer chain from h0: final h and each layer's ids and weights."""
    h = h0.clone()
    ids, ws = [], []
    for l in range(len(st.layers)):
        st.layer(l, h, lg[l])
        b = st.buffers(1)
        ids.append(b["ids"][0].clone())
        ws.append(b["w"][0].clone())
    torch.cuda.synchronize()
    return h, torch.stack(ids), torch.stack(ws)


def check_stack_decode(st, h0, lg, what):
    want, ids, ws = chain_reference(st, h0, lg)
    out = torch.full_like(h0, float("nan"))
    log(f"stack one-launch decode: {what}, {len(st.layers)} layers")
    st.decode(h0, out, lg)
    torch.cuda.synchronize()
    b = st.stack_buffers()
    np.testing.assert_array_equal(b["ids"].cpu().numpy(), ids.cpu().numpy(), err_msg=what)
    assert np.array_equal(bits(b["w"]), bits(ws)), what
    assert np.array_equal(bits(out), bits(want)), f"{what}: max diff {(out - want).abs().max().item():.3e}"
    assert int(b["ws"][32].item()) == 0, f"{what}: a wait timed out"   # error word at byte 128
    return out


def test_stack_one_launch_matches_chain(chain):
    formats, st, tabs = chain
    lg = dev(synth.logits(N_LAYERS, 512, tag="stack-test/one/l").reshape(N_LAYERS, 1, 512))
    h0 = dev(synth.activations(1, 2048, tag="stack-test/one/h"))
    first = check_stack_decode(st, h0, lg, "first call")
    again = check_stack_decode(st, h0, lg, "second call")        # the next call's tags
    assert np.array_equal(bits(first), bits(again))
    h1 = dev(synth.activations(1, 2048, tag="stack-test/one/h1"))
    check_stack_decode(st, h1, lg, "another input")


def test_stack_one_launch_graph_replays(chain):
    formats, st, tabs = chain
    lg = dev(synth.logits(N_LAYERS, 512, tag="stack-test/onegraph/l").reshape(N_LAYERS, 1, 512))
    h0 = dev(synth.activations(1, 2048, tag="stack-test/onegraph/h"))
    want, _, _ = chain_reference(st, h0, lg)
    st.stack_buffers()                                           # set-up outside the capture
    out = torch.zeros_like(h0)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            st.decode(h0, out, lg)
    torch.cuda.synchronize()
    for rep in range(3):
        out.zero_()
        torch.cuda.synchronize()
        log(f"stack one-launch graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out), bits(want)), f"replay {rep}"
        other = torch.zeros_like(h0)                             # eager work between replays
        st.decode(h0, other, lg)
        torch.cuda.synchronize()
        assert np.array_equal(bits(other), bits(want)), f"eager after replay {rep}"


@pytest.fixture(scope="module")
def small_chain(grids_compact):
    """inter 256, 64 experts, no shared expert, k = 4; the middle layer holds both
    formats (experts 0-31 IQ2_XS-like, 32-63 IQ1_M-like)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    grids = device_grids(*grids_compact)
    kw = dict(inter=256, n_experts=64, has_shared=0)
    specs = [[(1, 64)], [(1, 32), (2, 32)], [(2, 64)]]
    layers = []
    for i, spec in enumerate(specs):
        h = synth.make_layer(spec, tag=f"stack-test/small{i}", **kw)
        layers.append(moe.DeviceLayer(h.hidden, h.inter, h.n_experts, h.has_shared, h.banks, grids))
    yield layers


def test_stack_one_launch_small_shape(small_chain):
    st = S.LayerStack(small_chain, 4)
    lg = dev(synth.logits(3, 64, tag="stack-test/small/l").reshape(3, 1, 64))
    h0 = dev(synth.activations(1, 2048, tag="stack-test/small/h"))
    check_stack_decode(st, h0, lg, "inter 256, mixed formats")
    one = S.LayerStack(small_chain[1:2], 4)                      # a chain of one layer
    check_stack_decode(one, h0, lg[1:2], "one layer")
