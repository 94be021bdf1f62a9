"""GPU parity of the residual chain of routed layers, h <- h + MoE_l(RMSNorm(h)), through
the C ABI (codebook_quantized_routed_amd.stack): the first 8 layers of the 48-layer
format map (2 IQ2_XS-like, 6 IQ1_M-like), field-shape layers, each with banks of its
own (seeded per layer, so a kernel that read another layer's weights would fail).

Every layer is checked against the oracle fed the GPU's own input to that layer, so the
check covers each layer without compounding errors over the chain: routing ids
bit-exact, outputs within 2e-5 of the layer output's L2 norm per row, and within 3e-5
of the layer's MoE output (the part the layer adds to the residual) per row.

The one-launch decode of the whole chain (moe_stack_decode_q) is checked two ways:
  - against the oracle on its own inputs: the launch over the first n layers gives
    the chain's state after n layers, so layer n of the one-launch kernel is checked by
    feeding the oracle the output of the launch over n layers and comparing with the
    output of the launch over n + 1 layers;
  - bit for bit against the per-layer chain (moe_rmsnorm + moe_layer_decode_q per
    layer), ids and weights of every layer included.
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
TOL_OUT = 2e-5    # of the layer output's L2 norm
TOL_DELTA = 3e-5  # of the layer's MoE output (layer output - layer input)


def oracle_threads() -> int:
    return max(1, min(16, O.threads_available()))


def host_layers(formats, tag, **kw):
    """One seeded layer per entry of ``formats``, each with banks of its own."""
    n_experts = kw.get("n_experts", 512)
    return [synth.make_layer([(f, n_experts)], tag=f"{tag}/l{l}", **kw) for l, f in enumerate(formats)]


@pytest.fixture(scope="module")
def grids(grids_compact):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return device_grids(*grids_compact)


@pytest.fixture(scope="module")
def chain(grids):
    formats = S.stack_formats(48)[:N_LAYERS]
    host = host_layers(formats, "stack-test", has_shared=1)
    layers = [moe.DeviceLayer(h.hidden, h.inter, h.n_experts, h.has_shared, h.banks, grids) for h in host]
    tabs = [O.ExpertTable(h) for h in host]
    yield formats, S.LayerStack(layers, K), tabs


def check_layer(tab, g, hin, hout, lg, ids_gpu, what, k=K, shared=True):
    """hin, hout [n][H]; lg [n][E]; ids_gpu [n][kp]: rows are independent tokens.  The
    oracle layer is fed the GPU's input hin."""
    x = O.rmsnorm(hin)
    r = O.moe_layer(tab, g, x, k, shared, logits=lg, acc=hin, n_threads=oracle_threads())
    np.testing.assert_array_equal(ids_gpu, r["ids"], err_msg=what)
    worst_out = worst_delta = 0.0
    for t in range(hin.shape[0]):
        err = np.abs(hout[t].astype(np.float64) - r["acc"][t]).max()
        out_norm = np.linalg.norm(r["acc"][t].astype(np.float64))
        delta_norm = np.linalg.norm(r["acc"][t].astype(np.float64) - hin[t])
        assert err <= TOL_OUT * out_norm, f"{what} row {t}: {err:.3e} > {TOL_OUT} * ||out|| {out_norm:.3e}"
        assert err <= TOL_DELTA * delta_norm, f"{what} row {t}: {err:.3e} > {TOL_DELTA} * ||delta|| {delta_norm:.3e}"
        worst_out = max(worst_out, err / out_norm)
        worst_delta = max(worst_delta, err / delta_norm)
    log(f"  {what}: rows={hin.shape[0]} max|err|/||out|| = {worst_out:.3e}, /||delta|| = {worst_delta:.3e}")


def test_stack_formats_map():
    f = S.stack_formats(48)
    assert len(f) == 48 and f.count(1) == 11 and f.count(2) == 37
    assert f[0] == 1 and f[6] == 2


def test_stack_layers_have_distinct_banks(chain):
    """Same-format layers of the fixture hold different bytes (the first bytes of
    expert 0's gate codes differ between every pair of layers)."""
    formats, st, tabs = chain
    heads = [bytes(l.tensors[0][:64].cpu().numpy()) for l in st.layers]
    assert len(set(heads)) == len(heads)


def test_stack_decode_every_layer(chain, ogrids):
    formats, st, tabs = chain
    h = dev(synth.activations(1, 2048, tag="stack-test/dec/h"))
    lg = synth.logits(N_LAYERS, 512, tag="stack-test/dec/l").reshape(N_LAYERS, 1, 512)
    for l in range(N_LAYERS):
        log(f"stack decode layer {l} (format {formats[l]})")
        hin = h.cpu().numpy().copy()
        st.layer(l, h, dev(lg[l]))
        torch.cuda.synchronize()
        check_layer(tabs[l], ogrids, hin, h.cpu().numpy(), lg[l], st.buffers(1)["ids"].cpu().numpy(),
                    f"decode layer {l}")
    assert st.decode_error(1) == 0


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
        check_layer(tabs[l], ogrids, hin, h.cpu().numpy()[rows], lg[l][rows], ids, f"prefill layer {l}")


@pytest.mark.parametrize("layer", [0, 1])
def test_stack_prefill_t1024_every_row(chain, ogrids, layer):
    """The stack's 1024-token prefill through one IQ2_XS-like layer (layer 0) and one
    IQ1_M-like layer (layer 1) at full size: every row against the oracle."""
    formats, st, tabs = chain
    T = 1024
    log(f"stack prefill T={T} layer {layer} (format {formats[layer]})")
    h = dev(synth.activations(T, 2048, tag=f"stack-test/pre1024/{layer}/h"))
    lg = synth.logits(T, 512, tag=f"stack-test/pre1024/{layer}/l")
    hin = h.cpu().numpy().copy()
    st.layer(layer, h, dev(lg))
    torch.cuda.synchronize()
    ids = st.buffers(T)["ids"].cpu().numpy()
    check_layer(tabs[layer], ogrids, hin, h.cpu().numpy(), lg, ids, f"prefill T={T} layer {layer}")


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
    """The per-layer chain from h0: final h, each layer's ids and weights, and the
    state after every layer."""
    h = h0.clone()
    ids, ws, states = [], [], []
    for l in range(len(st.layers)):
        st.layer(l, h, lg[l])
        b = st.buffers(1)
        ids.append(b["ids"][0].clone())
        ws.append(b["w"][0].clone())
        states.append(h.clone())
    torch.cuda.synchronize()
    return h, torch.stack(ids), torch.stack(ws), states


def check_stack_decode(st, h0, lg, what):
    want, ids, ws, _ = chain_reference(st, h0, lg)
    out = torch.full_like(h0, float("nan"))
    log(f"stack one-launch decode: {what}, {len(st.layers)} layers")
    st.decode(h0, out, lg)
    torch.cuda.synchronize()
    b = st.stack_buffers()
    np.testing.assert_array_equal(b["ids"].cpu().numpy(), ids.cpu().numpy(), err_msg=what)
    assert np.array_equal(bits(b["w"]), bits(ws)), what
    assert np.array_equal(bits(out), bits(want)), f"{what}: max diff {(out - want).abs().max().item():.3e}"
    assert st.stack_error() == 0, f"{what}: a wait timed out"
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


def one_launch_prefixes(layers, k, h0, lg):
    """Output of the one-launch decode over layers[:n] for n = 1 .. len(layers), and the
    ids of each layer (from the launch over all layers)."""
    outs = []
    for n in range(1, len(layers) + 1):
        st = S.LayerStack(layers[:n], k)
        out = torch.full_like(h0, float("nan"))
        st.decode(h0, out, lg[:n])
        torch.cuda.synchronize()
        assert st.stack_error() == 0, f"prefix {n}: a wait timed out"
        outs.append(out.cpu().numpy().copy())
        ids = st.stack_buffers()["ids"].cpu().numpy().copy()
    return outs, ids


def check_one_launch_vs_oracle(layers, tabs, ogrids, k, shared, h0, lg, what):
    """Layer l of the one-launch kernel against the oracle on the kernel's own input to
    that layer (teacher-forced), for every layer; and the one-launch states equal the
    per-layer chain's bit for bit."""
    outs, ids = one_launch_prefixes(layers, k, h0, lg)
    st = S.LayerStack(layers, k)
    _, _, _, states = chain_reference(st, h0, lg)
    lg_host = lg.cpu().numpy()
    prev = h0.cpu().numpy()
    for l, out in enumerate(outs):
        assert np.array_equal(out.view(np.uint32), states[l].cpu().numpy().view(np.uint32)), f"{what} layer {l}"
        check_layer(tabs[l], ogrids, prev, out, lg_host[l], ids[l:l + 1], f"{what} one-launch layer {l}", k, shared)
        prev = out


def test_stack_one_launch_vs_oracle(chain, ogrids):
    formats, st, tabs = chain
    lg = dev(synth.logits(N_LAYERS, 512, tag="stack-test/onev/l").reshape(N_LAYERS, 1, 512))
    h0 = dev(synth.activations(1, 2048, tag="stack-test/onev/h"))
    check_one_launch_vs_oracle(st.layers, tabs, ogrids, K, True, h0, lg, "field stack")


@pytest.mark.parametrize("kind", ["few_values", "signed_zeros", "all_zero"])
def test_stack_one_launch_ties(chain, ogrids, kind):
    """Every layer routed by logits full of ties and signed zeros (the fallback selection
    for few_values and all_zero): ids bit-exact against the oracle, and the same bits
    as the per-layer chain."""
    formats, st, tabs = chain
    lg_host = synth.tie_logits(kind, N_LAYERS, 512, tag=f"stack-test/ties/{kind}").reshape(N_LAYERS, 1, 512)
    lg = dev(lg_host)
    h0 = dev(synth.activations(1, 2048, tag=f"stack-test/ties/{kind}/h"))
    check_stack_decode(st, h0, lg, f"ties {kind}")
    ids = st.stack_buffers()["ids"].cpu().numpy()
    for l in range(N_LAYERS):
        want, _ = O.route(lg_host[l], K, True)
        np.testing.assert_array_equal(ids[l:l + 1], want, err_msg=f"layer {l}")


def test_stack_one_launch_graph_replays(chain):
    formats, st, tabs = chain
    lg = dev(synth.logits(N_LAYERS, 512, tag="stack-test/onegraph/l").reshape(N_LAYERS, 1, 512))
    h0 = dev(synth.activations(1, 2048, tag="stack-test/onegraph/h"))
    want, _, _, _ = chain_reference(st, h0, lg)
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
    assert st.stack_error() == 0


def test_stack_workspace_rezeroed(chain):
    """A workspace zeroed whole (as the contract asks whenever its synchronisation words
    are reset) serves again: the tags restart and the result is the same bits."""
    formats, st, tabs = chain
    lg = dev(synth.logits(N_LAYERS, 512, tag="stack-test/rezero/l").reshape(N_LAYERS, 1, 512))
    h0 = dev(synth.activations(1, 2048, tag="stack-test/rezero/h"))
    a = check_stack_decode(st, h0, lg, "before re-zeroing")
    b = st.stack_buffers()
    moe.stack_prepare(b["layers"], b["ws"])
    c = check_stack_decode(st, h0, lg, "after re-zeroing")
    assert np.array_equal(bits(a), bits(c))


@pytest.fixture(scope="module")
def small_chain(grids):
    """inter 256, 64 experts, no shared expert, k = 4; the middle layer holds both
    formats (experts 0-31 IQ2_XS-like, 32-63 IQ1_M-like)."""
    kw = dict(inter=256, n_experts=64, has_shared=0)
    specs = [[(1, 64)], [(1, 32), (2, 32)], [(2, 64)]]
    host = [synth.make_layer(spec, tag=f"stack-test/small{i}", **kw) for i, spec in enumerate(specs)]
    layers = [moe.DeviceLayer(h.hidden, h.inter, h.n_experts, h.has_shared, h.banks, grids) for h in host]
    yield layers, [O.ExpertTable(h) for h in host]


def test_stack_one_launch_small_shape(small_chain, ogrids):
    layers, tabs = small_chain
    st = S.LayerStack(layers, 4)
    lg = dev(synth.logits(3, 64, tag="stack-test/small/l").reshape(3, 1, 64))
    h0 = dev(synth.activations(1, 2048, tag="stack-test/small/h"))
    check_stack_decode(st, h0, lg, "inter 256, mixed formats")
    check_one_launch_vs_oracle(layers, tabs, ogrids, 4, False, h0, lg, "inter 256, mixed formats")
    one = S.LayerStack(layers[1:2], 4)                           # a chain of one layer
    check_stack_decode(one, h0, lg[1:2], "one layer")


@pytest.fixture(scope="module")
def chain48(grids):
    """All 48 layers of the format map (11 IQ2_XS-like, 37 IQ1_M-like) at a small expert
    count, every layer with banks of its own: 64 experts + shared, inter 512, top-4."""
    formats = S.stack_formats(48)
    host = host_layers(formats, "stack-test/48", n_experts=64, has_shared=1)
    layers = [moe.DeviceLayer(h.hidden, h.inter, h.n_experts, h.has_shared, h.banks, grids) for h in host]
    yield layers, [O.ExpertTable(h) for h in host]


def test_stack48_one_launch_vs_oracle(chain48, ogrids):
    """The full 48-layer chain in one launch: bit for bit the per-layer chain (ids,
    weights, output), and every layer against the oracle on the launch's own input."""
    layers, tabs = chain48
    st = S.LayerStack(layers, 4)
    lg = dev(synth.logits(48, 64, tag="stack-test/48/l").reshape(48, 1, 64))
    h0 = dev(synth.activations(1, 2048, tag="stack-test/48/h"))
    check_stack_decode(st, h0, lg, "48 layers")
    check_one_launch_vs_oracle(layers, tabs, ogrids, 4, True, h0, lg, "48 layers")
