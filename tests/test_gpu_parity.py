"""GPU parity: the HIP path through the C ABI against the oracle on the same seeded bytes.

Bit-exact: expanded grids, dequantized weights, routing ids and grouping arrays, and
the accumulation given the same y and w.  Tolerance (max |error| <= 2e-5 * ||ref||_2 per
output row): expert outputs y and layer outputs acc.  Router weights: a few ulp (the
device exp differs from libm's by rounding only).
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
import oracle as O  # noqa: E402
import synth  # noqa: E402
from gpu_util import (Run, assert_rows_close, dev, device_grids, device_layer, log, run_layer,  # noqa: E402
                      y_in_slot_order)

IQ2, IQ1, IQ1S = synth.QTYPE_IQ2XS, synth.QTYPE_IQ1M, synth.QTYPE_IQ1S


@pytest.fixture(scope="module")
def grids(grids_compact):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return device_grids(*grids_compact)


@pytest.fixture(scope="module", autouse=True)
def oracle_threads():
    O.set_threads(8)
    yield
    O.set_threads(1)


def test_grids_expand_bit_exact(grids, ogrids, grids_compact):
    g = grids.cpu().numpy()
    np.testing.assert_array_equal(g[:4096].reshape(512, 8), ogrids.iq2_array())
    np.testing.assert_array_equal(g[4096:20480].view(np.int8).reshape(2048, 8), ogrids.iq1_array())

    # the compact rows the mat-vec kernels build their LDS tables from
    c2, c1 = grids_compact
    np.testing.assert_array_equal(g[20480:21504].view(np.uint16), c2)
    np.testing.assert_array_equal(g[21504:25600].view(np.uint16), c1)
    assert g.size == moe.grids_bytes() == 25600 + 8192 + 32768 + 65536
    # the matrix-core decode tables, from the oracle's grid values and the pages' sign
    # and scale mapping: fp16 IQ2 rows; per (7 explicit signs, 4-bit scale) the eight
    # values +-(2s + 1), the eighth sign being the parity of the seven; IQ1 rows with
    # +1/8, then with -1/8 added
    dec = g[25600:]
    np.testing.assert_array_equal(dec[:8192].view(np.float16).reshape(512, 8),
                                  ogrids.iq2_array().astype(np.float16))
    e = np.arange(128 * 16)
    s7, sc = e >> 4, e & 15
    parity = np.array([bin(v).count("1") & 1 for v in range(128)])[s7]
    bits = (s7 | (parity << 7))[:, None] >> np.arange(8)[None, :] & 1
    ss = np.where(bits == 1, -(2 * sc + 1)[:, None], (2 * sc + 1)[:, None]).astype(np.float16)
    np.testing.assert_array_equal(dec[8192:40960].view(np.float16).reshape(2048, 8), ss)
    G1 = ogrids.iq1_array().astype(np.float64)
    d1 = dec[40960:].view(np.float16).reshape(2, 2048, 8)
    np.testing.assert_array_equal(d1[0], (G1 + 0.125).astype(np.float16))
    np.testing.assert_array_equal(d1[1], (G1 - 0.125).astype(np.float16))


def _dequant_gpu(qt, rows, cols, streams, grids):
    out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    moe.dequant_f32(qt, rows, cols, dev(streams[0]), dev(streams[1]), dev(streams[2]), grids, out)
    return out.cpu().numpy()


@pytest.mark.parametrize("qt,rows,cols", [(IQ2, 512, 2048), (IQ2, 2048, 512), (IQ1, 512, 2048), (IQ1, 2048, 512),
                                          (IQ2, 8, 256), (IQ1, 24, 768)])
def test_dequant_bit_exact_seeded(grids, ogrids, qt, rows, cols):
    log(f"dequant qt={qt} {rows}x{cols}")
    streams = [a[0] for a in synth.qbank(qt, 1, rows, cols, 9, f"dq/{qt}/{rows}/{cols}")]
    got = _dequant_gpu(qt, rows, cols, streams, grids)
    ref = O.dequant(O.qmat(qt, rows, cols, streams), ogrids)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_bit_exact_every_code(grids, ogrids):
    """Every IQ2 code under every scale and every IQ1 code under every scale."""
    from test_oracle_dequant import encode_iq1, encode_iq2
    rows, cols = 4096, 2048
    ng, nb = cols // 8, cols // 256
    code = np.arange(rows * ng, dtype=np.int64).reshape(rows, ng) % 65536
    r_, b_, i_ = np.arange(rows)[:, None, None], np.arange(nb)[None, :, None], np.arange(8)[None, None, :]
    d = synth.uniform(1, "dq/d", rows * nb).reshape(rows, nb)
    d16 = (1e-3 * (0.5 + d)).astype(np.float16).view(np.uint16)
    s2 = encode_iq2(code & 511, code >> 9, (r_ // 256 + b_ + i_ + r_) % 16, d16)
    got = _dequant_gpu(IQ2, rows, cols, s2, grids)
    ref = O.dequant(O.qmat(IQ2, rows, cols, s2), ogrids)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    rows = 128
    code = np.arange(rows * ng, dtype=np.int64).reshape(rows, ng) % 4096
    r_, i_ = np.arange(rows)[:, None, None], np.arange(16)[None, None, :]
    s1 = encode_iq1(code & 2047, code >> 11, (r_ // 16 + b_ + i_ + r_) % 8, d16[:rows])
    got = _dequant_gpu(IQ1, rows, cols, s1, grids)
    ref = O.dequant(O.qmat(IQ1, rows, cols, s1), ogrids)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


ROUTE_CASES = [  # T, E, k, shared, zipf
    (1, 512, 10, True, 0.0), (8, 512, 10, True, 0.0), (256, 512, 10, False, 0.0), (256, 512, 10, False, 1.1),
    (1024, 512, 10, True, 0.0), (1, 16, 4, False, 0.0), (33, 16, 16, True, 0.0), (5, 1023, 16, True, 0.0),
    (3, 64, 1, False, 0.0), (2000, 100, 7, True, 0.0),
    # 65 .. 272 slots in one workgroup (the counting sort): duplicates, every expert in the
    # first set up to 16 tokens, wide experts at T = 20
    (20, 16, 5, True, 0.0), (12, 64, 9, True, 0.0), (11, 512, 10, True, 1.1), (13, 40, 4, True, 0.0),
    (16, 512, 16, True, 0.0), (16, 64, 16, True, 0.0), (9, 16, 8, False, 0.0), (16, 512, 15, True, 1.1),
]


@pytest.mark.parametrize("T,E,k,shared,zipf", ROUTE_CASES)
def test_route_group_bit_exact(T, E, k, shared, zipf):
    log(f"route_group T={T} E={E} k={k} shared={shared} zipf={zipf}")
    lg = synth.logits(T, E, tag=f"rg/{T}/{E}", zipf_alpha=zipf)
    r = Run(T, E, k, shared, 256, 256)
    r.route(dev(lg))
    g = r.host()
    ids, w = O.route(lg, k, shared)
    np.testing.assert_array_equal(g["ids"], ids)
    np.testing.assert_allclose(g["w"], w, rtol=8 * 2.0 ** -24, atol=0)
    counts, offsets, ss, sp = O.group(ids, E + int(shared))
    np.testing.assert_array_equal(g["counts"], counts)
    np.testing.assert_array_equal(g["offsets"], offsets)
    np.testing.assert_array_equal(g["sorted_slot"], ss)
    np.testing.assert_array_equal(g["slot_pos"], sp)
    check_work(g["work"], counts, offsets, ss, T)


def check_work(work, counts, offsets, ss, T):
    """Work list: record 0 = (n1, slots, n2, tiles); the experts with 1..m(T) slots in
    records 1..n1, ascending id, as (e, offsets[e], offsets[e+1], first slot); after the
    n_ids + 1 records, the other experts' tiles of MFMA_TILE_TOKENS positions, ascending
    (id, start)."""
    n_ids = len(counts)
    m = moe.matvec_max_tokens(T)
    act = np.flatnonzero(counts)
    narrow = act[counts[act] <= m]
    wide = act[counts[act] > m]
    tiles = [(e, p, min(p + moe.MFMA_TILE_TOKENS, offsets[e + 1]), 0)
             for e in wide for p in range(offsets[e], offsets[e + 1], moe.MFMA_TILE_TOKENS)]
    rec = work.reshape(-1, 4)
    assert len(rec) >= n_ids + 1 + len(tiles)
    np.testing.assert_array_equal(rec[0], [len(narrow), offsets[-1], len(wide), len(tiles)])
    want = np.stack([narrow, offsets[narrow], offsets[narrow + 1], ss[offsets[narrow]]], axis=1).reshape(-1, 4)
    np.testing.assert_array_equal(rec[1:1 + len(narrow)], want)
    np.testing.assert_array_equal(rec[n_ids + 1:n_ids + 1 + len(tiles)], np.array(tiles, dtype=np.int64).reshape(-1, 4))


def test_route_ties_and_explicit_mode():
    l = np.array([[1.0, 3.0, 3.0, 0.5, 3.0, 2.0, 2.0, -1.0]], dtype=np.float32)
    r = Run(1, 8, 5, True, 256, 256)
    r.route(dev(l))
    g = r.host()
    np.testing.assert_array_equal(g["ids"][0], [1, 2, 4, 5, 6, 8])
    # explicit ids / weights: only the shared slot and the grouping are written
    ids = np.array([[7, 0, 3], [3, 1, 0]], np.int32)
    w = np.array([[0.5, 0.3, 0.2], [0.6, 0.3, 0.1]], np.float32)
    r = Run(2, 8, 3, True, 256, 256)
    r.route(None, ids, w)
    g = r.host()
    np.testing.assert_array_equal(g["ids"][:, :3], ids)
    np.testing.assert_array_equal(g["ids"][:, 3], [8, 8])
    np.testing.assert_array_equal(g["w"][:, :3], w)
    full = np.concatenate([ids, [[8], [8]]], axis=1)
    counts, offsets, ss, sp = O.group(full, 9)
    np.testing.assert_array_equal(g["sorted_slot"], ss)
    np.testing.assert_array_equal(g["offsets"], offsets)
    check_work(g["work"], counts, offsets, ss, 2)



TIE_KINDS = ["few_values", "signed_zeros", "all_zero"]


@pytest.mark.parametrize("kind", TIE_KINDS)
@pytest.mark.parametrize("T,E,k,shared", [(1, 512, 10, True), (8, 512, 10, True), (256, 512, 10, False),
                                          (1, 1023, 16, True), (8, 1023, 16, False), (256, 1023, 16, False)])
def test_route_group_ties_bit_exact(kind, T, E, k, shared):
    """Logits full of ties and of zeros of both signs: -0.0 ties with +0.0 and the lower
    id wins, as in the oracle.  few_values and all_zero put more than 64 keys at the
    top-k threshold (the fallback selection by k arg-max rounds); signed_zeros decides
    the selection among +0.0 and -0.0 on the candidate path.  T = 1 and 8 at 512
    experts run the one-workgroup route + group kernel, the others the top-k kernel and
    the grouping kernel."""
    log(f"route ties {kind} T={T} E={E} k={k} shared={shared}")
    lg = synth.tie_logits(kind, T, E, tag=f"rgt/{kind}/{T}/{E}")
    r = Run(T, E, k, shared, 256, 256)
    r.route(dev(lg))
    g = r.host()
    ids, w = O.route(lg, k, shared)
    np.testing.assert_array_equal(g["ids"], ids)
    np.testing.assert_allclose(g["w"], w, rtol=8 * 2.0 ** -24, atol=0)
    counts, offsets, ss, sp = O.group(ids, E + int(shared))
    np.testing.assert_array_equal(g["counts"], counts)
    np.testing.assert_array_equal(g["offsets"], offsets)
    np.testing.assert_array_equal(g["sorted_slot"], ss)
    np.testing.assert_array_equal(g["slot_pos"], sp)
    check_work(g["work"], counts, offsets, ss, T)


# ------------------------------------------------------------------------- whole layer

LAYER_CASES = {
    # name: (banks, H, I, E, shared, T, k, zipf)
    "tiny16_top4_iq2": ([(IQ2, 16)], 2048, 512, 16, 0, 1, 4, 0.0),
    "decode_iq2_top10_shared": ([(IQ2, 512)], 2048, 512, 512, 1, 1, 10, 0.0),
    "decode8_iq1_top10_shared": ([(IQ1, 512)], 2048, 512, 512, 1, 8, 10, 0.0),
    "small_mixed_ragged": ([(IQ2, 12), (IQ1, 20)], 512, 256, 32, 1, 19, 6, 0.0),
    "small_mixed_many_tokens": ([(IQ1, 8), (IQ2, 8)], 256, 512, 16, 0, 96, 5, 0.0),
    "mixed_h2048_t24_zipf": ([(IQ2, 24), (IQ1, 40)], 2048, 512, 64, 1, 24, 8, 1.0),
    # many tokens per expert: the matrix-core path, one to three 16-token tiles per expert
    "dense_iq2_t64": ([(IQ2, 16)], 2048, 512, 16, 0, 64, 4, 0.0),
    "dense_iq1_t40_shared": ([(IQ1, 8)], 2048, 512, 8, 1, 40, 3, 0.0),
    "mixed_t128_zipf": ([(IQ2, 32), (IQ1, 32)], 2048, 512, 64, 0, 128, 10, 1.1),
    "mixed_h512_i1024_t48": ([(IQ1, 6), (IQ2, 6)], 512, 1024, 12, 1, 48, 2, 0.0),
    "decode_mixed_i256_shared": ([(IQ2, 20), (IQ1, 12)], 2048, 256, 32, 1, 1, 6, 0.0),
    # IQ1_S-like banks, repacked into the IQ1_M-like layout when the layer is loaded
    "decode_iq1s_top10_shared": ([(IQ1S, 512)], 2048, 512, 512, 1, 1, 10, 0.0),
    "iq1s_mixed_t6": ([(IQ1S, 32), (IQ2, 32)], 2048, 512, 64, 1, 6, 4, 0.0),
    "dense_iq1s_t40_shared": ([(IQ1S, 8)], 2048, 512, 8, 1, 40, 3, 0.0),
    # the widest routing (16 experts + the shared one): a wave of the fused down +
    # accumulate holds more slots than it loads up front
    "top16_shared_t8": ([(IQ2, 32), (IQ1, 32)], 2048, 512, 64, 1, 8, 16, 0.0),
    "top13_t5": ([(IQ1, 24), (IQ2, 24)], 2048, 512, 48, 0, 5, 13, 0.0),
    # one format at inter 256: the one-launch kernel's single-format instances, 4 lanes per row
    "decode_iq1_i256": ([(IQ1, 16)], 2048, 256, 16, 1, 1, 4, 0.0),
    "decode_iq2_i256": ([(IQ2, 16)], 2048, 256, 16, 0, 1, 5, 0.0),
    # 2 to 8 tokens: gate / up on the matrix-core decode kernel (one part of one or two
    # super-blocks per wave at hidden 256 / 512, two parts at 1024)
    "decode2_iq2_top10_shared": ([(IQ2, 512)], 2048, 512, 512, 1, 2, 10, 0.0),
    "dec_h256_i256_mixed_t7": ([(IQ2, 12), (IQ1, 12)], 256, 256, 24, 1, 7, 3, 0.0),
    "dec_h512_iq2_t3": ([(IQ2, 16)], 512, 512, 16, 0, 3, 4, 0.0),
    "dec_h1024_iq1_t4_zipf": ([(IQ1, 16)], 1024, 512, 16, 0, 4, 4, 1.0),
    # every expert takes all 8 tokens: the 16-row A operand full
    "dec_every_expert_all_tokens": ([(IQ2, 4)], 2048, 512, 4, 1, 8, 4, 0.0),
    # one token, 16 experts + the shared one: 17 x 256 gate / up items, more than the
    # one-launch grid has waves (second items), and two sorted positions per down wave;
    # one bank (addresses from fixed argument offsets) and two banks
    "decode_top16_shared_iq2": ([(IQ2, 64)], 2048, 512, 64, 1, 1, 16, 0.0),
    "decode_top16_shared_mixed": ([(IQ2, 32), (IQ1, 32)], 2048, 512, 64, 1, 1, 16, 0.0),
}


def _repack_gpu(rows, cols, streams):
    ql, qh, d = (dev(a.reshape(-1)) for a in streams)
    out = [torch.empty(rows * cols // 8, dtype=torch.uint8, device="cuda"),
           torch.empty(rows * cols // 16, dtype=torch.uint8, device="cuda"),
           torch.empty(rows * cols // 256 * 8, dtype=torch.uint8, device="cuda")]
    moe.repack_iq1s(ql, qh, d, rows, cols, *out)
    return out


@pytest.mark.parametrize("n,rows,cols", [(1, 512, 2048), (1, 2048, 512), (3, 512, 2048), (1, 8, 256), (2, 24, 768)])
def test_repack_iq1s_bit_exact(grids, ogrids, n, rows, cols):
    """IQ1_S-like streams repacked on the GPU and dequantized as IQ1_M-like == the oracle's
    dequantization of the IQ1_S-like streams themselves, bit for bit (n matrices back to
    back, as in a bank)."""
    log(f"repack iq1s n={n} {rows}x{cols}")
    s = synth.qbank(IQ1S, n, rows, cols, 9, f"repack/{n}/{rows}/{cols}")
    out = _repack_gpu(n * rows, cols, s)
    g = torch.empty((n * rows, cols), dtype=torch.float32, device="cuda")
    moe.dequant_f32(IQ1, n * rows, cols, out[0], out[1], out[2], grids, g)
    got = g.cpu().numpy()
    for e in range(n):
        ref = O.dequant(O.qmat(IQ1S, rows, cols, [a[e] for a in s]), ogrids)
        assert np.array_equal(got[e * rows:(e + 1) * rows].view(np.uint32), ref.view(np.uint32)), e


def test_repack_iq1s_every_code(grids, ogrids):
    """Every 11-bit index under every (scale, delta sign) of its sub-block, repacked."""
    from test_oracle_dequant import encode_iq1s
    rows, cols = 128, 2048
    ng, nb = cols // 8, cols // 256
    idx11 = np.arange(rows * ng, dtype=np.int64).reshape(rows, ng) % 2048
    combo = (np.arange(rows)[:, None] // 8 + np.arange(ng // 4)[None, :]) % 16
    d16 = (1e-3 * (0.5 + synth.uniform(3, "repack/d", rows * nb))).astype(np.float16).view(np.uint16).reshape(rows, nb)
    s = encode_iq1s(idx11, combo >> 3, combo & 7, d16)
    out = _repack_gpu(rows, cols, s)
    g = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
    moe.dequant_f32(IQ1, rows, cols, out[0], out[1], out[2], grids, g)
    ref = O.dequant(O.qmat(IQ1S, rows, cols, s), ogrids)
    assert np.array_equal(g.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.fixture(scope="module")
def layers(grids):
    cache = {}

    def get(name):
        if name not in cache:
            banks, H, I, E, shared, *_ = LAYER_CASES[name]
            sl = synth.make_layer(banks, hidden=H, inter=I, n_experts=E, has_shared=shared, tag=f"L/{name}")
            cache[name] = (sl, O.ExpertTable(sl), device_layer(sl, grids))
        return cache[name]
    return get


@pytest.mark.parametrize("name", list(LAYER_CASES))
def test_layer_matches_oracle(layers, ogrids, name):
    banks, H, I, E, shared, T, k, zipf = LAYER_CASES[name]
    log(f"layer {name}: T={T} E={E} k={k} H={H} I={I}")
    sl, tab, dl = layers(name)
    x = synth.activations(T, H, tag=f"L/{name}/x")
    lg = synth.logits(T, E, tag=f"L/{name}/l", zipf_alpha=zipf)
    acc0 = synth.activations(T, H, tag=f"L/{name}/acc") if T > 1 else None
    g = run_layer(dl, x, k, shared, logits=lg, acc=acc0)
    ref = O.moe_layer(tab, ogrids, x, k, shared, logits=lg, acc=acc0)
    np.testing.assert_array_equal(g["ids"], ref["ids"])
    assert_rows_close(y_in_slot_order(g), ref["y"], f"{name} y")
    assert_rows_close(g["acc"], ref["acc"], f"{name} acc")
    # accumulation is exactly defined given y and w: feed the oracle the GPU's y and w
    acc_in = np.zeros((T, H), np.float32) if acc0 is None else acc0
    np.testing.assert_array_equal(g["acc"], O.accumulate(y_in_slot_order(g), g["w"], g["ids"], acc_in))


@pytest.mark.parametrize("name", list(LAYER_CASES))
def test_decode_path_matches_split_path(layers, ogrids, name):
    """gate/up + fused down-accumulate against the oracle; bit for bit equal to ffn_q +
    accumulate when every expert takes the mat-vec path (the fused down is a mat-vec);
    and ffn_q == gate/up followed by down."""
    banks, H, I, E, shared, T, k, zipf = LAYER_CASES[name]
    log(f"decode path {name}: T={T}")
    sl, tab, dl = layers(name)
    x = synth.activations(T, H, tag=f"D/{name}/x")
    lg = synth.logits(T, E, tag=f"D/{name}/l", zipf_alpha=zipf)
    acc0 = synth.activations(T, H, tag=f"D/{name}/acc")
    a = run_layer(dl, x, k, shared, logits=lg, acc=acc0)
    b = run_layer(dl, x, k, shared, logits=lg, acc=acc0, decode=True)
    if a["counts"].max() <= moe.matvec_max_tokens(T):  # every expert on the mat-vec kernels
        assert np.array_equal(a["acc"].view(np.uint32), b["acc"].view(np.uint32))
    else:
        ref = O.moe_layer(tab, ogrids, x, k, shared, logits=lg, acc=acc0)
        # the layer output's bound (2e-5 of ||acc||), and 3e-5 of the part the layer adds
        # (acc - acc0: the bound plus one rounding of the accumulator's own magnitude)
        assert_rows_close(b["acc"], ref["acc"], f"{name} fused acc")
        assert_rows_close(b["acc"] - acc0, ref["acc"] - acc0, f"{name} fused acc - acc0", rel=3e-5)
    r = Run(T, E, k, shared, H, I)
    r.route(dev(lg))
    h = torch.zeros((T * r.kp, I), dtype=torch.float32, device="cuda")
    r.gateup(dl, dev(x), h)
    y2 = torch.zeros_like(r.y)
    moe.expert_down_q(dl.desc, h, T, r.kp, r.work, y2)
    r.ffn(dl, dev(x))
    torch.cuda.synchronize()
    assert torch.equal(r.y, y2)


@pytest.mark.parametrize("zipf", [0.0, 1.1])
def test_prefill_field_shape_every_token(grids, ogrids, zipf):
    """The batched field-shape layer at full size: 256 tokens, experts 0-255 IQ2_XS-like
    and 256-511 IQ1_M-like, top-10 (uniform and Zipf(1.1) logits).  Routing of every
    token bit for bit; every token's output row against the oracle, element by element;
    and every expert output y the same way."""
    T, E, k, H, I = 256, 512, 10, 2048, 512
    log(f"prefill field shape T={T} zipf={zipf}")
    sl = synth.make_layer([(IQ2, 256), (IQ1, 256)], hidden=H, inter=I, n_experts=E, has_shared=0, tag="L/prefill")
    dl = device_layer(sl, grids)
    tab = O.ExpertTable(sl)
    x = synth.activations(T, H, tag=f"P/{zipf}/x")
    lg = synth.logits(T, E, tag=f"P/{zipf}/l", zipf_alpha=zipf)
    g = run_layer(dl, x, k, False, logits=lg)
    counts = g["counts"]
    m = moe.matvec_max_tokens(T)
    log(f"  experts on matrix cores: {(counts > m).sum()}, mat-vec: {((counts > 0) & (counts <= m)).sum()}, "
        f"max tokens {counts.max()}")
    ref = O.moe_layer(tab, ogrids, x, k, False, logits=lg, n_threads=max(1, min(16, O.threads_available())))
    np.testing.assert_array_equal(g["ids"], ref["ids"])
    assert_rows_close(y_in_slot_order(g), ref["y"], f"prefill zipf={zipf} y")
    assert_rows_close(g["acc"], ref["acc"], f"prefill zipf={zipf} acc")


def call_counts(ws):
    """(sum of the per-group call counters, error word) of a decode workspace: the
    uint32 error word sits at byte 128, the 32 counters at byte 256 + 128 g (uint64)."""
    sync = ws[: moe.DECODE_SYNC_BYTES // 4].cpu().numpy()
    counters = sync.view(np.uint64)[32::16][:32]
    return int(counters.sum()), int(sync.view(np.uint32)[32])


FUSED_CASES = ["decode_iq2_top10_shared", "tiny16_top4_iq2", "mixed_h2048_t24_zipf", "decode_mixed_i256_shared",
               "decode_iq1s_top10_shared", "decode_iq1_i256", "decode_iq2_i256", "decode_top16_shared_iq2",
               "decode_top16_shared_mixed"]


@pytest.mark.parametrize("name", FUSED_CASES)
def test_fused_decode_matches_three_calls(layers, name):
    """moe_layer_decode_q (one launch) writes the same bits as moe_route_group +
    moe_expert_gateup_q + moe_expert_down_accumulate_q, on consecutive calls that share
    one workspace, with router logits and with an explicit selection."""
    banks, H, I, E, shared, T, k, zipf = LAYER_CASES[name]
    sl, tab, dl = layers(name)
    kp = k + shared
    ws = torch.zeros(moe.decode_workspace_bytes(kp, I) // 4, dtype=torch.int32, device="cuda")
    for call in range(3):
        log(f"fused decode {name} call {call}")
        x = synth.activations(1, H, tag=f"F/{name}/{call}/x")
        acc0 = synth.activations(1, H, tag=f"F/{name}/{call}/acc")
        if call < 2:
            lg = synth.logits(1, E, tag=f"F/{name}/{call}/l", zipf_alpha=zipf)
            ref = run_layer(dl, x, k, shared, logits=lg, acc=acc0, decode=True)
            sel = None
        else:  # explicit experts and weights
            lg = None
            ids = np.argsort(synth.u64(3, f"F/{name}/ids", E), kind="stable")[:k].astype(np.int32)[None, :]
            wts = synth.uniform(3, f"F/{name}/w", k).astype(np.float32)[None, :]
            ref = run_layer(dl, x, k, shared, ids=ids, w=wts, acc=acc0, decode=True)
            sel = (ids, wts)
        r = Run(1, E, k, shared, H, I)
        if sel is not None:
            r.ids[:, :k] = dev(sel[0])
            r.w[:, :k] = dev(sel[1])
        acc_d = dev(acc0.astype(np.float32))
        moe.layer_decode_q(dl.desc, None if lg is None else dev(lg), dev(x), k, shared, r.ids, r.w, r.counts,
                           r.offsets, r.sorted_slot, r.slot_pos, r.work, acc_d, ws)
        got = r.host()
        for key in ("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos", "work"):
            np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
        assert np.array_equal(acc_d.cpu().numpy().view(np.uint32), ref["acc"].view(np.uint32))
        counted, error = call_counts(ws)
        if call == 0:
            n_wg = counted                               # workgroups per launch
            assert n_wg > 0
        assert counted == (call + 1) * n_wg              # every workgroup counts every call
        assert error == 0                                # no wait timed out


@pytest.mark.parametrize("kind", TIE_KINDS)
def test_fused_decode_ties(layers, ogrids, kind):
    """The one-launch decode on logits full of ties and signed zeros (field shape: 512
    experts + shared, top-10; few_values and all_zero take the fallback selection):
    ids bit-exact against the oracle, acc within the bound, and the same bits as the
    three calls."""
    name = "decode_iq2_top10_shared"
    banks, H, I, E, shared, T, k, zipf = LAYER_CASES[name]
    sl, tab, dl = layers(name)
    kp = k + shared
    ws = torch.zeros(moe.decode_workspace_bytes(kp, I) // 4, dtype=torch.int32, device="cuda")
    log(f"fused decode ties {kind}")
    x = synth.activations(1, H, tag=f"FT/{kind}/x")
    lg = synth.tie_logits(kind, 1, E, tag=f"FT/{kind}/l")
    ref3 = run_layer(dl, x, k, shared, logits=lg, decode=True)
    r = Run(1, E, k, shared, H, I)
    acc_d = torch.zeros((1, H), dtype=torch.float32, device="cuda")
    moe.layer_decode_q(dl.desc, dev(lg), dev(x), k, shared, r.ids, r.w, r.counts, r.offsets, r.sorted_slot,
                       r.slot_pos, r.work, acc_d, ws)
    got = r.host()
    acc = acc_d.cpu().numpy()
    ref = O.moe_layer(tab, ogrids, x, k, shared, logits=lg)
    np.testing.assert_array_equal(got["ids"], ref["ids"])
    np.testing.assert_allclose(got["w"], ref["w"], rtol=8 * 2.0 ** -24, atol=0)
    assert_rows_close(acc, ref["acc"], f"fused ties {kind} acc")
    for key in ("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos", "work"):
        np.testing.assert_array_equal(got[key], ref3[key], err_msg=key)
    assert np.array_equal(acc.view(np.uint32), ref3["acc"].view(np.uint32))
    assert call_counts(ws)[1] == 0


def test_fused_decode_workspace_shared_across_shapes(layers):
    """One workspace serves layers of different shapes (inter 512 and 256, different
    slot counts) in any order: every call matches the three calls bit for bit and
    advances the barrier words by one round."""
    names = ["decode_iq2_top10_shared", "decode_mixed_i256_shared", "decode_mixed_i256_shared",
             "decode_iq2_top10_shared", "tiny16_top4_iq2", "decode_mixed_i256_shared"]
    ws = torch.zeros(moe.decode_workspace_bytes(moe.MAX_K + 1, 512) // 4, dtype=torch.int32, device="cuda")
    n_wg = None
    for call, name in enumerate(names):
        banks, H, I, E, shared, T, k, zipf = LAYER_CASES[name]
        log(f"shared workspace call {call}: {name}")
        sl, tab, dl = layers(name)
        x = synth.activations(1, H, tag=f"W/{call}/x")
        acc0 = synth.activations(1, H, tag=f"W/{call}/acc")
        lg = synth.logits(1, E, tag=f"W/{call}/l", zipf_alpha=zipf)
        ref = run_layer(dl, x, k, shared, logits=lg, acc=acc0, decode=True)
        r = Run(1, E, k, shared, H, I)
        acc_d = dev(acc0.astype(np.float32))
        moe.layer_decode_q(dl.desc, dev(lg), dev(x), k, shared, r.ids, r.w, r.counts, r.offsets, r.sorted_slot,
                           r.slot_pos, r.work, acc_d, ws)
        got = r.host()
        for key in ("ids", "w", "counts", "offsets", "sorted_slot", "slot_pos", "work"):
            np.testing.assert_array_equal(got[key], ref[key], err_msg=key)
        assert np.array_equal(acc_d.cpu().numpy().view(np.uint32), ref["acc"].view(np.uint32)), name
        counted, error = call_counts(ws)
        n_wg = counted if n_wg is None else n_wg
        assert counted == (call + 1) * n_wg
        assert error == 0


def test_permutation_invariance_and_determinism(layers):
    sl, tab, dl = layers("small_mixed_ragged")
    T, k = 7, 6
    x = synth.activations(T, 512, tag="perm/x")
    ids = np.stack([np.argsort(synth.u64(5, f"perm/{t}", 32), kind="stable")[:k] for t in range(T)]).astype(np.int32)
    w = synth.uniform(5, "perm/w", T * k).reshape(T, k).astype(np.float32)
    base = run_layer(dl, x, k, True, ids=ids, w=w)["acc"]
    again = run_layer(dl, x, k, True, ids=ids, w=w)["acc"]
    assert np.array_equal(base.view(np.uint32), again.view(np.uint32))
    for s in range(3):
        p = np.stack([np.argsort(synth.u64(s, f"pp/{t}", k), kind="stable") for t in range(T)])
        got = run_layer(dl, x, k, True, ids=np.take_along_axis(ids, p, 1), w=np.take_along_axis(w, p, 1))["acc"]
        assert np.array_equal(got.view(np.uint32), base.view(np.uint32))


def test_single_expert_weight_one(layers, ogrids):
    sl, tab, dl = layers("small_mixed_ragged")
    x = synth.activations(3, 512, tag="one/x")
    ids = np.array([[3], [20], [31]], np.int32)
    g = run_layer(dl, x, 1, False, ids=ids, w=np.ones((3, 1), np.float32))
    for t in range(3):
        ref = O.expert_ffn(tab, int(ids[t, 0]), ogrids, x[t])
        assert_rows_close(g["acc"][t], ref, f"single expert {ids[t, 0]}")
        # 0 + 1.0 * y == y exactly on the device too
        np.testing.assert_array_equal(g["acc"][t], y_in_slot_order(g)[t])


def test_rmsnorm_matches_oracle():
    h = synth.activations(33, 2048, tag="rms/h") * 3.0
    out = torch.empty((33, 2048), dtype=torch.float32, device="cuda")
    moe.rmsnorm(dev(h), 33, 2048, 1e-6, out)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out.cpu().numpy(), O.rmsnorm(h, 1e-6), rtol=4e-6, atol=1e-7)
    hd = dev(h)
    moe.rmsnorm(hd, 33, 2048, 1e-6, hd)  # in place
    np.testing.assert_array_equal(hd.cpu().numpy(), out.cpu().numpy())


@pytest.mark.parametrize("qt", [IQ2, IQ1])
def test_tile_longer_than_one_pass(grids, ogrids, qt):
    """A caller's work list may hold a matrix-core tile of more than 16 tokens (the
    grouping never writes one): both tile kernels then run it in passes of 16.  One tile
    of 40 tokens of expert 3, built by hand; every token's y against the oracle's FFN."""
    T, E, H, I, e = 40, 8, 2048, 512, 3
    log(f"tile of {T} tokens, format {qt}")
    sl = synth.make_layer([(qt, E)], hidden=H, inter=I, n_experts=E, has_shared=0, tag=f"L/longtile/{qt}")
    dl = device_layer(sl, grids)
    tab = O.ExpertTable(sl)
    x = synth.activations(T, H, tag=f"longtile/{qt}/x")
    n_ids = E
    work = np.zeros(moe.work_ints(T, 1, n_ids), np.int32).reshape(-1, 4)
    work[0] = [0, T, 1, 1]               # no mat-vec expert, T slots, one expert, one tile
    work[n_ids + 1] = [e, 0, T, 0]       # the tile: expert e, sorted positions 0 .. T
    ss = dev(np.arange(T, dtype=np.int32))  # one slot per token, already in order
    h = torch.zeros((T, I), dtype=torch.float32, device="cuda")
    y = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    wk = dev(work.reshape(-1))
    xd = dev(x)
    moe.expert_gateup_q(dl.desc, xd, T, 1, ss, wk, h)
    moe.expert_down_q(dl.desc, h, T, 1, wk, y)
    torch.cuda.synchronize()
    ref = np.stack([O.expert_ffn(tab, e, ogrids, x[t]) for t in range(T)])
    assert_rows_close(y.cpu().numpy(), ref, f"tile of {T} tokens, format {qt}")
