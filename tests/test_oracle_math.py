"""Pins for the oracle's decode, matmul and routed SwiGLU FFN.

Each check is fixed by something other than the oracle's own code: a
brute-force triple loop over integer codes with numpy's fp16, closed forms
(K = 1, integer codebooks), invariants the model cards state (dead rows are
exact zeros; packing is a pure representation change), numpy / scipy library
routines, and linearity.  The cases are chosen so that a dropped term, a wrong
index or sign, or a transposed operand fails at least one of them.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _brute_decode(T, e):
    """Python loops over the integer codes, numpy fp16 for the values."""
    cb = T.codebook.view(np.float16).astype(np.float64)
    sc = T.scales.view(np.float16).astype(np.float64)
    W = np.zeros((T.rows, T.cols), dtype=np.float64)
    for r in range(T.rows):
        s = e * T.rows + r if T.row_map is None else T.row_map[e * T.rows + r]
        if s < 0:
            continue
        for j in range(T.n_sub):
            code = int(T.raw_codes[s, j])
            for t in range(T.d):
                c = j * T.d + t
                W[r, c] = sc[s, c // 64] * cb[code, t]
    return W


GEOMS = [(2, 8, 4), (4, 9, 3), (2, 10, 4), (4, 11, 2), (8, 13, 4), (1, 3, 2)]


@pytest.mark.parametrize("d,bits,K", GEOMS)
@pytest.mark.parametrize("cols", [64, 128, 192])
def test_decode_brute_force_tiny(d, bits, K, cols):
    T = synth.make_tensor(11, d * 100 + bits, rows=4, cols=cols, d=d, bits=bits, K=K,
                          n_experts=2, keep_codes=True)
    for e in range(2):
        W = oracle.decode(T, e)
        ref = _brute_decode(T, e)
        # exact: fp16 x fp16 fits in fp32
        assert np.array_equal(W.astype(np.float64), ref)


@pytest.mark.parametrize("d,bits", [(2, 8), (4, 9), (4, 11), (2, 10)])
def test_skipzero_rows_are_positive_zero_and_live_rows_unchanged(d, bits):
    """Dead rows output exact zeros, live rows are identical to the full-row
    tensor ("Qwen3.5-397B-A17B-VQ-2.4bpw: Model Card", changelog 2026-10-01)."""
    rows, cols, E = 12, 256, 3
    full = synth.make_tensor(5, 1, rows=rows, cols=cols, d=d, bits=bits, n_experts=E,
                             keep_codes=True)
    rng = np.random.default_rng(9)
    row_map = np.full(E * rows, -1, dtype=np.int32)
    keep = []
    for e in range(E):
        live = np.sort(rng.choice(rows, size=rows - 4, replace=False))
        for r in live:
            row_map[e * rows + r] = len(keep)
            keep.append(e * rows + r)
    keep = np.array(keep)
    sz = synth.VQTensorHost(rows, cols, d, bits, full.K, E, full.codebook,
                            full.codes[keep], full.scales[keep], row_map, full.raw_codes[keep])
    x = synth.make_x(3, 3, 2, cols, "f32")
    for e in range(E):
        Wf, Ws = oracle.decode(full, e), oracle.decode(sz, e)
        dead = row_map[e * rows:(e + 1) * rows] < 0
        assert np.all(Ws[dead].view(np.uint32) == 0)           # +0.0 bit patterns
        assert np.array_equal(Ws[~dead].view(np.uint32), Wf[~dead].view(np.uint32))
        ys = oracle.linear(sz, e, x)
        assert np.all(ys[:, dead].view(np.uint64) == 0)
        yf = oracle.linear(full, e, x)
        assert np.array_equal(ys[:, ~dead], yf[:, ~dead])


def test_skipzero_equals_full_rows_with_zero_scales():
    rows, cols = 8, 128
    T = synth.make_tensor(6, 1, rows=rows, cols=cols, d=4, bits=9, keep_codes=True)
    dead = np.array([1, 4, 7])
    zs = T.scales.copy()
    zs[dead] = 0
    Z = synth.VQTensorHost(rows, cols, 4, 9, T.K, 1, T.codebook, T.codes, zs, None)
    live = np.setdiff1d(np.arange(rows), dead)
    row_map = np.full(rows, -1, dtype=np.int32)
    row_map[live] = np.arange(len(live))
    S = synth.VQTensorHost(rows, cols, 4, 9, T.K, 1, T.codebook, T.codes[live], T.scales[live],
                           row_map)
    x = synth.make_x(6, 2, 3, cols, "bf16")
    assert np.array_equal(oracle.linear(Z, 0, x), oracle.linear(S, 0, x))


def test_k1_codebook_closed_form():
    """K = 1 (b = 0): every subvector is the same codebook entry c, so
    y[r] = sum_g s[r][g] * sum_{j in g} sum_t c[t] x[j*d + t]."""
    rows, cols, d = 5, 256, 4
    T = synth.make_tensor(7, 1, rows=rows, cols=cols, d=d, bits=0, K=1, keep_codes=True)
    assert T.codes.shape == (rows, 0)
    x = synth.make_x(7, 2, 2, cols, "f32").astype(np.float64)
    c = T.codebook.view(np.float16).astype(np.float64)[0]
    s = T.scales.view(np.float16).astype(np.float64)
    xg = x.reshape(2, cols // 64, 64 // d, d)
    inner = (xg * c).sum(axis=(2, 3))                   # [n, groups]
    ref = inner @ s.T                                   # [n, rows]
    got = oracle.linear(T, 0, x)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_identical_entries_equal_k1():
    """At b = 8, a codebook whose 256 entries are all equal behaves like K=1."""
    rows, cols, d = 6, 192, 2
    T = synth.make_tensor(8, 1, rows=rows, cols=cols, d=d, bits=8)
    cb = np.repeat(T.codebook[:1], 256, axis=0)
    T8 = synth.VQTensorHost(rows, cols, d, 8, 256, 1, cb, T.codes, T.scales, None)
    T0 = synth.VQTensorHost(rows, cols, d, 0, 1, 1, T.codebook[:1],
                            np.zeros((rows, 0), np.uint32), T.scales, None)
    x = synth.make_x(8, 2, 2, cols, "f32")
    assert np.array_equal(oracle.linear(T8, 0, x), oracle.linear(T0, 0, x))


def test_integer_codebook_exact_integer_matmul():
    """Entries in {0, 1}, unit scales and small integer x give an exact
    integer product, compared with numpy's integer matmul."""
    rows, cols, d, bits = 7, 320, 4, 4
    K = 16
    cb = np.array([[(k >> t) & 1 for t in range(d)] for k in range(K)], dtype=np.float64)
    T = synth.make_tensor(9, 1, rows=rows, cols=cols, d=d, bits=bits, K=K, keep_codes=True)
    T.codebook = synth.to_half_bits(cb)
    T.scales = synth.to_half_bits(np.ones_like(T.scales, dtype=np.float64))
    W_int = np.zeros((rows, cols), dtype=np.int64)
    for r in range(rows):
        for j in range(cols // d):
            k = int(T.raw_codes[r, j])
            for t in range(d):
                W_int[r, j * d + t] = (k >> t) & 1
    xi = np.random.default_rng(1).integers(-8, 9, size=(3, cols))
    got = oracle.linear(T, 0, xi.astype(np.float32))
    assert np.array_equal(got, (xi @ W_int.T).astype(np.float64))


def test_orientation_out_by_in():
    """W is [out][in]: a weight that is non-zero only at (row 2, col 70)
    sends x[70] to y[2] and nowhere else."""
    rows, cols, d = 4, 128, 2
    codes = np.zeros((rows, cols // d), dtype=np.uint32)
    codes[2, 35] = 1                                     # subvector 35 = cols 70, 71
    cb = synth.to_half_bits(np.array([[0.0, 0.0], [1.0, 0.0]]))
    sc = synth.to_half_bits(np.ones((rows, 2)))
    T = synth.VQTensorHost(rows, cols, d, 1, 2, 1, cb, synth.pack_codes(codes, 1), sc, None)
    x = np.zeros((1, cols), dtype=np.float32)
    x[0, 70] = 3.0
    y = oracle.linear(T, 0, x)
    ref = np.zeros((1, rows))
    ref[0, 2] = 3.0
    assert np.array_equal(y, ref)
    x[0, 70], x[0, 71] = 0.0, 5.0                       # second element of the pair
    assert np.array_equal(oracle.linear(T, 0, x), np.zeros((1, rows)))


def test_group_scale_indexing():
    """Scale g applies to columns [64g, 64g+64) only."""
    rows, cols, d = 2, 256, 4
    T = synth.make_tensor(12, 1, rows=rows, cols=cols, d=d, bits=5, K=32, keep_codes=True)
    W = oracle.decode(T, 0).astype(np.float64)
    s = T.scales.view(np.float16).astype(np.float64)
    cb = T.codebook.view(np.float16).astype(np.float64)
    for r in range(rows):
        for g in range(cols // 64):
            sub = T.raw_codes[r, g * 16:(g + 1) * 16]
            np.testing.assert_array_equal(W[r, 64 * g:64 * g + 64], s[r, g] * cb[sub].ravel())


@pytest.mark.parametrize("d,bits", [(2, 8), (4, 9), (2, 10), (4, 11)])
def test_linear_matches_numpy_matmul_of_decoded(d, bits):
    T = synth.make_tensor(13, bits, rows=48, cols=384, d=d, bits=bits, n_experts=2)
    for xdt in ("f32", "bf16"):
        x = synth.make_x(13, 5, 3, 384, xdt)
        xv = x.astype(np.float64) if xdt == "f32" else \
            (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        for e in range(2):
            ref = xv @ oracle.decode(T, e).astype(np.float64).T
            np.testing.assert_allclose(oracle.linear(T, e, x), ref, rtol=1e-12, atol=1e-12)


def test_linearity_in_x_and_scales():
    T = synth.make_tensor(14, 1, rows=16, cols=256, d=4, bits=9)
    x1 = synth.make_x(14, 1, 2, 256, "f32").astype(np.float64)
    x2 = synth.make_x(14, 2, 2, 256, "f32").astype(np.float64)
    y = oracle.linear(T, 0, x1 + 2 * x2)
    np.testing.assert_allclose(y, oracle.linear(T, 0, x1) + 2 * oracle.linear(T, 0, x2),
                               rtol=1e-12, atol=1e-12)
    T2 = synth.VQTensorHost(T.rows, T.cols, T.d, T.bits, T.K, 1, T.codebook, T.codes,
                            synth.to_half_bits(2 * T.scales.view(np.float16).astype(np.float64)),
                            None)
    np.testing.assert_array_equal(oracle.linear(T2, 0, x1), 2 * oracle.linear(T, 0, x1))


def test_codebook_permutation_invariance():
    """Permuting the codebook and re-coding every index gives the same W."""
    rows, cols, d, bits = 6, 256, 2, 8
    T = synth.make_tensor(15, 1, rows=rows, cols=cols, d=d, bits=bits, K=200, keep_codes=True)
    perm = np.random.default_rng(3).permutation(200)
    inv = np.argsort(perm)
    cb2 = T.codebook[perm]                       # cb2[i] = cb[perm[i]]
    codes2 = inv[T.raw_codes]                    # cb2[inv[k]] = cb[k]
    T2 = synth.VQTensorHost(rows, cols, d, bits, 200, 1, cb2, synth.pack_codes(codes2, bits),
                            T.scales, None)
    assert np.array_equal(oracle.decode(T, 0).view(np.uint32), oracle.decode(T2, 0).view(np.uint32))


def test_check_rejects_bad_inputs():
    T = synth.make_tensor(16, 1, rows=4, cols=64, d=2, bits=8, K=100, keep_codes=True)
    oracle.check(T)
    bad = synth.VQTensorHost(4, 64, 2, 8, 100, 1, T.codebook,
                             synth.pack_codes(np.full((4, 32), 150), 8), T.scales, None)
    with pytest.raises(ValueError):
        oracle.check(bad)
    with pytest.raises(ValueError):
        oracle.decode(bad, 0)
    dup = synth.VQTensorHost(4, 64, 2, 8, 100, 1, T.codebook, T.codes, T.scales,
                             np.array([0, 1, 1, 2], dtype=np.int32))
    with pytest.raises(ValueError):
        oracle.check(dup)


def test_swiglu_matches_scipy_expit():
    for g in np.linspace(-30, 30, 61):
        for u in (-2.5, 0.0, 1.0, 3.25):
            assert oracle.swiglu(g, u) == pytest.approx(g * expit(g) * u, rel=1e-14, abs=1e-300)


def _ffn_by_composition(gate, up, down, x, ids, w):
    """Routed SwiGLU FFN assembled from numpy matmuls of the decoded weights,
    scipy's logistic function, and an explicit slot loop."""
    xv = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    T, k = ids.shape
    y = np.zeros((T, gate.cols))
    for t in range(T):
        for s in range(k):
            e = ids[t, s]
            g = oracle.decode(gate, e).astype(np.float64) @ xv[t]
            u = oracle.decode(up, e).astype(np.float64) @ xv[t]
            h = g * expit(g) * u
            y[t] += float(w[t, s]) * (oracle.decode(down, e).astype(np.float64) @ h)
    return y


@pytest.mark.parametrize("dead", [0, 3])
def test_moe_ffn_matches_composition(dead):
    E, k, H, I, T = 6, 3, 128, 64, 5
    gate = synth.make_tensor(21, 1, rows=I, cols=H, d=2, bits=8, n_experts=E, dead_rows=dead)
    up = synth.make_tensor(21, 2, rows=I, cols=H, d=2, bits=8, n_experts=E, dead_rows=dead)
    down = synth.make_tensor(21, 3, rows=H, cols=I, d=2, bits=8, n_experts=E, dead_rows=dead)
    x = synth.make_x(21, 4, T, H, "bf16")
    ids, w = synth.make_routes(21, 5, T, E, k)
    got = oracle.moe_ffn(gate, up, down, x, ids, w)
    ref = _ffn_by_composition(gate, up, down, x, ids, w)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)
    # a token subset gives the same rows
    sub = oracle.moe_ffn(gate, up, down, x, ids, w, tokens=[4, 1])
    np.testing.assert_array_equal(sub, got[[4, 1]])


def test_moe_ffn_swapped_slots_change_output():
    """Sensitivity: exchanging the gate weights of two slots changes y (a
    combine that ignored the slot-to-weight pairing would not notice)."""
    E, k, H, I, T = 4, 2, 64, 64, 2
    gate = synth.make_tensor(22, 1, rows=I, cols=H, d=4, bits=9, n_experts=E)
    up = synth.make_tensor(22, 2, rows=I, cols=H, d=4, bits=9, n_experts=E)
    down = synth.make_tensor(22, 3, rows=H, cols=I, d=4, bits=9, n_experts=E)
    x = synth.make_x(22, 4, T, H, "bf16")
    ids = np.array([[0, 1], [2, 3]], dtype=np.int32)
    w = np.array([[0.9, 0.1], [0.3, 0.7]], dtype=np.float32)
    y1 = oracle.moe_ffn(gate, up, down, x, ids, w)
    y2 = oracle.moe_ffn(gate, up, down, x, ids, w[:, ::-1].copy())
    assert np.abs(y1 - y2).max() > 1e-3


# --------------------------------------------------------------------------
# Row gather (the per-layer n-gram embedding tables of the card
# "Qwen3.8-Flash-Next-VQ-4.4bpw" are VQ tensors at d=2/K=256 read by row).
# --------------------------------------------------------------------------

def _brute_row(T, lid):
    """Python loops over the integer codes of one logical row (id = e*rows + r)."""
    cb = T.codebook.view(np.float16).astype(np.float64)
    sc = T.scales.view(np.float16).astype(np.float64)
    s = lid if T.row_map is None else int(T.row_map[lid])
    out = np.zeros(T.cols, dtype=np.float64)
    if s < 0:
        return out
    for j in range(T.n_sub):
        code = int(T.raw_codes[s, j])
        for t in range(T.d):
            out[j * T.d + t] = sc[s, (j * T.d + t) // 64] * cb[code, t]
    return out


@pytest.mark.parametrize("d,bits,K,dead", [(2, 8, 256, 0), (2, 8, 200, 3), (4, 9, 512, 2),
                                           (8, 11, 2048, 0), (2, 10, 1024, 1)])
def test_gather_brute_force_rows(d, bits, K, dead):
    """Each gathered row equals the brute-force decode of that row, over ids in
    random order across tables, with repeats and dead rows."""
    rows, cols, E = 9, 192, 3
    T = synth.make_tensor(21, d * 100 + bits, rows=rows, cols=cols, d=d, bits=bits, K=K,
                          n_experts=E, dead_rows=dead, keep_codes=True)
    rng = np.random.default_rng(3)
    ids = rng.integers(0, E * rows, size=40).astype(np.int64)
    ids[5] = ids[17]
    Y = oracle.gather(T, ids)
    assert Y.shape == (40, cols) and Y.dtype == np.float32
    for i, lid in enumerate(ids):
        assert np.array_equal(Y[i].astype(np.float64), _brute_row(T, int(lid)))


def test_gather_equals_rows_of_decode():
    """Gathering every logical row of every table in order rebuilds the dense
    decode of each table, bit for bit (dead rows +0.0 included)."""
    rows, cols, E = 7, 256, 4
    T = synth.make_tensor(22, 1, rows=rows, cols=cols, d=2, bits=8, n_experts=E, dead_rows=2)
    Y = oracle.gather(T, np.arange(E * rows))
    dense = np.concatenate([oracle.decode(T, e) for e in range(E)])
    assert np.array_equal(Y.view(np.uint32), dense.view(np.uint32))
    dead = np.nonzero(T.row_map < 0)[0]
    assert len(dead) == 2 * E
    assert not Y[dead].view(np.uint32).any()          # +0.0, sign bit clear


def test_gather_closed_form_table():
    """Entries (k, -k/2), scale 2^-(r mod 4) per row and code j of row r equal to
    (3j + 5r) mod 256 give W[r][2j] = (3j+5r mod 256) * 2^-(r mod 4) and
    W[r][2j+1] = -W[r][2j]/2."""
    rows, cols, d = 6, 128, 2
    n_sub = cols // d
    k = np.arange(256, dtype=np.float64)
    cb = synth.to_half_bits(np.stack([k, -k / 2], axis=1))
    raw = np.array([[(3 * j + 5 * r) % 256 for j in range(n_sub)] for r in range(rows)])
    codes = synth.pack_codes(raw, 8)
    sc = synth.to_half_bits(np.repeat((2.0 ** -(np.arange(rows) % 4))[:, None], cols // 64, 1))
    T = synth.VQTensorHost(rows, cols, d, 8, 256, 1, cb, codes, sc, None)
    ids = np.array([5, 0, 3, 3], dtype=np.int64)
    Y = oracle.gather(T, ids)
    for i, r in enumerate(ids):
        v = ((3 * np.arange(n_sub) + 5 * r) % 256) * 2.0 ** -(r % 4)
        assert np.array_equal(Y[i, 0::2], v.astype(np.float32))
        assert np.array_equal(Y[i, 1::2], (-v / 2).astype(np.float32))


def test_gather_out_of_range_ids_are_nan_rows():
    T = synth.make_tensor(23, 1, rows=4, cols=64, d=2, bits=8, n_experts=2)
    ids = np.array([-1, 0, 8, 7, np.iinfo(np.int64).min, 1 << 40], dtype=np.int64)
    Y = oracle.gather(T, ids)
    bad = [0, 2, 4, 5]
    assert np.isnan(Y[bad]).all()
    assert np.isfinite(Y[[1, 3]]).all()
    assert oracle.gather(T, np.zeros(0, np.int64)).shape == (0, 64)


# --------------------------------------------------------------------------
# A stack of MoE layers on a residual stream, layers of mixed geometry (the
# promoted layers of "GLM-5.3-Flash-VQ-2.7bpw" and
# "Qwen3.8-Flash-Next-VQ-4.4bpw").
# --------------------------------------------------------------------------

def _stack_layer(seed, d, bits, hidden=128, inter=64, E=6, top_k=2, n_tok=3, dead=0,
                 zero_w=False):
    G = synth.make_tensor(seed, 1, rows=inter, cols=hidden, d=d, bits=bits, n_experts=E,
                          dead_rows=dead)
    U = synth.make_tensor(seed, 2, rows=inter, cols=hidden, d=d, bits=bits, n_experts=E,
                          dead_rows=dead)
    D = synth.make_tensor(seed, 3, rows=hidden, cols=inter, d=d, bits=bits, n_experts=E,
                          dead_rows=dead)
    ids, w = synth.make_routes(seed, 4, n_tok, E, top_k)
    if zero_w:
        w = np.zeros_like(w)
    return (G, U, D, ids, w)


def _x64(n_tok=3, hidden=128):
    return synth.make_x(60, 1, n_tok, hidden, "f32").astype(np.float64)


def test_stack_one_layer_is_residual_plus_ffn():
    A = _stack_layer(61, 4, 9)
    x = _x64()
    assert np.array_equal(oracle.moe_stack([A], x), x + oracle.moe_ffn(*A[:3], x, A[3], A[4]))


def test_stack_identity_layers():
    """A layer whose down projection is all dead, or whose gate weights are
    all zero, adds exactly nothing; inserting it changes no bit."""
    A, B = _stack_layer(62, 4, 9), _stack_layer(63, 2, 8)
    dead = _stack_layer(64, 4, 11, dead=0)
    dead = (dead[0], dead[1], synth.make_tensor(64, 3, rows=128, cols=64, d=4, bits=11,
                                                n_experts=6, dead_rows=128), dead[3], dead[4])
    zw = _stack_layer(65, 2, 10, zero_w=True)
    x = _x64()
    ref = oracle.moe_stack([A, B], x)
    assert np.array_equal(oracle.moe_stack([A, dead, B], x), ref)
    assert np.array_equal(oracle.moe_stack([zw, A, B, zw], x), ref)
    assert np.array_equal(oracle.moe_stack([dead, zw], x), x)
    assert np.array_equal(oracle.moe_stack([], x), x)


def test_stack_zero_state_stays_zero():
    """silu(0) * 0 = 0: from h = 0 every layer adds exact zeros."""
    layers = [_stack_layer(66 + i, d, b) for i, (d, b) in enumerate([(4, 9), (2, 8), (4, 11)])]
    x = np.zeros((3, 128))
    assert not oracle.moe_stack(layers, x).any()


def test_stack_layer_order_matters():
    A, B = _stack_layer(70, 4, 9), _stack_layer(71, 2, 10)
    x = _x64()
    ab, ba = oracle.moe_stack([A, B], x), oracle.moe_stack([B, A], x)
    assert not np.allclose(ab, ba, rtol=1e-6, atol=0)
    # and the second layer sees the first layer's output, not x
    h1 = oracle.moe_stack([A], x)
    assert np.array_equal(ab, h1 + oracle.moe_ffn(*B[:3], h1, B[3], B[4]))
