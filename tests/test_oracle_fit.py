"""Pins for the oracle's fit of the format (scales, k-means / Lloyd over the
weight subvectors, fp16 codebook, encode and pack): numpy's IEEE conversions
and arithmetic, brute-force argmin, closed forms and invariants of Lloyd's
algorithm (the cards' "Methodology" sections name k-means / Lloyd over the
weight subvectors, data-free)."""
import numpy as np
import pytest

import oracle
import synth


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def _bf16(x):
    return synth.to_bf16_bits(np.asarray(x, dtype=np.float32))


def _bf16_to_f32(h):
    return (np.asarray(h, dtype=np.uint32) << 16).view(np.float32)


def _weights(seed, n_rows, cols, spread=0.02):
    """bf16 weights ~ N(0, spread) with a heavier tail, as trained experts have."""
    g = np.random.default_rng(seed)
    w = g.standard_normal((n_rows, cols)) * spread
    w *= np.where(g.random((n_rows, cols)) < 0.02, 4.0, 1.0)
    return _bf16(w)


def _normalised(w, scales, d):
    """fp32 v = w / s per subvector (IEEE division), zeros where s == 0."""
    n, cols = w.shape
    wf = _bf16_to_f32(w).reshape(n, cols // 64, 64)
    s = scales.view(np.float16).astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s == 0, np.float32(0), wf / s).astype(np.float32)
    return v.reshape(n * cols // d, d)


def _nearest_bruteforce(v, C):
    """argmin over k of sum_t (v_t - c_t)^2, fp32 with every op rounded, the
    terms added in t order; first minimum wins."""
    acc = np.zeros((v.shape[0], C.shape[0]), dtype=np.float32)
    for t in range(v.shape[1]):
        diff = (v[:, t:t + 1] - C[None, :, t]).astype(np.float32)
        acc = (acc + (diff * diff).astype(np.float32)).astype(np.float32)
    return np.argmin(acc, axis=1)


# --------------------------------------------------------------------------

def test_float_to_half_matches_numpy():
    g = np.random.default_rng(1)
    halves = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (halves[:-1] + halves[1:]) / 2          # exact ties in fp32
    vals = np.concatenate([
        halves, mids, -mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
        np.nextafter(mids.astype(np.float32), np.float32(-np.inf)),
        g.standard_normal(20000) * 10.0 ** g.integers(-9, 6, 20000),
        [65504.0, 65519.99, 65520.0, 1e9, 0.0, -0.0, 2.0 ** -25, 2.0 ** -26, 3 * 2.0 ** -25],
    ]).astype(np.float32)
    got = np.array([oracle.float_to_half(float(v)) for v in vals], dtype=np.uint16)
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_scales_are_fp16_group_absmax():
    w = _weights(2, 37, 320)
    w[3, 64:128] = 0                                   # an all-zero group
    got = oracle.fit_scales(w)
    want = np.abs(_bf16_to_f32(w)).reshape(37, 5, 64).max(-1).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)
    assert got[3, 1] == 0


@pytest.mark.parametrize("d,bits,K", [(2, 8, 256), (4, 9, 512), (8, 10, 300), (2, 11, 2048)])
def test_encode_is_bruteforce_argmin_then_packing(d, bits, K):
    n, cols = 9, 192
    w = _weights(3 + d, n, cols)
    sc = oracle.fit_scales(w)
    cb = synth.to_half_bits(np.random.default_rng(4).uniform(-1, 1, (K, d)))
    got = oracle.encode(w, sc, cb, d, bits)
    v = _normalised(w, sc, d)
    codes = _nearest_bruteforce(v, cb.view(np.float16).astype(np.float32))
    assert np.array_equal(got, synth.pack_codes(codes.reshape(n, cols // d), bits))


def test_kmeans_zero_iterations_is_the_initial_draw():
    w = _weights(5, 20, 128)
    sc = oracle.fit_scales(w)
    init = np.array([3, 17, 40, 639, 0, 5], dtype=np.int64)
    C = oracle.kmeans(w, sc, 4, 6, np.arange(640), init, 0)
    assert np.array_equal(C, _normalised(w, sc, 4)[init])


def _clustered(d, K, per, seed):
    """Weights whose groups all hold a 1.0 (so s = 1 and v = w exactly) and
    whose other subvectors are K centres on a 1/64 grid plus symmetric
    offsets of +-1/128 in coordinate 0: every cluster mean is its centre."""
    g = np.random.default_rng(seed)
    centres = g.integers(-40, 40, (K, d)) / 64.0
    subs = []
    for k in range(K):
        for p in range(per):
            off = np.zeros(d)
            off[0] = (1 if p % 2 == 0 else -1) / 128.0
            subs.append(centres[k] + off)
    subs = np.array(subs)
    g.shuffle(subs)
    n_sub_row = 64 // d - 1          # one subvector per group carries the 1.0
    rows = []
    for i in range(0, len(subs), n_sub_row):
        chunk = subs[i:i + n_sub_row]
        if len(chunk) < n_sub_row:
            break
        rows.append(np.concatenate([np.ones(d), chunk.ravel()]))
    w = _bf16(np.array(rows))
    return w, centres


def test_kmeans_recovers_separated_cluster_means():
    d, K = 4, 8
    w, centres = _clustered(d, K, 60, 6)    # 480 subvectors: 32 whole rows
    sc = oracle.fit_scales(w)
    assert np.all(sc == synth.to_half_bits(np.ones(1))[0])
    v = _normalised(w, sc, d)
    data = np.nonzero(np.any(v != 1.0, axis=1))[0]      # every subvector but the 1.0s
    # start from one member of each cluster
    lab = [int(np.argmin(np.abs(centres - x).sum(1))) for x in v[data]]
    init = np.array([data[lab.index(k)] for k in range(K)], dtype=np.int64)
    C = oracle.kmeans(w, sc, d, K, data, init, 3)
    assert np.array_equal(C.astype(np.float64), centres)


def test_kmeans_sample_order_does_not_matter():
    w = _weights(7, 64, 256)
    sc = oracle.fit_scales(w)
    g = np.random.default_rng(8)
    sample = g.choice(64 * 64, 3000, replace=False)
    init = g.choice(64 * 64, 32, replace=False)
    a = oracle.kmeans(w, sc, 4, 32, sample, init, 5)
    b = oracle.kmeans(w, sc, 4, 32, g.permutation(sample), init, 5)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_lloyd_distortion_never_increases():
    w = _weights(9, 48, 256)
    sc = oracle.fit_scales(w)
    g = np.random.default_rng(10)
    sample = g.choice(48 * 128, 4000, replace=False)
    init = g.choice(48 * 128, 64, replace=False)
    v = _normalised(w, sc, 2)[sample].astype(np.float64)
    prev = np.inf
    for it in range(7):
        C = oracle.kmeans(w, sc, 2, 64, sample, init, it).astype(np.float64)
        sse = ((v[:, None, :] - C[None]) ** 2).sum(-1).min(1).sum()
        assert sse <= prev * (1 + 1e-9)
        prev = sse


def test_k1_centroid_is_the_sample_mean():
    w = _weights(11, 16, 128)
    sc = oracle.fit_scales(w)
    sample = np.arange(0, 16 * 32, 3)
    C = oracle.kmeans(w, sc, 4, 1, sample, [0], 2)
    mean = _normalised(w, sc, 4)[sample].astype(np.float64).mean(0)
    np.testing.assert_allclose(C[0], mean, rtol=0, atol=2.0 ** -29)


def test_empty_cluster_keeps_its_centroid():
    """Subvector 0 is made an outlier near (1, 1, 1, 1) and left out of the
    fit set: the cluster started from it gets no member and keeps its value,
    while the others move."""
    w = _weights(12, 8, 64)
    w[0, :4] = _bf16(np.full(4, 0.06))
    w[0, 4:64] = _bf16(np.zeros(60))
    sc = oracle.fit_scales(w)
    v = _normalised(w, sc, 4)
    sample = np.arange(1, 8 * 16)
    C = oracle.kmeans(w, sc, 4, 3, sample, [0, 5, 9], 4)
    assert np.array_equal(C[0], v[0])
    assert not np.array_equal(C[1:], v[[5, 9]])


def test_fit_reproduces_exactly_representable_weights():
    """Weights built from a known fp16 codebook, codes and power-of-two
    scales are fitted back exactly when the fit starts from the true
    entries: same codebook, scales, codes, and decode(fit) == w."""
    d, bits, K, n, cols = 2, 8, 16, 12, 128
    g = np.random.default_rng(13)
    entries = np.unique(g.integers(-32, 33, (64, d)), axis=0)[:K] / 32.0
    entries[0] = [1.0, -1.0]                        # group maxima are exactly 1
    codes = g.integers(1, K, (n, cols // d))
    codes[:, ::32] = 0                              # every group holds entry 0
    scale = 2.0 ** -g.integers(3, 7, (n, cols // 64))
    wv = entries[codes].reshape(n, cols // 64, 64) * scale[:, :, None]
    w = _bf16(wv.reshape(n, cols))
    first = {}
    for i, c in enumerate(codes.ravel()):
        first.setdefault(int(c), i)
    init = np.array([first[k] for k in range(K)], dtype=np.int64)
    cb, sc, packed = oracle.fit(w, d, bits, K, np.arange(n * cols // d), init, 3)
    assert np.array_equal(cb, synth.to_half_bits(entries))
    assert np.array_equal(sc, synth.to_half_bits(scale))
    assert np.array_equal(packed, synth.pack_codes(codes, bits))
    T = synth.VQTensorHost(n, cols, d, bits, K, 1, cb, packed, sc, None)
    assert np.array_equal(oracle.decode(T, 0), _bf16_to_f32(w).reshape(n, cols))


def test_fit_reconstruction_error_is_small():
    d, bits, K, n, cols = 2, 8, 256, 96, 512
    w = _weights(14, n, cols)
    g = np.random.default_rng(15)
    N = n * cols // d
    cb, sc, packed = oracle.fit(w, d, bits, K, g.choice(N, 8000, replace=False),
                                g.choice(N, K, replace=False), 8)
    T = synth.VQTensorHost(n, cols, d, bits, K, 1, cb, packed, sc, None)
    wf = _bf16_to_f32(w).reshape(n, cols).astype(np.float64)
    err = np.linalg.norm(oracle.decode(T, 0) - wf) / np.linalg.norm(wf)
    assert err < 0.12, err


def test_fit_is_its_steps_composed():
    """The whole fit equals scales, then k-means, then each centroid rounded
    to fp16 (round to nearest even, numpy's conversion), then encode: the
    large fit is checked step by step on that basis."""
    d, bits, K, n, cols = 4, 9, 64, 40, 256
    w = _weights(16, n, cols)
    g = np.random.default_rng(17)
    N = n * cols // d
    sample = np.sort(g.choice(N, 2000, replace=False))
    init = g.choice(N, K, replace=False)
    cb, sc, packed = oracle.fit(w, d, bits, K, sample, init, 4)
    sc2 = oracle.fit_scales(w)
    C = oracle.kmeans(w, sc2, d, K, sample, init, 4)
    cb2 = C.astype(np.float16).view(np.uint16)
    assert np.array_equal(sc, sc2)
    assert np.array_equal(cb, cb2)
    assert np.array_equal(packed, oracle.encode(w, sc2, cb2, d, bits))
