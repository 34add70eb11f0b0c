"""Pins for the oracle's number formats and packed-code stream.

Nothing here re-types the oracle's formulas: each check compares the oracle
with something fixed independently of it -- hand-packed words, numpy's own
fp16 / bit-unpacking routines, reinterpreting the stream as bytes, or the
bits-per-weight figures the model cards print.
"""
import os

import numpy as np
import pytest

import oracle
import synth
from conftest import GOLDEN, parse_packed_blocks


@pytest.fixture(scope="module", autouse=True)
def _built():
    oracle.build(force=False)


def test_half_decode_matches_numpy_all_patterns():
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.half_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signs of zero are kept
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_bf16_decode_matches_upper_half_of_binary32_all_patterns():
    pats = np.arange(1 << 16, dtype=np.uint32)
    ref = (pats << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    got = np.array([oracle.bf16_to_double(int(p)) for p in pats])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("case", parse_packed_blocks(), ids=lambda c: f"b{c[0]}")
def test_hand_packed_blocks_unpack(case):
    bits, codes, words = case
    assert len(words) == bits, "a 32-code block is exactly b words"
    got = oracle.unpack_row(np.array(words, dtype=np.uint32), bits, 32)
    assert got.tolist() == codes


@pytest.mark.parametrize("case", parse_packed_blocks(), ids=lambda c: f"b{c[0]}")
def test_generator_packs_hand_blocks(case):
    bits, codes, words = case
    packed = synth.pack_codes(np.array([codes], dtype=np.uint32), bits)
    assert packed[0].tolist() == words


def test_b8_stream_is_a_byte_array():
    rng = np.random.default_rng(7)
    words = rng.integers(0, 1 << 32, size=40, dtype=np.uint32)
    got = oracle.unpack_row(words, 8, 160)
    assert np.array_equal(got, np.frombuffer(words.astype("<u4").tobytes(), dtype=np.uint8))


def test_b16_stream_is_a_uint16_array():
    rng = np.random.default_rng(8)
    words = rng.integers(0, 1 << 32, size=32, dtype=np.uint32)
    got = oracle.unpack_row(words, 16, 64)
    assert np.array_equal(got, np.frombuffer(words.astype("<u4").tobytes(), dtype="<u2"))


@pytest.mark.parametrize("bits", list(range(1, 17)))
def test_unpack_matches_numpy_unpackbits(bits):
    rng = np.random.default_rng(100 + bits)
    n_blocks = 3
    words = rng.integers(0, 1 << 32, size=n_blocks * bits, dtype=np.uint32)
    stream = np.unpackbits(np.frombuffer(words.astype("<u4").tobytes(), dtype=np.uint8),
                           bitorder="little").astype(np.uint64)
    n = 32 * n_blocks
    fields = stream[: n * bits].reshape(n, bits)
    ref = (fields << np.arange(bits, dtype=np.uint64)).sum(axis=1)
    got = oracle.unpack_row(words, bits, n)
    assert np.array_equal(got.astype(np.uint64), ref)


@pytest.mark.parametrize("bits", [8, 9, 10, 11, 12, 13])
def test_every_code_at_every_block_position(bits):
    """Brute force: every value 0..2^b-1 appears at every position j mod 32
    (all straddle offsets) and round-trips through generator and oracle."""
    K = 1 << bits
    rows = []
    for v0 in range(0, K, 32):
        base = np.arange(v0, v0 + 32, dtype=np.uint32) % K
        for rot in range(32):
            rows.append(np.roll(base, rot))
    codes = np.stack(rows)
    packed = synth.pack_codes(codes, bits)
    # one-block rows laid end to end form one continuous stream
    got = oracle.unpack_row(packed.ravel(), bits, codes.size)
    assert np.array_equal(got, codes.ravel())


def test_words_per_row_padding():
    # 176 codes = 5.5 blocks -> 6 blocks of 11 words (the down projection of
    # a 704-wide expert at d=4, 11-bit)
    assert oracle.words_per_row(704, 4, 11) == 66
    assert oracle.words_per_row(2048, 4, 9) == 144
    assert oracle.words_per_row(4096, 2, 8) == 512
    assert oracle.words_per_row(4096, 2, 10) == 640
    for cols, d, bits in [(704, 4, 11), (2048, 4, 9), (512, 2, 8), (64, 8, 13)]:
        assert oracle.words_per_row(cols, d, bits) == synth.words_per_row(cols, d, bits)


def _golden_bpw():
    rows = []
    with open(os.path.join(GOLDEN, "bits_per_weight.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                d, bits, bpw = line.split()
                rows.append((int(d), int(bits), float(bpw)))
    return rows


@pytest.mark.parametrize("d,bits,bpw", _golden_bpw())
def test_stored_bits_per_weight_match_cards(d, bits, bpw):
    """Codes + fp16 group scales, stored as the oracle reads them, cost the
    bits per weight the model cards print."""
    rows, cols = 16, 2048
    T = synth.make_tensor(1, 1, rows=rows, cols=cols, d=d, bits=bits)
    wpr = oracle.words_per_row(cols, d, bits)
    assert T.codes.shape == (rows, wpr)
    stored_bits = 8 * (T.codes.nbytes + T.scales.nbytes)
    assert stored_bits / (rows * cols) == pytest.approx(bpw, abs=1e-12)
