"""GPU parity of the row gather (VQ embedding tables read by row) through the
C ABI, against the CPU oracle on the same seeded inputs.  The decode is exact
(fp16 x fp16 fits fp32), so every comparison is bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth
import vq_dequant_matmul_amd as vq

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    vq.load_library()


def _gather(T, W, ids):
    got = vq.vq_row_gather(W, torch.from_numpy(np.ascontiguousarray(ids, np.int64)).cuda())
    torch.cuda.synchronize()
    return got.cpu().numpy()


def _same_bits(a, b):
    return np.array_equal(a.view(np.uint32), b.view(np.uint32))


# d, bits, K: the d2/K256 tables of the card and the other geometries of the format
GEOMS = [(2, 8, 256), (2, 10, 1024), (4, 9, 512), (4, 11, 2048), (2, 13, 8192),
         (8, 9, 512), (8, 13, 4096), (4, 13, 8192), (2, 12, 3000)]


@pytest.mark.parametrize("d,bits,K", GEOMS)
@pytest.mark.parametrize("cols,dead", [(256, 0), (192, 3), (64, 1)])
def test_gather_bit_exact(d, bits, K, cols, dead):
    """Random ids over all tables, repeats included; n spans several
    workgroups and ends in a partial one."""
    rows, E = 50, 4
    T = synth.make_tensor(41, d * 100 + bits, rows=rows, cols=cols, d=d, bits=bits, K=K,
                          n_experts=E, dead_rows=dead)
    W = vq.VQTensor.from_host(T)
    rng = np.random.default_rng(d * 1000 + bits + cols)
    n = 3000 + 37
    ids = rng.integers(0, E * rows, size=n).astype(np.int64)
    got = _gather(T, W, ids)
    ref = oracle.gather(T, ids)
    assert got.shape == (n, cols)
    assert _same_bits(got, ref)


def test_gather_bad_ids_nan_and_dead_rows_positive_zero():
    rows, E, cols = 16, 3, 128
    T = synth.make_tensor(42, 1, rows=rows, cols=cols, d=2, bits=8, n_experts=E, dead_rows=4)
    W = vq.VQTensor.from_host(T)
    dead = np.nonzero(T.row_map < 0)[0].astype(np.int64)
    ids = np.array([-1, E * rows, 0, np.iinfo(np.int64).max, np.iinfo(np.int64).min, 5,
                    *dead, 1 << 40], dtype=np.int64)
    got = _gather(T, W, ids)
    ref = oracle.gather(T, ids)
    bad = [0, 1, 3, 4, len(ids) - 1]
    assert np.isnan(got[bad]).all()
    live = [i for i in range(len(ids)) if i not in bad]
    assert _same_bits(got[live], ref[live])
    assert not got[6:6 + len(dead)].view(np.uint32).any()   # +0.0


def test_gather_all_rows_equal_dequantize():
    """Gathering every row of every table in order equals vq_dequantize of
    each table, concatenated (two GPU paths agree)."""
    rows, E, cols = 33, 5, 320
    T = synth.make_tensor(43, 1, rows=rows, cols=cols, d=4, bits=9, n_experts=E, dead_rows=2)
    W = vq.VQTensor.from_host(T)
    got = _gather(T, W, np.arange(E * rows))
    deq = torch.cat([vq.vq_dequantize(W, e) for e in range(E)]).cpu().numpy()
    assert _same_bits(got, deq)


def test_gather_small_and_empty():
    T = synth.make_tensor(44, 1, rows=8, cols=64, d=2, bits=8, n_experts=2)
    W = vq.VQTensor.from_host(T)
    for n in (1, 2, 15, 16, 17):
        ids = np.arange(n, dtype=np.int64) % 16
        assert _same_bits(_gather(T, W, ids), oracle.gather(T, ids))
    out = vq.vq_row_gather(W, torch.zeros(0, dtype=torch.int64, device="cuda"))
    assert out.shape == (0, 64)


def test_gather_all_rows_dead_table():
    """A tensor whose rows are all dead stores nothing (its code and scale
    pointers may point anywhere): the output is +0.0."""
    import ctypes
    T = synth.make_tensor(45, 1, rows=8, cols=128, d=2, bits=8, n_experts=2, dead_rows=8)
    assert T.n_stored == 0
    W = vq.VQTensor.from_host(T)
    cb = W.codebook.data_ptr()
    c = vq._CTensor(T.rows, T.cols, T.d, T.bits, T.K, T.n_experts, 0, cb, cb, cb,
                    W.row_map.data_ptr())
    ids = torch.arange(16, dtype=torch.int64, device="cuda")
    y = torch.full((16, 128), 3.0, device="cuda")
    st = vq.load_library().vq_row_gather(ctypes.byref(c), 16, ctypes.c_void_p(ids.data_ptr()),
                                         ctypes.c_void_p(y.data_ptr()), vq._stream())
    assert st == 0
    torch.cuda.synchronize()
    assert not y.cpu().numpy().view(np.uint32).any()


def test_gather_writes_only_its_rows():
    """Rows of a preallocated output beyond n are left alone."""
    T = synth.make_tensor(46, 1, rows=8, cols=256, d=2, bits=8)
    W = vq.VQTensor.from_host(T)
    out = torch.full((10, 256), 7.0, device="cuda")
    ids = torch.tensor([3, 1, 4, 1, 5], dtype=torch.int64, device="cuda")
    vq.vq_row_gather(W, ids, out=out[:5])
    torch.cuda.synchronize()
    assert bool((out[5:] == 7.0).all())
    assert _same_bits(out[:5].cpu().numpy(), oracle.gather(T, ids.cpu().numpy()))


def test_gather_graph_replay():
    """Captured in a HIP graph and replayed with eager calls in between, every
    replay equals the eager result bit for bit."""
    T = synth.make_tensor(47, 1, rows=64, cols=256, d=2, bits=8, n_experts=3)
    W = vq.VQTensor.from_host(T)
    ids = torch.from_numpy(np.random.default_rng(1).integers(0, 192, 500)).cuda()
    eager = vq.vq_row_gather(W, ids).clone()
    out = torch.empty_like(eager)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        vq.vq_row_gather(W, ids, out=out)
    for _ in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), eager.view(torch.int32))
        vq.vq_row_gather(W, torch.flip(ids, [0]))
        torch.cuda.synchronize()


def test_gather_full_size_sampled():
    """The measured workload (40 tables of 2^18 rows x 256 columns at d=2/K=256,
    4096 tokens x 40 lookups) in one launch, as timed; 2048 sampled output rows
    are checked against the oracle row by row."""
    wl = synth.GATHER_WORKLOADS["ple_gather_d2k256_tables40_rows262144_cols256_t4096"]
    T = synth.make_gather_table(wl)
    W = vq.VQTensor.from_host(T)
    ids = synth.make_gather_ids(wl, 0)
    y = vq.vq_row_gather(W, torch.from_numpy(ids).cuda())
    torch.cuda.synchronize()
    pick = np.sort(np.random.default_rng(2).choice(len(ids), 2048, replace=False))
    pick = np.concatenate([[0, len(ids) - 1], pick])
    got = y[torch.from_numpy(pick).cuda()].cpu().numpy()
    assert _same_bits(got, oracle.gather(T, ids[pick]))
    assert bool(torch.isfinite(y).all())


@pytest.mark.parametrize("d,bits,K,dead", [(4, 13, 8192, 5), (2, 8, 256, 0)])
def test_gather_large_batches(d, bits, K, dead):
    """Gathers large enough for eight chunks per thread, with a small
    codebook (queued grid) and a 64 KiB one (resident grid-stride launch):
    every row against the oracle."""
    rows, E, cols = 400, 8, 256
    T = synth.make_tensor(48, d * 100 + bits, rows=rows, cols=cols, d=d, bits=bits, K=K,
                          n_experts=E, dead_rows=dead)
    W = vq.VQTensor.from_host(T)
    n = 12011                                   # 768704 chunks of 4 columns
    ids = np.random.default_rng(bits).integers(-2, E * rows + 2, size=n).astype(np.int64)
    got = _gather(T, W, ids)
    ref = oracle.gather(T, ids)
    bad = (ids < 0) | (ids >= E * rows)
    assert np.isnan(got[bad]).all()
    assert _same_bits(got[~bad], ref[~bad])
