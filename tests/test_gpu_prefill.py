"""GPU parity of the many-token path: the grouped MFMA GEMM (one projection)
and the routed SwiGLU FFN for prefill batches, through the C ABI, against
the CPU oracle on the same seeded inputs.  Full-size workloads are checked on
sampled tokens (every token's output is independent of the others)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import vq_dequant_matmul_amd as vq
from parity import check_close, dead_rows, x_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    vq.load_library()


def _dev(T):
    return vq.VQTensor.from_host(T)


GEMM_CASES = [
    # d, bits, rows, cols, E, rows per expert (list), dtype, dead
    (4, 11, 704, 2816, 4, [130, 0, 77, 193], "bf16", 0),
    (4, 11, 2816, 704, 3, [64, 1, 150], "bf16", 0),        # 5.5 blocks per row
    (2, 8, 1024, 4096, 3, [80, 96, 33], "bf16", 127),      # skip-zero rows
    (4, 9, 200, 512, 2, [7, 300], "f32", 5),               # ragged rows and tiles
    (2, 10, 96, 1024, 5, [0, 0, 40, 0, 9], "bf16", 0),
    (8, 12, 64, 256, 2, [33, 31], "bf16", 0),
    (4, 13, 130, 384, 2, [17, 60], "bf16", 3),
    (2, 8, 300, 448, 3, [40, 100, 5], "bf16", 9),          # 8-bit, 7 groups a row
    (2, 8, 520, 256, 2, [64, 97], "f32", 3),               # 8-bit, 4 groups, ragged rows
    # 8-bit d2 blocks near 100 rows: 128-row tiles in the chunk-only LDS layout
    (2, 8, 600, 512, 4, [100, 128, 97, 33], "bf16", 11),
    (2, 8, 1024, 1024, 3, [120, 88, 101], "bf16", 0),
    (2, 8, 700, 768, 4, [128, 120, 7, 110], "bf16", 21),   # one-block tile among 128-row ones
    # the same block sizes with 7 groups a row: no chunks, 96-row tiles
    (2, 8, 300, 448, 4, [100, 128, 97, 33], "bf16", 0),
]


@pytest.mark.parametrize("d,bits,rows,cols,E,counts,dt,dead", GEMM_CASES)
def test_expert_gemm_parity(d, bits, rows, cols, E, counts, dt, dead):
    K = min(1 << bits, 8192 if d == 4 else (4096 if d == 8 else 1 << bits))
    T = synth.make_tensor(70, d * 100 + bits, rows=rows, cols=cols, d=d, bits=bits, K=K,
                          n_experts=E, dead_rows=dead)
    n = sum(counts)
    x = synth.make_x(70, 9, n, cols, dt)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    y = vq.vq_expert_gemm(_dev(T), x_to_torch(x), torch.from_numpy(offs).cuda()).cpu().numpy()
    for e in range(E):
        lo, hi = offs[e], offs[e + 1]
        if lo == hi:
            continue
        ref = oracle.linear(T, e, x[lo:hi])
        check_close(y[lo:hi], ref, f"gemm expert {e}")
        dz = dead_rows(T, e)
        assert np.all(y[lo:hi][:, dz].view(np.uint32) == 0), "dead rows must be +0.0"


def test_expert_gemm_deterministic():
    T = synth.make_tensor(71, 1, rows=512, cols=1024, d=4, bits=9, n_experts=2)
    x = x_to_torch(synth.make_x(71, 2, 300, 1024, "bf16"))
    offs = torch.tensor([0, 170, 300], dtype=torch.int32).cuda()
    W = _dev(T)
    a = vq.vq_expert_gemm(W, x, offs).cpu().numpy()
    b = vq.vq_expert_gemm(W, x, offs).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def _run_moe(gate, up, down, x, ids, w):
    y = vq.vq_moe_ffn(_dev(gate), _dev(up), _dev(down), x_to_torch(x),
                      torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda())
    return y.cpu().numpy()


@pytest.mark.parametrize("T,E,k,H,I,d,bits,dead,dt", [
    (17, 8, 2, 256, 192, 4, 9, 0, "bf16"),      # just above the decode batch limit
    (64, 8, 3, 512, 256, 2, 8, 5, "bf16"),      # skip-zero
    (200, 16, 4, 384, 320, 4, 11, 0, "f32"),    # fp32 activations
    (96, 4, 4, 256, 128, 2, 10, 0, "bf16"),     # every expert routed by every token
    (40, 64, 2, 256, 128, 8, 9, 0, "bf16"),     # mostly empty experts
    (50, 8, 2, 384, 256, 2, 8, 0, "bf16"),      # 8-bit: 6 groups (gate, up), 4 (down)
    (48, 8, 2, 256, 192, 4, 13, 2, "bf16"),     # 13-bit: gate, then up with SwiGLU
    (200, 16, 8, 512, 256, 2, 8, 7, "bf16"),    # 8-bit, ~100 rows an expert: 128-row tiles
])
def test_moe_prefill_small(T, E, k, H, I, d, bits, dead, dt):
    seed = 80 + T
    gate = synth.make_tensor(seed, 1, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead)
    up = synth.make_tensor(seed, 2, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead)
    down = synth.make_tensor(seed, 3, rows=H, cols=I, d=d, bits=bits, n_experts=E, dead_rows=dead)
    x = synth.make_x(seed, 4, T, H, dt)
    ids, w = synth.make_routes(seed, 5, T, E, k)
    y = _run_moe(gate, up, down, x, ids, w)
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), "moe prefill")


@pytest.mark.parametrize("name,n_sample", [
    ("moe_prefill_e128_h2816_i704_d4k2048_t2048", 6),
    ("moe_prefill_e512_h4096_i1024_d2k256_t4096_sz", 4),
])
def test_moe_prefill_full_size_sampled(name, n_sample):
    wl = synth.WORKLOADS[name]
    gate, up, down = synth.make_moe_layer(wl)
    x, ids, w = synth.make_moe_inputs(wl, 0)
    y = _run_moe(gate, up, down, x, ids, w)
    assert np.all(np.isfinite(y))
    rng = np.random.default_rng(5)
    tokens = np.sort(rng.choice(wl.n_tok, size=n_sample, replace=False)).astype(np.int32)
    ref = oracle.moe_ffn(gate, up, down, x, ids, w, tokens=tokens)
    check_close(y[tokens], ref, name)


def _cover_tokens(ids, E, experts, seed):
    """Every token routed to one of `experts` (each such expert's whole block
    of rows, so all of its M tiles), plus a greedy choice of further tokens
    until every routed expert is covered by at least one token."""
    sel = set(np.nonzero(np.isin(ids, list(experts)).any(axis=1))[0].tolist())
    covered = set(np.unique(ids[sorted(sel)]).tolist()) if sel else set()
    want = set(np.unique(ids).tolist())
    rng = np.random.default_rng(seed)
    for t in rng.permutation(ids.shape[0]):
        if covered >= want:
            break
        new = set(ids[t].tolist()) - covered
        if new:
            sel.add(int(t))
            covered |= new
    assert covered >= want
    return np.array(sorted(sel), dtype=np.int32)


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name", [
    "moe_prefill_e128_h2816_i704_d4k2048_t2048",
    "moe_prefill_e512_h4096_i1024_d2k256_t4096_sz",
])
def test_moe_prefill_full_size_tiles(name):
    """The full-size layers in the benchmarked launch configuration: all
    tokens of the largest, the smallest and a median expert block (every M
    tile of those experts, including remainder tiles), plus tokens covering
    every routed expert, against the oracle."""
    wl = synth.WORKLOADS[name]
    gate, up, down = synth.make_moe_layer(wl)
    x, ids, w = synth.make_moe_inputs(wl, 0)
    y = _run_moe(gate, up, down, x, ids, w)
    assert np.all(np.isfinite(y))
    counts = np.bincount(ids.ravel(), minlength=wl.n_experts)
    order = np.argsort(counts, kind="stable")
    live = order[counts[order] > 0]
    experts = {int(live[-1]), int(live[0]), int(live[len(live) // 2])}
    tokens = _cover_tokens(ids, wl.n_experts, experts, 7)
    ref = oracle.moe_ffn(gate, up, down, x, ids, w, tokens=tokens)
    check_close(y[tokens], ref, f"{name} ({len(tokens)} tokens)")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", [
    "moe_prefill_e128_h2816_i704_d4k2048_t2048",
    "moe_prefill_e512_h4096_i1024_d2k256_t4096_sz",
])
@pytest.mark.parametrize("proj", [0, 2])
def test_expert_gemm_full_size(name, proj):
    """vq_expert_gemm on a full-size projection with the workload's routed
    block sizes; the largest, smallest and a median block are checked."""
    wl = synth.WORKLOADS[name]
    T = synth.make_moe_layer(wl)[proj]
    _, ids, _ = synth.make_moe_inputs(wl, 0)
    counts = np.bincount(ids.ravel(), minlength=wl.n_experts)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    x = synth.make_x(wl.seed, 77 + proj, int(offs[-1]), T.cols, "bf16")
    y = vq.vq_expert_gemm(_dev(T), x_to_torch(x), torch.from_numpy(offs).cuda()).cpu().numpy()
    assert np.all(np.isfinite(y))
    order = np.argsort(counts, kind="stable")
    for e in {int(order[-1]), int(order[0]), int(order[len(order) // 2])}:
        lo, hi = offs[e], offs[e + 1]
        if lo == hi:
            continue
        check_close(y[lo:hi], oracle.linear(T, e, x[lo:hi]), f"{name} proj {proj} expert {e}")
        assert np.all(y[lo:hi][:, dead_rows(T, e)].view(np.uint32) == 0)


def test_moe_prefill_deterministic():
    E, k, H, I, T = 16, 4, 512, 256, 128
    gate = synth.make_tensor(90, 1, rows=I, cols=H, d=4, bits=9, n_experts=E)
    up = synth.make_tensor(90, 2, rows=I, cols=H, d=4, bits=9, n_experts=E)
    down = synth.make_tensor(90, 3, rows=H, cols=I, d=4, bits=9, n_experts=E)
    x = synth.make_x(90, 4, T, H, "bf16")
    ids, w = synth.make_routes(90, 5, T, E, k)
    a = _run_moe(gate, up, down, x, ids, w)
    b = _run_moe(gate, up, down, x, ids, w)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def _layer(seed, E, H, I, d, bits, dead=(0, 0, 0)):
    return (synth.make_tensor(seed, 1, rows=I, cols=H, d=d, bits=bits, n_experts=E,
                              dead_rows=dead[0]),
            synth.make_tensor(seed, 2, rows=I, cols=H, d=d, bits=bits, n_experts=E,
                              dead_rows=dead[1]),
            synth.make_tensor(seed, 3, rows=H, cols=I, d=d, bits=bits, n_experts=E,
                              dead_rows=dead[2]))


def test_moe_prefill_hot_experts_and_repeated_ids():
    """Every token routed to two of three hot experts out of 32 (several M
    tiles per hot expert while the tile size follows the mean load, the
    other 29 experts empty), and every seventh token names one expert in
    both slots."""
    T, E, k, H, I = 300, 32, 2, 256, 192
    gate, up, down = _layer(95, E, H, I, 4, 9)
    t = np.arange(T)
    ids = np.stack([t % 3, (t + 1) % 3], axis=1).astype(np.int32)
    ids[::7, 1] = ids[::7, 0]
    w = np.random.default_rng(96).random((T, k)).astype(np.float32)
    x = synth.make_x(95, 4, T, H, "bf16")
    y = _run_moe(gate, up, down, x, ids, w)
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), "hot experts")


def test_moe_prefill_top1():
    T, E, k, H, I = 300, 16, 1, 384, 256
    gate, up, down = _layer(97, E, H, I, 2, 10)
    x = synth.make_x(97, 4, T, H, "bf16")
    ids, w = synth.make_routes(97, 5, T, E, k)
    y = _run_moe(gate, up, down, x, ids, w)
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), "top-1")


class _NoStoredRows(vq.VQTensor):
    n_stored = property(lambda self: 0)


def _dev_all_dead(T):
    """An all-dead tensor stores nothing: the library gets non-null one-row
    placeholder arrays and n_stored = 0."""
    assert T.n_stored == 0
    T.codes = np.zeros((1, T.codes.shape[1]), np.uint32)
    T.scales = np.zeros((1, T.scales.shape[1]), np.uint16)
    D = _dev(T)
    return _NoStoredRows(D.rows, D.cols, D.d, D.bits, D.K, D.n_experts, D.codebook, D.codes,
                         D.scales, D.row_map)


@pytest.mark.parametrize("which", ["gate", "down"])
def test_moe_prefill_all_rows_dead(which):
    """A projection that stores no rows: with down dead every output is
    exactly +0.0; with gate dead, h = silu(0) * up is zero and so is y."""
    T, E, k, H, I = 64, 8, 2, 256, 128
    dead = (I, 0, 0) if which == "gate" else (0, 0, H)
    gate, up, down = _layer(98, E, H, I, 4, 9, dead)
    x = synth.make_x(98, 4, T, H, "bf16")
    ids, w = synth.make_routes(98, 5, T, E, k)
    ref = oracle.moe_ffn(gate, up, down, x, ids, w)
    G = _dev_all_dead(gate) if which == "gate" else _dev(gate)
    D = _dev_all_dead(down) if which == "down" else _dev(down)
    y = vq.vq_moe_ffn(G, _dev(up), D, x_to_torch(x), torch.from_numpy(ids).cuda(),
                      torch.from_numpy(w).cuda()).cpu().numpy()
    assert np.all(ref == 0) and np.all(y == 0)
    if which == "down":
        assert np.all(y.view(np.uint32) == 0)


def test_moe_prefill_down_magnitudes():
    """Down rows whose scales span 2^-16 .. 2^12 inside every 64-column
    chunk, and experts 2^10 apart: the down projection's fp16 outputs carry
    one exponent per (tile, 64 columns), so each chunk's large columns set
    it and each expert's tile has its own; the combined output still matches
    the oracle."""
    T, E, k, H, I = 160, 8, 2, 512, 256
    gate, up, down = _layer(99, E, H, I, 2, 8, (0, 0, 5))
    rng = np.random.default_rng(99)
    sc = down.scales.view(np.float16).astype(np.float64)
    row_exp = rng.integers(-16, 13, size=(sc.shape[0], 1))
    expert_of = np.repeat(np.arange(E), H)
    if down.row_map is not None:
        stored = down.row_map >= 0
        owner = np.empty(sc.shape[0], dtype=np.int64)
        owner[down.row_map[stored]] = expert_of[stored]
    else:
        owner = expert_of
    exp_shift = np.where(owner % 2 == 0, 0, -10)[:, None]
    down.scales = synth.to_half_bits(sc * np.exp2(row_exp + exp_shift))
    x = synth.make_x(99, 4, T, H, "bf16")
    ids, w = synth.make_routes(99, 5, T, E, k)
    y = _run_moe(gate, up, down, x, ids, w)
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), "down magnitudes")
