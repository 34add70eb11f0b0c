"""GPU parity of the bandwidth-bound path: exact dequantisation, the
one-expert gemv, and the routed SwiGLU FFN for small batches, all through
the C ABI, against the CPU oracle on the same seeded inputs."""
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


# --------------------------------------------------------------------------
# exact dequantisation (bit-exact unpacking)
# --------------------------------------------------------------------------

DEQ_CASES = [
    (d, bits, K, cols, dead)
    for d, bits, K in [(2, 8, 256), (2, 10, 1024), (4, 9, 512), (4, 11, 2048), (4, 8, 256),
                       (2, 11, 2048), (8, 9, 512), (8, 13, 4096), (4, 13, 8192), (2, 12, 4096),
                       (8, 11, 2048), (8, 10, 1024)]
    for cols, dead in [(704, 0), (256, 3)]
]


@pytest.mark.parametrize("d,bits,K,cols,dead", DEQ_CASES)
def test_dequantize_bit_exact(d, bits, K, cols, dead):
    rows, E = 24, 3
    T = synth.make_tensor(31, d * 100 + bits, rows=rows, cols=cols, d=d, bits=bits, K=K,
                          n_experts=E, dead_rows=dead)
    W = _dev(T)
    for e in range(E):
        got = vq.vq_dequantize(W, e).cpu().numpy()
        ref = oracle.decode(T, e)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), f"expert {e}"


def test_dequantize_k_below_2b():
    T = synth.make_tensor(32, 1, rows=16, cols=128, d=4, bits=11, K=1500, n_experts=2)
    W = _dev(T)
    for e in range(2):
        assert np.array_equal(vq.vq_dequantize(W, e).cpu().numpy().view(np.uint32),
                              oracle.decode(T, e).view(np.uint32))


# --------------------------------------------------------------------------
# one expert, a few tokens
# --------------------------------------------------------------------------

def test_gemv_linear_256x512_fp32_one_token():
    """The single-linear workload: 256x512 at d=2/K=256, fp32 activations."""
    cfg = synth.LINEAR_256x512
    T = synth.make_tensor(cfg["seed"], 1, rows=cfg["rows"], cols=cfg["cols"], d=cfg["d"],
                          bits=cfg["bits"])
    x = synth.make_x(cfg["seed"], 2, 1, cfg["cols"], "f32")
    y = vq.vq_expert_gemv(_dev(T), 0, x_to_torch(x)).cpu().numpy()
    check_close(y, oracle.linear(T, 0, x), "linear 256x512")


GEMV_CASES = [
    # d, bits, rows, cols, n_tok, dtype, dead
    (2, 8, 256, 512, 1, "f32", 0),
    (2, 8, 96, 4096, 1, "bf16", 0),
    (4, 9, 100, 2048, 1, "bf16", 0),
    (4, 9, 77, 768, 3, "bf16", 5),
    (4, 11, 64, 704, 2, "bf16", 0),       # 5.5 blocks per row (padded)
    (4, 11, 40, 2816, 5, "f32", 4),        # 44 groups -> segment of 64 lanes
    (2, 10, 64, 1024, 8, "bf16", 0),
    (2, 10, 33, 4160, 1, "bf16", 0),       # 65 groups -> two groups per lane
    (2, 8, 20, 8192, 2, "f32", 2),         # 128 groups
    (8, 12, 50, 512, 4, "bf16", 0),
    (8, 9, 31, 1344, 16, "bf16", 3),
    (4, 12, 45, 192, 64, "bf16", 0),
    (2, 11, 17, 64, 7, "f32", 0),
]


@pytest.mark.parametrize("d,bits,rows,cols,n_tok,dt,dead", GEMV_CASES)
def test_gemv_parity(d, bits, rows, cols, n_tok, dt, dead):
    E = 2
    T = synth.make_tensor(41, d * 1000 + bits + cols, rows=rows, cols=cols, d=d, bits=bits,
                          n_experts=E, dead_rows=dead)
    x = synth.make_x(41, 7, n_tok, cols, dt)
    W = _dev(T)
    for e in range(E):
        y = vq.vq_expert_gemv(W, e, x_to_torch(x)).cpu().numpy()
        ref = oracle.linear(T, e, x)
        check_close(y, ref, f"gemv e={e}")
        dz = dead_rows(T, e)
        assert np.all(y[:, dz].view(np.uint32) == 0), "dead rows must be +0.0"


def test_gemv_deterministic():
    T = synth.make_tensor(42, 1, rows=512, cols=2048, d=4, bits=9, n_experts=1)
    x = x_to_torch(synth.make_x(42, 2, 3, 2048, "bf16"))
    W = _dev(T)
    a = vq.vq_expert_gemv(W, 0, x).cpu().numpy()
    b = vq.vq_expert_gemv(W, 0, x).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_gemv_large_activations_stay_finite():
    """Activations far outside fp16's range (bf16 allows them) still give the
    right answer: each 64-column block is range-scaled by a power of two."""
    T = synth.make_tensor(43, 1, rows=64, cols=512, d=2, bits=8)
    x = synth.make_x(43, 2, 2, 512, "f32") * np.float32(1e6)
    x[1, :64] *= np.float32(1e-12)
    y = vq.vq_expert_gemv(_dev(T), 0, x_to_torch(synth.to_bf16_bits(x))).cpu().numpy()
    check_close(y, oracle.linear(T, 0, synth.to_bf16_bits(x)), "large x")


# --------------------------------------------------------------------------
# routed SwiGLU FFN, decode batches
# --------------------------------------------------------------------------

def _moe_case(wl, n_experts=None, step=0):
    gate, up, down = synth.make_moe_layer(wl, n_experts=n_experts)
    x, ids, w = synth.make_moe_inputs(wl, step, n_experts=n_experts)
    return gate, up, down, x, ids, w


def _run_moe(gate, up, down, x, ids, w):
    G, U, D = _dev(gate), _dev(up), _dev(down)
    y = vq.vq_moe_ffn(G, U, D, x_to_torch(x), torch.from_numpy(ids).cuda(),
                      torch.from_numpy(w).cuda())
    return y.cpu().numpy()


@pytest.mark.parametrize("name", [
    "moe_decode_e128_h2048_i768_d4k512_b1",
    "moe_decode_e512_h4096_i1024_d2k256_b1",
    "moe_decode_e512_h4096_i1024_d2k256_b8",
    "moe_decode_e512_h4096_i1024_d2k1024_b1",
    "moe_decode_e512_h4096_i1024_d2k1024_b8",
])
def test_moe_decode_full_size(name):
    wl = synth.WORKLOADS[name]
    gate, up, down, x, ids, w = _moe_case(wl)
    y = _run_moe(gate, up, down, x, ids, w)
    ref = oracle.moe_ffn(gate, up, down, x, ids, w)
    check_close(y, ref, name)


@pytest.mark.parametrize("T,E,k,d,bits,dead", [
    (1, 4, 4, 2, 8, 0),       # every expert routed
    (16, 8, 3, 4, 9, 0),      # many tokens per expert
    (5, 16, 2, 4, 11, 7),     # skip-zero rows
    (3, 6, 2, 8, 10, 0),
])
def test_moe_decode_small(T, E, k, d, bits, dead):
    H, I = 256, 192
    wl = synth.MoEWorkload("small", E, k, H, I, d, bits, T, seed=50 + T)
    gate = synth.make_tensor(wl.seed, 1, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead)
    up = synth.make_tensor(wl.seed, 2, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead)
    down = synth.make_tensor(wl.seed, 3, rows=H, cols=I, d=d, bits=bits, n_experts=E, dead_rows=dead)
    x, ids, w = synth.make_moe_inputs(wl, 0)
    y = _run_moe(gate, up, down, x, ids, w)
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), "small moe")


@pytest.mark.parametrize("T,E,k,H,I", [
    (16, 64, 64, 128, 64),     # n_tokens * top_k = 1024, the routed-list maximum
    (2, 4, 2, 8192, 64),       # hidden 8192: 128 groups per row, the decode maximum
])
def test_moe_decode_maximum_sizes(T, E, k, H, I):
    wl = synth.MoEWorkload("max", E, k, H, I, 4, 9, T, seed=90 + T)
    gate = synth.make_tensor(wl.seed, 1, rows=I, cols=H, d=4, bits=9, n_experts=E, dead_rows=3)
    up = synth.make_tensor(wl.seed, 2, rows=I, cols=H, d=4, bits=9, n_experts=E)
    down = synth.make_tensor(wl.seed, 3, rows=H, cols=I, d=4, bits=9, n_experts=E, dead_rows=5)
    x, ids, w = synth.make_moe_inputs(wl, 0)
    y = _run_moe(gate, up, down, x, ids, w)
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), f"max T={T} k={k} H={H}")


# --------------------------------------------------------------------------
# batches past 16 tokens: the decode kernels up to max(176, 3/4 of the
# experts) routed pairs
# --------------------------------------------------------------------------

def _engine(gate, up, down, T, k):
    return vq.vq_moe_ffn_engine(_dev(gate), _dev(up), _dev(down), T, k)


@pytest.mark.parametrize("name,engine", [
    ("moe_batch_e512_h4096_i1024_d2k256_t17", vq.VQ_ENGINE_DECODE),   # 170 pairs
    ("moe_batch_e512_h4096_i1024_d2k256_t32", vq.VQ_ENGINE_DECODE),   # 320 pairs
    ("moe_batch_e512_h4096_i1024_d2k256_t64", vq.VQ_ENGINE_MFMA),
])
def test_moe_batch_full_size(name, engine):
    """17, 32 and 64 tokens on the 512-expert top-10 layer (0.3 to 1.25
    routed pairs per expert); every token is checked."""
    wl = synth.WORKLOADS[name]
    gate, up, down, x, ids, w = _moe_case(wl)
    assert _engine(gate, up, down, wl.n_tok, wl.top_k) == engine
    y = _run_moe(gate, up, down, x, ids, w)
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), name)


@pytest.mark.parametrize("E,T,engine", [
    (32, 44, vq.VQ_ENGINE_DECODE),     # 176 routed pairs
    (32, 45, vq.VQ_ENGINE_MFMA),       # 180
    (512, 96, vq.VQ_ENGINE_DECODE),    # 384 = 3/4 of the experts
    (512, 97, vq.VQ_ENGINE_MFMA),      # 388
])
def test_moe_batch_engine_boundary(E, T, engine):
    """Either side of the engine switch, at the fixed 176-pair limit and at
    the expert-count limit: same layer, both engines, both against the
    oracle."""
    k, H, I = 4, 256, 128
    wl = synth.MoEWorkload("boundary", E, k, H, I, 4, 9, T, seed=95)
    gate = synth.make_tensor(wl.seed, 1, rows=I, cols=H, d=4, bits=9, n_experts=E, dead_rows=2)
    up = synth.make_tensor(wl.seed, 2, rows=I, cols=H, d=4, bits=9, n_experts=E)
    down = synth.make_tensor(wl.seed, 3, rows=H, cols=I, d=4, bits=9, n_experts=E, dead_rows=4)
    x, ids, w = synth.make_moe_inputs(wl, 0)
    assert _engine(gate, up, down, T, k) == engine
    y = _run_moe(gate, up, down, x, ids, w)
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), f"T={T}")


def test_moe_decode_repeated_expert_in_token():
    """An id repeated within a token is served as two slots of one expert."""
    E, k, H, I = 4, 3, 128, 64
    gate = synth.make_tensor(60, 1, rows=I, cols=H, d=4, bits=9, n_experts=E)
    up = synth.make_tensor(60, 2, rows=I, cols=H, d=4, bits=9, n_experts=E)
    down = synth.make_tensor(60, 3, rows=H, cols=I, d=4, bits=9, n_experts=E)
    x = synth.make_x(60, 4, 2, H, "bf16")
    ids = np.array([[1, 1, 3], [0, 3, 3]], dtype=np.int32)
    w = np.array([[0.5, 0.25, 0.25], [0.2, 0.3, 0.5]], dtype=np.float32)
    y = _run_moe(gate, up, down, x, ids, w)
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), "repeated ids")


def test_moe_decode_deterministic():
    wl = synth.WORKLOADS["moe_decode_e128_h2048_i768_d4k512_b1"]
    gate, up, down, x, ids, w = _moe_case(wl, n_experts=16)
    ids = ids % 16
    a = _run_moe(gate, up, down, x, ids, w)
    b = _run_moe(gate, up, down, x, ids, w)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# --------------------------------------------------------------------------
# one token
# --------------------------------------------------------------------------

def _one_token_layer(E=16, H=2048, I=768, d=4, bits=9, dead=0, seed=70, down_bits=None):
    gate = synth.make_tensor(seed, 1, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead)
    up = synth.make_tensor(seed, 2, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead)
    down = synth.make_tensor(seed, 3, rows=H, cols=I, d=d, bits=down_bits or bits, n_experts=E,
                             dead_rows=dead)
    return gate, up, down


def test_moe_decode_one_token_workspace_reuse():
    """Consecutive one-token calls on one workspace: every output matches
    the oracle (nothing carries over from the previous call)."""
    E, k, H, I = 16, 8, 2048, 768
    gate, up, down = _one_token_layer(E, H, I)
    G, U, D = _dev(gate), _dev(up), _dev(down)
    wl = synth.MoEWorkload("one", E, k, H, I, 4, 9, 1, seed=71)
    ws = torch.empty(vq.vq_moe_ffn_workspace_size(G, U, D, 1, k), dtype=torch.uint8, device="cuda")
    for step in range(6):
        x, ids, w = synth.make_moe_inputs(wl, step)
        y = vq.vq_moe_ffn(G, U, D, x_to_torch(x), torch.from_numpy(ids).cuda(),
                          torch.from_numpy(w).cuda(), workspace=ws)
        check_close(y.cpu().numpy(), oracle.moe_ffn(gate, up, down, x, ids, w), f"step {step}")


@pytest.mark.parametrize("case", ["f32_x", "skip_zero", "repeated_id", "top1", "d2k1024_gpl2",
                                  "mixed_bits"])
def test_moe_decode_one_token_variants(case):
    E, k, H, I, d, bits, dead, down_bits, dt = 12, 4, 1024, 512, 4, 9, 0, None, "bf16"
    if case == "f32_x":
        dt = "f32"
    elif case == "skip_zero":
        dead = 40
    elif case == "top1":
        k = 1
    elif case == "d2k1024_gpl2":
        H, d, bits = 8192, 2, 10
    elif case == "mixed_bits":
        down_bits = 8
        d = 2
    gate, up, down = _one_token_layer(E, H, I, d, bits, dead, seed=80, down_bits=down_bits)
    x = synth.make_x(81, 5, 1, H, dt)
    rng = np.random.default_rng(82)
    ids = rng.choice(E, size=(1, k), replace=False).astype(np.int32)
    if case == "repeated_id":
        ids[0, 1] = ids[0, 0]
    w = rng.random((1, k)).astype(np.float32)
    y = _run_moe(gate, up, down, x, ids, w)
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), case)


def test_moe_decode_one_token_graph_replay():
    """One-token FFN calls captured in a HIP graph: every replay, with eager
    calls in between, gives the eager result bit for bit."""
    E, k, H, I = 16, 8, 1024, 512
    gate, up, down = _one_token_layer(E, H, I, seed=90)
    G, U, D = _dev(gate), _dev(up), _dev(down)
    wl = synth.MoEWorkload("one", E, k, H, I, 4, 9, 1, seed=91)
    ws = torch.empty(vq.vq_moe_ffn_workspace_size(G, U, D, 1, k), dtype=torch.uint8, device="cuda")
    steps = [synth.make_moe_inputs(wl, s) for s in range(3)]
    xs = [x_to_torch(x) for x, _, _ in steps]
    ids = [torch.from_numpy(i).cuda() for _, i, _ in steps]
    ws_ = [torch.from_numpy(w).cuda() for _, _, w in steps]
    outs = [torch.empty((1, H), dtype=torch.float32, device="cuda") for _ in steps]
    eager = []
    for s in range(3):
        vq.vq_moe_ffn(G, U, D, xs[s], ids[s], ws_[s], out=outs[s], workspace=ws)
        eager.append(outs[s].clone())
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for s in range(3):
            vq.vq_moe_ffn(G, U, D, xs[s], ids[s], ws_[s], out=outs[s], workspace=ws)
    for rep in range(3):
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for s in range(3):
            assert torch.equal(outs[s].view(torch.int32), eager[s].view(torch.int32)), (rep, s)
        # eager work between replays
        vq.vq_moe_ffn(G, U, D, xs[0], ids[0], ws_[0], workspace=ws)
        torch.cuda.synchronize()
