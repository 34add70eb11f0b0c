"""GPU parity of the MoE layer stack (decode through several MoE layers of
mixed geometry on a residual stream) through the C ABI, against the CPU
oracle on the same seeded inputs.  The tolerance applies to what the layers
add, h_L - x, per token."""
import numpy as np
import pytest
import torch

import oracle
import synth
import vq_dequant_matmul_amd as vq
from parity import check_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    vq.load_library()


def _host_layer(seed, d, bits, hidden, inter, E, top_k, n_tok, dead=0.0):
    wl = synth.MoEWorkload(f"s{seed}", E, top_k, hidden, inter, d, bits, n_tok, dead, seed)
    G, U, D = synth.make_moe_layer(wl)
    ids, w = synth.make_routes(seed, 7, n_tok, E, top_k)
    return (G, U, D, ids, w)


def _dev_layers(host):
    out = []
    for G, U, D, ids, w in host:
        out.append((vq.VQTensor.from_host(G), vq.VQTensor.from_host(U), vq.VQTensor.from_host(D),
                    torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()))
    return out


def _run(host, x):
    h = torch.from_numpy(np.ascontiguousarray(x, np.float32)).cuda()
    vq.vq_moe_stack(_dev_layers(host), h)
    torch.cuda.synchronize()
    return h.cpu().numpy()


# (d, bits) per layer: promoted layers in the middle, mixed d, skip-zero
STACKS = [
    ("glm_like", [(4, 9), (4, 11), (4, 9), (4, 11)], 0.0),
    ("flash_next_like", [(2, 10), (2, 8), (2, 8), (2, 10)], 0.1243),
    ("mixed_d", [(4, 9), (2, 8), (8, 10), (2, 11)], 0.05),
]


@pytest.mark.parametrize("name,geoms,dead", STACKS)
@pytest.mark.parametrize("n_tok", [1, 3, 8])
def test_stack_matches_oracle(name, geoms, dead, n_tok):
    hidden, inter, E, top_k = 512, 192, 16, 4
    host = [_host_layer(100 + 10 * i + n_tok, d, b, hidden, inter, E, top_k, n_tok, dead)
            for i, (d, b) in enumerate(geoms)]
    x = synth.make_x(5, n_tok, n_tok, hidden, "f32")
    got = _run(host, x)
    ref = oracle.moe_stack(host, x)
    check_close(got - x, ref - x, f"{name} n_tok={n_tok}")


@pytest.mark.parametrize("n_tok,top_k", [(1, 8), (16, 8)])
def test_one_layer_stack_is_x_plus_ffn(n_tok, top_k):
    """One layer equals x + vq_moe_ffn(x) bit for bit: the fused down+combine
    path (one token) and the down-then-combine path (16 tokens x 8 slots do
    not fit the fused kernel's LDS) both add the same sums to x."""
    host = [_host_layer(130 + n_tok, 4, 9, 1024, 768, 32, top_k, n_tok)]
    x = synth.make_x(6, n_tok, n_tok, 1024, "f32")
    got = _run(host, x)
    (G, U, D, ids, w), = _dev_layers(host)
    y = vq.vq_moe_ffn(G, U, D, torch.from_numpy(x).cuda(), ids, w)
    want = (torch.from_numpy(x).cuda() + y).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_dead_down_layer_leaves_state_unchanged():
    """A layer whose down projection stores no rows adds nothing: the state
    is bit-identical to the stack without it."""
    n_tok, hidden, inter, E, top_k = 2, 256, 128, 8, 2
    A = _host_layer(140, 4, 9, hidden, inter, E, top_k, n_tok)
    B = _host_layer(141, 2, 8, hidden, inter, E, top_k, n_tok)
    Z = _host_layer(142, 4, 11, hidden, inter, E, top_k, n_tok)
    Zd = synth.make_tensor(142, 3, rows=hidden, cols=inter, d=4, bits=11, n_experts=E,
                           dead_rows=hidden)
    assert Zd.n_stored == 0
    x = synth.make_x(7, 1, n_tok, hidden, "f32")
    # an all-dead tensor stores nothing: hand the library non-null placeholder
    # arrays of one row and report n_stored = 0
    Zd.codes = np.zeros((1, Zd.codes.shape[1]), np.uint32)
    Zd.scales = np.zeros((1, Zd.scales.shape[1]), np.uint16)

    class _NoStoredRows(vq.VQTensor):
        n_stored = property(lambda self: 0)

    dev = _dev_layers([A, (Z[0], Z[1], Zd, Z[3], Z[4]), B])
    D = dev[1][2]
    dev[1] = (dev[1][0], dev[1][1], _NoStoredRows(D.rows, D.cols, D.d, D.bits, D.K, D.n_experts,
                                                  D.codebook, D.codes, D.scales, D.row_map),
              dev[1][3], dev[1][4])
    h1 = torch.from_numpy(x).cuda()
    vq.vq_moe_stack(dev, h1)
    h2 = torch.from_numpy(x).cuda()
    vq.vq_moe_stack([dev[0], dev[2]], h2)
    torch.cuda.synchronize()
    assert torch.equal(h1.view(torch.int32), h2.view(torch.int32))


def test_stack_graph_replay():
    n_tok, hidden, inter, E, top_k = 1, 512, 192, 16, 4
    host = [_host_layer(150 + i, 4, b, hidden, inter, E, top_k, n_tok)
            for i, b in enumerate([9, 11, 9])]
    dev = _dev_layers(host)
    x = torch.from_numpy(synth.make_x(8, 1, n_tok, hidden, "f32")).cuda()
    h = x.clone()
    vq.vq_moe_stack(dev, h)
    eager = h.clone()
    ws = torch.empty(vq.vq_moe_stack_workspace_size(dev, n_tok, top_k), dtype=torch.uint8,
                     device="cuda")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.copy_(x)
        vq.vq_moe_stack(dev, h, workspace=ws)
    for _ in range(3):
        h.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int32), eager.view(torch.int32))
        vq.vq_moe_stack(dev, x.clone())          # eager work between replays
        torch.cuda.synchronize()


def test_stack_errors():
    host = [_host_layer(160, 4, 9, 256, 128, 8, 2, 1), _host_layer(161, 4, 9, 512, 128, 8, 2, 1)]
    dev = _dev_layers(host)
    h = torch.zeros((1, 256), device="cuda")
    with pytest.raises(vq.VQError, match="layer 1: hidden size"):
        vq.vq_moe_stack(dev, h)
    with pytest.raises(vq.VQError, match="tokens"):
        vq.vq_moe_stack(dev[:1], torch.zeros((17, 256), device="cuda"))


@pytest.mark.parametrize("name", ["moe_stack42_e128_h2048_i768_d4k512_p8k2048_b1"])
def test_full_size_stack(name):
    """The 42-layer stack of the measured workload (one token, eight
    promoted 11-bit layers), against the oracle."""
    sw = synth.STACK_WORKLOADS[name]
    host = {}
    for l in range(sw.n_layers):
        bits = sw.layer_bits(l)
        if bits not in host:
            host[bits] = synth.make_stack_layer(sw, l)
    devt = {bits: [vq.VQTensor.from_host(t) for t in host[bits]] for bits in host}
    x, ids, w = synth.make_stack_inputs(sw, 0)
    dev = [(*devt[sw.layer_bits(l)], torch.from_numpy(ids[l]).cuda(),
            torch.from_numpy(w[l]).cuda()) for l in range(sw.n_layers)]
    h = torch.from_numpy(x).cuda()
    vq.vq_moe_stack(dev, h)
    torch.cuda.synchronize()
    got = h.cpu().numpy()
    ref = oracle.moe_stack([(*host[sw.layer_bits(l)], ids[l], w[l])
                            for l in range(sw.n_layers)], x)
    check_close(got - x, ref - x, name)
