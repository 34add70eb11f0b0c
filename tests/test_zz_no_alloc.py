"""vq_moe_ffn_noalloc (the routed FFN with its workspace in the library's
static device array) against vq_moe_ffn with a caller workspace, through the
C ABI: two calls in a row, the second with a smaller input, each bit-equal to
vq_moe_ffn and within the parity bar of the oracle; and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import vq_dequant_matmul_amd as vq
from parity import check_close, x_to_torch

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    vq.load_library()


def _layer(seed, E, H, I, d, bits, dead):
    return [vq.VQTensor.from_host(t) for t in (
        synth.make_tensor(seed, 1, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead),
        synth.make_tensor(seed, 2, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead),
        synth.make_tensor(seed, 3, rows=H, cols=I, d=d, bits=bits, n_experts=E))], [
        synth.make_tensor(seed, 1, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead),
        synth.make_tensor(seed, 2, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead),
        synth.make_tensor(seed, 3, rows=H, cols=I, d=d, bits=bits, n_experts=E)]


@pytest.mark.parametrize("first,second", [
    ((96, 4), (5, 4)),       # MFMA path, then the decode engine
    ((16, 8), (1, 8)),       # decode engine twice
    ((200, 4), (40, 4)),     # MFMA path twice, smaller tiles the second time
])
def test_noalloc_matches_moe_ffn(first, second):
    E, H, I = 32, 1024, 512
    dev, host = _layer(400 + first[0], E, H, I, 4, 9, 7)
    for call, (n_tok, k) in enumerate((first, second)):
        assert vq.vq_moe_ffn_workspace_size(*dev, n_tok, k) <= SCRATCH
        x = synth.make_x(401, call, n_tok, H, "bf16")
        ids, w = synth.make_routes(402, call, n_tok, E, k)
        xt, it, wt = x_to_torch(x), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
        y_na = vq.vq_moe_ffn_noalloc(*dev, xt, it, wt)
        y_ws = vq.vq_moe_ffn(*dev, xt, it, wt)
        torch.cuda.synchronize()
        a, b = y_na.cpu().numpy(), y_ws.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"call {call}"
        check_close(a, oracle.moe_ffn(*host, x, ids, w), f"noalloc call {call}")


def test_noalloc_rejects_batches_beyond_the_array():
    E, H, I = 64, 4096, 1024
    dev, _ = _layer(410, E, H, I, 2, 8, 0)
    n_tok, k = 2048, 8
    assert vq.vq_moe_ffn_workspace_size(*dev, n_tok, k) > SCRATCH
    x = torch.zeros((n_tok, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros((n_tok, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((n_tok, k), dtype=torch.float32, device="cuda")
    with pytest.raises(vq.VQError, match="static scratch array"):
        vq.vq_moe_ffn_noalloc(*dev, x, ids, w)
