"""GPU parity of the invariants the format fixes, and of the three stage
calls of the small-batch FFN, through the C ABI against the CPU oracle.

- A one-entry codebook (K = 1, every code 0) and a codebook whose 256
  entries are all equal make every weight of a group the same vector times
  the group's scale (card "Qwen3.5-397B-A17B-VQ-2.6bpw", "Methodology": the
  weight is scale times the code's codebook vector), through the gemv, the
  grouped GEMM and both FFN paths.
- Skip-zero rows ("Qwen3.5-397B-A17B-VQ-2.4bpw: Model Card", changelog
  2026-10-01) output exact zeros, also inside the staged FFN: a row dead in
  gate or in up gives h = +0.0 bit for bit.
- Activations far below 1 (rows of magnitude 1e-35) keep their precision.
- Codes >= K read entry K-1 in the exact dequantisation, never past the
  codebook.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import vq_dequant_matmul_amd as vq
from parity import check_close, check_close_terms, dead_rows, x_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _setup():
    oracle.build(force=False)
    vq.load_library()


def _dev(T):
    return vq.VQTensor.from_host(T)


def _constant_codebook(T):
    """T with every codebook entry replaced by entry 0 (codes unchanged)."""
    T.codebook[:] = T.codebook[0][None, :]
    return T


def _tensor(kind, seed, stream, **kw):
    if kind == "k1":
        return synth.make_tensor(seed, stream, K=1, **kw)
    return _constant_codebook(synth.make_tensor(seed, stream, **kw))


KINDS = ["k1", "equal256"]


def _closed_form(T, e, x):
    """y[n][r] = sum_g s[r][g] * sum_{j in g} <c, x[n][j*d : j*d+d]> for a
    codebook whose entries all equal c (fp64, from the stored bits)."""
    c = T.codebook[0].view(np.float16).astype(np.float64)
    xf = x.astype(np.float64) if x.dtype != np.uint16 else \
        (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    n_tok, cols = xf.shape
    # per (token, group): sum over the group's subvectors of <c, x_j>
    xs = xf.reshape(n_tok, cols // 64, 64 // T.d, T.d) @ c
    xg = xs.sum(axis=2)                                   # [n_tok, groups]
    y = np.zeros((n_tok, T.rows))
    for r in range(T.rows):
        s = T.row_map[e * T.rows + r] if T.row_map is not None else e * T.rows + r
        if s < 0:
            continue
        sc = T.scales[s].view(np.float16).astype(np.float64)
        y[:, r] = xg @ sc
    return y


@pytest.mark.parametrize("kind", KINDS)
def test_constant_codebook_gemv(kind):
    T = _tensor(kind, 300, 1, rows=96, cols=512, d=2, bits=8, n_experts=2, dead_rows=7)
    x = synth.make_x(300, 2, 3, 512, "bf16")
    for e in range(2):
        y = vq.vq_expert_gemv(_dev(T), e, x_to_torch(x)).cpu().numpy()
        ref = oracle.linear(T, e, x)
        check_close(ref, _closed_form(T, e, x), f"{kind} oracle vs closed form")
        check_close(y, ref, f"{kind} gemv expert {e}")
        assert np.all(y[:, dead_rows(T, e)].view(np.uint32) == 0)


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("d,bits", [(2, 8), (4, 8)])
def test_constant_codebook_gemm(kind, d, bits):
    T = _tensor(kind, 301, d, rows=320, cols=1024, d=d, bits=bits, n_experts=3, dead_rows=9)
    counts = [70, 0, 150]
    x = synth.make_x(301, 4, sum(counts), 1024, "bf16")
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    y = vq.vq_expert_gemm(_dev(T), x_to_torch(x), torch.from_numpy(offs).cuda()).cpu().numpy()
    for e in range(3):
        lo, hi = offs[e], offs[e + 1]
        if lo == hi:
            continue
        check_close(y[lo:hi], oracle.linear(T, e, x[lo:hi]), f"{kind} gemm expert {e}")
        assert np.all(y[lo:hi][:, dead_rows(T, e)].view(np.uint32) == 0)


def _moe(kind, seed, E, H, I, d, bits, dead):
    gate = _tensor(kind, seed, 1, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead)
    up = _tensor(kind, seed, 2, rows=I, cols=H, d=d, bits=bits, n_experts=E, dead_rows=dead)
    down = _tensor(kind, seed, 3, rows=H, cols=I, d=d, bits=bits, n_experts=E, dead_rows=dead)
    return gate, up, down


def _ffn_terms(gate, up, down, x, ids, w):
    """Each token's FFN output with every product taken by magnitude:
    sum_s |w_s| |W_down| |h_s|, h_s from the oracle's projections (fp64)."""
    swiglu = np.vectorize(oracle.swiglu)
    dn = {}
    out = np.zeros((x.shape[0], gate.cols))
    for t in range(x.shape[0]):
        for s in range(ids.shape[1]):
            e = int(ids[t, s])
            if e not in dn:
                dn[e] = np.abs(oracle.decode(down, e).astype(np.float64))
            h = swiglu(oracle.linear(gate, e, x[t:t + 1])[0], oracle.linear(up, e, x[t:t + 1])[0])
            out[t] += abs(float(w[t, s])) * (dn[e] @ np.abs(h))
    return out


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("n_tok", [1, 5, 96])     # decode engine; MFMA path
def test_constant_codebook_moe_ffn(kind, n_tok):
    """The decode engine meets the per-token bar outright.  The MFMA path
    rounds each weight once to fp16 (scale times entry), and with one
    codebook vector that rounding repeats across the whole group instead of
    averaging out; on a token whose slot outputs cancel (||y|| near 3 % of
    its terms' size) the relative error then reaches ~3e-3, as a CPU
    emulation of that rounding gives too.  There the error is held to the
    bar relative to the size of the token's terms, and every token whose
    terms do not cancel to the plain per-token bar."""
    E, k, H, I = 16, 4, 512, 256
    gate, up, down = _moe(kind, 302 + n_tok, E, H, I, 2, 8, 5)
    x = synth.make_x(302, 4, n_tok, H, "bf16")
    ids, w = synth.make_routes(302, 5, n_tok, E, k)
    y = vq.vq_moe_ffn(_dev(gate), _dev(up), _dev(down), x_to_torch(x),
                      torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()).cpu().numpy()
    ref = oracle.moe_ffn(gate, up, down, x, ids, w)
    if n_tok <= 16:
        check_close(y, ref, f"{kind} moe ffn T={n_tok}")
    else:
        check_close_terms(y, ref, _ffn_terms(gate, up, down, x, ids, w),
                          f"{kind} moe ffn T={n_tok}")


# --------------------------------------------------------------------------
# the three stages of the small-batch FFN, one by one
# --------------------------------------------------------------------------

def _stage_layer(seed):
    E, H, I = 12, 768, 320
    # gate and up drop different rows, so h has rows dead in one of them only
    gate = synth.make_tensor(seed, 1, rows=I, cols=H, d=4, bits=9, n_experts=E, dead_rows=11)
    up = synth.make_tensor(seed, 2, rows=I, cols=H, d=4, bits=9, n_experts=E, dead_rows=13)
    down = synth.make_tensor(seed, 3, rows=H, cols=I, d=4, bits=9, n_experts=E, dead_rows=17)
    return gate, up, down


@pytest.mark.parametrize("n_tok,k", [(1, 4), (3, 6), (16, 8)])
def test_stage_gate_up(n_tok, k):
    gate, up, down = _stage_layer(310 + n_tok)
    x = synth.make_x(310, 4, n_tok, gate.cols, "bf16")
    ids, _ = synth.make_routes(310 + n_tok, 5, n_tok, gate.n_experts, k)
    h = vq.vq_moe_gate_up(_dev(gate), _dev(up), x_to_torch(x),
                          torch.from_numpy(ids).cuda()).cpu().numpy()
    assert h.shape == (n_tok * k, gate.rows)
    swiglu = np.vectorize(oracle.swiglu)
    for t in range(n_tok):
        for s in range(k):
            e = int(ids[t, s])
            q = t * k + s
            g = oracle.linear(gate, e, x[t:t + 1])[0]
            u = oracle.linear(up, e, x[t:t + 1])[0]
            check_close(h[q], swiglu(g, u), f"h pair {q}")
            dead = dead_rows(gate, e) | dead_rows(up, e)
            assert dead.any()
            assert np.all(h[q][dead].view(np.uint32) == 0), "h of a dead row must be +0.0"


@pytest.mark.parametrize("n_tok,k", [(1, 4), (2, 8), (16, 8)])
def test_stage_down(n_tok, k):
    gate, up, down = _stage_layer(320 + n_tok)
    ids, _ = synth.make_routes(320 + n_tok, 5, n_tok, down.n_experts, k)
    h = synth.make_x(320, 6, n_tok * k, down.cols, "f32")
    z = vq.vq_moe_down(_dev(down), torch.from_numpy(h).cuda(),
                       torch.from_numpy(ids).cuda()).cpu().numpy()
    for q in range(n_tok * k):
        e = int(ids.ravel()[q])
        check_close(z[q], oracle.linear(down, e, h[q:q + 1])[0], f"z pair {q}")
        assert np.all(z[q][dead_rows(down, e)].view(np.uint32) == 0)


@pytest.mark.parametrize("n_tok,k,hidden", [(1, 8, 2048), (7, 10, 4096), (16, 2, 64)])
def test_stage_combine(n_tok, k, hidden):
    rng = np.random.default_rng(330 + n_tok)
    z = rng.standard_normal((n_tok * k, hidden)).astype(np.float32)
    _, w = synth.make_routes(330, 5, n_tok, 64, k)
    zt, wt = torch.from_numpy(z).cuda(), torch.from_numpy(w).cuda()
    y = vq.vq_moe_combine(zt, wt).cpu().numpy()
    ref = np.einsum("ts,tsc->tc", w.astype(np.float64),
                    z.reshape(n_tok, k, hidden).astype(np.float64))
    check_close(y, ref, "combine")
    y2 = vq.vq_moe_combine(zt, wt).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_stages_compose_to_ffn():
    """gate_up -> down -> combine equals the oracle's whole FFN."""
    gate, up, down = _stage_layer(340)
    n_tok, k = 4, 6
    x = synth.make_x(340, 4, n_tok, gate.cols, "bf16")
    ids, w = synth.make_routes(340, 5, n_tok, gate.n_experts, k)
    idt = torch.from_numpy(ids).cuda()
    h = vq.vq_moe_gate_up(_dev(gate), _dev(up), x_to_torch(x), idt)
    z = vq.vq_moe_down(_dev(down), h, idt)
    y = vq.vq_moe_combine(z, torch.from_numpy(w).cuda()).cpu().numpy()
    check_close(y, oracle.moe_ffn(gate, up, down, x, ids, w), "staged ffn")


# --------------------------------------------------------------------------
# tiny activations and out-of-range codes
# --------------------------------------------------------------------------

@pytest.mark.parametrize("n_tok", [1, 3, 40])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_tiny_activations(n_tok, dt):
    """Rows of magnitude ~1e-35: the power-of-two range scaling stays finite
    and keeps the relative precision (decode engine and MFMA path)."""
    E, k, H, I = 8, 2, 512, 192
    gate = synth.make_tensor(350, 1, rows=I, cols=H, d=4, bits=9, n_experts=E)
    up = synth.make_tensor(350, 2, rows=I, cols=H, d=4, bits=9, n_experts=E)
    down = synth.make_tensor(350, 3, rows=H, cols=I, d=4, bits=9, n_experts=E)
    x32 = synth.make_x(350, 4, n_tok, H, "f32") * np.float32(1e-35)
    x = x32 if dt == "f32" else synth.to_bf16_bits(x32)
    y = vq.vq_expert_gemv(_dev(gate), 3, x_to_torch(x[:1])).cpu().numpy()
    check_close(y, oracle.linear(gate, 3, x[:1]), "tiny gemv")
    offs = np.array([0, n_tok] + [n_tok] * (E - 1), dtype=np.int32)
    y = vq.vq_expert_gemm(_dev(gate), x_to_torch(x), torch.from_numpy(offs).cuda()).cpu().numpy()
    check_close(y, oracle.linear(gate, 0, x), "tiny gemm")
    # the FFN's h is ~1e-70: below fp32, so h and y are exactly zero
    ids, w = synth.make_routes(350, 5, n_tok, E, k)
    y = vq.vq_moe_ffn(_dev(gate), _dev(up), _dev(down), x_to_torch(x),
                      torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()).cpu().numpy()
    assert np.all(np.isfinite(y))
    assert np.abs(oracle.moe_ffn(gate, up, down, x, ids, w)).max() < 1e-60
    assert np.all(y == 0.0)


@pytest.mark.parametrize("d,bits,K", [(2, 8, 200), (4, 9, 300), (4, 11, 1500)])
def test_dequantize_codes_at_least_k(d, bits, K):
    """Codes >= K (a precondition violation) read entry K-1: the output is
    the decode of the same codes clamped to K-1, bit for bit."""
    full = synth.make_tensor(360, bits, rows=24, cols=256, d=d, bits=bits, n_experts=2,
                             keep_codes=True)
    raw = full.raw_codes
    assert (raw >= K).any()
    bad = synth.VQTensorHost(full.rows, full.cols, d, bits, K, 2,
                             np.ascontiguousarray(full.codebook[:K]), full.codes,
                             full.scales, None)
    clamped = synth.VQTensorHost(full.rows, full.cols, d, bits, K, 2, bad.codebook,
                                 synth.pack_codes(np.minimum(raw, K - 1), bits), full.scales,
                                 None)
    W = _dev(bad)
    for e in range(2):
        got = vq.vq_dequantize(W, e).cpu().numpy()
        assert np.all(np.isfinite(got))
        ref = oracle.decode(clamped, e)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
