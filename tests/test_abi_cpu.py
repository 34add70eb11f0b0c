"""The C ABI without a GPU: the library loads, exports every entry point that
include/vq.h declares, and rejects bad host-visible arguments with the
documented status and a message naming the field.  Only host validation
runs here (the pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import vq_dequant_matmul_amd as vq
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "vq.h")


@pytest.fixture(scope="module")
def lib():
    return vq.load_library()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vq_[a-z_]+)\s*\(", src)))


def test_every_declared_function_is_exported(lib):
    names = _declared_functions()
    assert "vq_moe_ffn" in names and "vq_expert_gemv" in names and "vq_expert_gemm" in names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in vq.h but not exported"


def test_abi_version(lib):
    assert lib.vq_abi_version() == 1


FAKE = 0x10000  # never dereferenced: validation fails or succeeds on host values only


def _t(**kw):
    base = dict(rows=64, cols=128, d=4, bits=9, K=512, n_experts=2, n_stored=128,
                codebook=FAKE, codes=FAKE, scales=FAKE, row_map=None)
    base.update(kw)
    return vq._CTensor(base["rows"], base["cols"], base["d"], base["bits"], base["K"],
                       base["n_experts"], base["n_stored"], base["codebook"], base["codes"],
                       base["scales"], base["row_map"])


@pytest.mark.parametrize("kw,status,needle", [
    ({}, 0, ""),
    (dict(cols=100), 1, "cols"),
    (dict(cols=0), 1, "cols"),
    (dict(rows=0), 1, "rows"),
    (dict(d=3), 2, "d = 3"),
    (dict(bits=7, K=128), 2, "bits"),
    (dict(bits=14), 2, "bits"),
    (dict(K=513), 1, "K"),
    (dict(K=0), 1, "K"),
    (dict(d=8, bits=13, K=8192), 2, "codebook"),   # 128 KiB codebook > 64 KiB
    (dict(n_experts=0), 1, "n_experts"),
    (dict(codes=None), 1, "non-NULL"),
    (dict(n_stored=100), 1, "n_stored"),
    (dict(row_map=FAKE, n_stored=129), 1, "n_stored"),
    (dict(codebook=FAKE + 2), 1, "aligned"),
])
def test_validate(lib, kw, status, needle):
    t = _t(**kw)
    st = lib.vq_validate(ctypes.byref(t))
    assert st == status
    if status:
        assert needle in lib.vq_last_error().decode()
        assert lib.vq_status_string(st).decode().startswith("VQ_ERR_")


def test_validate_accepts_skipzero_and_k8192_d4(lib):
    assert lib.vq_validate(ctypes.byref(_t(row_map=FAKE, n_stored=100))) == 0
    assert lib.vq_validate(ctypes.byref(_t(bits=13, K=8192))) == 0


def test_gemv_argument_errors(lib):
    t = _t()
    st = lib.vq_expert_gemv(ctypes.byref(t), 5, 1, FAKE, 1, FAKE, None)
    assert st == 1 and "expert" in lib.vq_last_error().decode()
    st = lib.vq_expert_gemv(ctypes.byref(t), 0, 65, FAKE, 1, FAKE, None)
    assert st == 1 and "n_tokens" in lib.vq_last_error().decode()
    st = lib.vq_expert_gemv(ctypes.byref(t), 0, 1, FAKE, 7, FAKE, None)
    assert st == 1 and "x_dtype" in lib.vq_last_error().decode()
    st = lib.vq_expert_gemv(ctypes.byref(t), 0, 1, FAKE + 4, 1, FAKE, None)
    assert st == 1 and "x:" in lib.vq_last_error().decode()
    # zero tokens is a no-op
    assert lib.vq_expert_gemv(ctypes.byref(t), 0, 0, None, 1, None, None) == 0


def test_moe_ffn_shape_and_workspace_errors(lib):
    g = _t(rows=64, cols=128)
    u = _t(rows=64, cols=128)
    dn = _t(rows=128, cols=64, K=512, n_stored=256)
    ok = lib.vq_moe_ffn_workspace_size(ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), 2, 2)
    assert ok > 0
    bad_dn = _t(rows=64, cols=128)
    st = lib.vq_moe_ffn(ctypes.byref(g), ctypes.byref(u), ctypes.byref(bad_dn), 2, 2, FAKE, 1,
                        FAKE, FAKE, FAKE, FAKE, ok, None)
    assert st == 1 and "down" in lib.vq_last_error().decode()
    st = lib.vq_moe_ffn(ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), 2, 3, FAKE, 1,
                        FAKE, FAKE, FAKE, FAKE, ok, None)
    assert st == 1 and "top_k" in lib.vq_last_error().decode()
    st = lib.vq_moe_ffn(ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), 2, 2, FAKE, 1,
                        FAKE, FAKE, FAKE, FAKE, ok - 1, None)
    assert st == 3 and "workspace" in lib.vq_last_error().decode()
    u2 = _t(rows=64, cols=128, bits=10, K=1024)
    st = lib.vq_moe_ffn(ctypes.byref(g), ctypes.byref(u2), ctypes.byref(dn), 2, 2, FAKE, 1,
                        FAKE, FAKE, FAKE, FAKE, ok, None)
    assert st == 2 and "share d and bits" in lib.vq_last_error().decode()


def test_binding_refuses_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    with pytest.raises(RuntimeError, match="GPU"):
        vq._require_gpu()


def test_kernel_events_arguments(lib):
    assert lib.vq_set_kernel_events(None, None) == 0
    st = lib.vq_set_kernel_events(FAKE, None)
    assert st == 1 and "both" in lib.vq_last_error().decode()


def test_row_gather_argument_errors(lib):
    t = _t()
    st = lib.vq_row_gather(ctypes.byref(t), -1, FAKE, FAKE, None)
    assert st == 1 and "n = -1" in lib.vq_last_error().decode()
    st = lib.vq_row_gather(ctypes.byref(t), 4, FAKE + 4, FAKE, None)
    assert st == 1 and "ids" in lib.vq_last_error().decode()
    st = lib.vq_row_gather(ctypes.byref(t), 4, FAKE, FAKE + 8, None)
    assert st == 1 and "y:" in lib.vq_last_error().decode()
    st = lib.vq_row_gather(ctypes.byref(t), 4, None, FAKE, None)
    assert st == 1 and "ids" in lib.vq_last_error().decode()
    st = lib.vq_row_gather(ctypes.byref(_t(d=3)), 4, FAKE, FAKE, None)
    assert st == 2 and "d = 3" in lib.vq_last_error().decode()
    # zero rows is a no-op, whatever the pointers
    assert lib.vq_row_gather(ctypes.byref(t), 0, None, None, None) == 0


def test_fit_argument_errors(lib):
    assert lib.vq_fit_workspace_size(4, 512, 1000) >= 1000 * 16 + 512 * 16
    ws = lib.vq_fit_workspace_size(4, 512, 100)
    def call(**kw):
        a = dict(n_rows=8, cols=128, d=4, bits=9, K=512, w=FAKE, n_sample=100, sample=FAKE,
                 init=FAKE, iters=2, cb=FAKE, sc=FAKE, codes=FAKE, ws=FAKE, wsb=ws)
        a.update(kw)
        return lib.vq_fit(a["n_rows"], a["cols"], a["d"], a["bits"], a["K"], a["w"],
                          a["n_sample"], a["sample"], a["init"], a["iters"], a["cb"], a["sc"],
                          a["codes"], a["ws"], a["wsb"], None)
    for kw, status, needle in [
        (dict(n_rows=0), 1, "n_rows"), (dict(cols=100), 1, "cols"), (dict(d=3), 2, "d = 3"),
        (dict(bits=14), 2, "bits"), (dict(K=513), 1, "K = 513"),
        (dict(d=8, bits=13, K=4096), 2, "K*d"), (dict(n_sample=(1 << 22) + 1), 1, "n_sample"),
        (dict(iters=-1), 1, "iters"), (dict(w=FAKE + 8), 1, "w:"), (dict(init=None), 1, "init"),
        (dict(codes=FAKE + 2), 1, "codes"), (dict(wsb=ws - 1), 3, "workspace"),
    ]:
        st = call(**kw)
        assert st == status, (kw, st)
        assert needle in lib.vq_last_error().decode(), (kw, lib.vq_last_error())


def test_prefill_size_limits(lib):
    """The grouped-GEMM path indexes its activation matrices (x rows, then
    one h row per routed pair) in 32-bit bytes and counts routed pairs in
    int32: sizes past either limit are refused before any GPU work."""
    g = _t(rows=2048, cols=8192, n_experts=16, n_stored=16 * 2048)
    u = _t(rows=2048, cols=8192, n_experts=16, n_stored=16 * 2048)
    dn = _t(rows=8192, cols=2048, n_experts=16, n_stored=16 * 8192)
    # 131072 tokens x top-8 x inter 2048 fp16 = 4 GiB of h
    args = (ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn))
    assert lib.vq_moe_ffn_workspace_size(*args, 131072, 8) == 0
    st = lib.vq_moe_ffn(*args, 131072, 8, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == 2 and "limit" in lib.vq_last_error().decode()
    # just below: accepted by the size check (then the workspace check fails)
    assert lib.vq_moe_ffn_workspace_size(*args, 131071, 8) > 0
    st = lib.vq_moe_ffn(*args, 131071, 8, FAKE, 1, FAKE, FAKE, FAKE, FAKE, 1, None)
    assert st == 3 and "workspace" in lib.vq_last_error().decode()
    # x itself: 262144 rows x 8192 columns of fp16 = 4 GiB
    w = _t(rows=64, cols=8192, n_experts=2, n_stored=128)
    st = lib.vq_expert_gemm(ctypes.byref(w), 262144, FAKE, 1, FAKE, FAKE, FAKE, 1 << 40, None)
    assert st == 2 and "limit" in lib.vq_last_error().decode()


def test_noalloc_refuses_batches_beyond_its_array(lib):
    """vq_moe_ffn_noalloc takes its workspace from a 64 MiB static device
    array: a batch that needs more is refused before any GPU work."""
    g = _t(rows=1024, cols=4096, n_experts=64, n_stored=64 * 1024)
    u = _t(rows=1024, cols=4096, n_experts=64, n_stored=64 * 1024)
    dn = _t(rows=4096, cols=1024, n_experts=64, n_stored=64 * 4096)
    args = (ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn))
    assert lib.vq_moe_ffn_workspace_size(*args, 2048, 8) > 64 << 20
    st = lib.vq_moe_ffn_noalloc(*args, 2048, 8, FAKE, 1, FAKE, FAKE, FAKE, None)
    assert st == 2 and "static scratch array" in lib.vq_last_error().decode()
    # argument errors come first, as in vq_moe_ffn
    st = lib.vq_moe_ffn_noalloc(*args, 2048, 65, FAKE, 1, FAKE, FAKE, FAKE, None)
    assert st == 1 and "top_k" in lib.vq_last_error().decode()


def test_ffn_engine_choice(lib):
    """vq_moe_ffn_engine (host only): the decode kernels for up to 16 tokens,
    and past that for at most max(176, 3/4 of the experts) routed pairs with
    hidden and inter at most 8192; the grouped GEMM otherwise."""
    def engine(T, k, E, H=4096, I=1024):
        g = _t(rows=I, cols=H, n_experts=E, n_stored=E * I)
        u = _t(rows=I, cols=H, n_experts=E, n_stored=E * I)
        dn = _t(rows=H, cols=I, n_experts=E, n_stored=E * H)
        out = ctypes.c_int32(-1)
        st = lib.vq_moe_ffn_engine(ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), T, k,
                                   ctypes.byref(out))
        assert st == 0, lib.vq_last_error().decode()
        return out.value
    D, M = vq.VQ_ENGINE_DECODE, vq.VQ_ENGINE_MFMA
    assert engine(0, 8, 128) == D and engine(1, 10, 512) == D and engine(16, 10, 512) == D
    assert engine(16, 64, 64, H=1024, I=512) == D    # 1024 pairs: by token count
    assert engine(17, 10, 512) == D       # 170 pairs
    assert engine(38, 10, 512) == D       # 380 pairs (limit 384 at 512 experts)
    assert engine(39, 10, 512) == M       # 390 pairs
    assert engine(18, 10, 200) == M       # 180 pairs: 176 at 200 experts
    assert engine(22, 8, 128) == D        # 176 pairs
    assert engine(23, 8, 128) == M
    assert engine(17, 8, 128, H=16384) == M   # hidden past the decode kernels
    assert engine(2048, 8, 128) == M
    # bad arguments: vq_moe_ffn's checks
    g = _t(rows=1024, cols=4096, n_experts=8, n_stored=8 * 1024)
    out = ctypes.c_int32(-1)
    st = lib.vq_moe_ffn_engine(ctypes.byref(g), ctypes.byref(g), ctypes.byref(g), 4, 2,
                               ctypes.byref(out))
    assert st == 1 and "down" in lib.vq_last_error().decode()
