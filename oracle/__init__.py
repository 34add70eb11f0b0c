"""CPU oracle for the vector-quantized MoE expert matmul.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library.  The arithmetic lives in plain C
(``vq_oracle.c``, built with gcc); this module only marshals numpy arrays.

What is computed (model cards "Qwen3.5-397B-A17B-VQ-2.6bpw", sections
"Methodology" and "Sub-byte bit-packing"; "Qwen3.5-397B-A17B-VQ-2.4bpw: Model
Card", changelog 2026-10-01 "vq-skipzero"; "GLM-5.3-Flash-VQ-2.7bpw",
section "Methodology"): unpack b-bit codes from row-local uint32 streams,
decode W = scale * codebook[code] exactly in fp32, multiply with fp64
accumulation, and for the MoE FFN apply SwiGLU and the gate-weighted sum over
the routed experts in fp64.  ``gather`` reads single decoded rows, as the
per-layer n-gram embedding tables of "Qwen3.8-Flash-Next-VQ-4.4bpw" are read.
``fit`` (with ``fit_scales``, ``kmeans``, ``encode``) produces the format from
bf16 weights by k-means / Lloyd over the weight subvectors (the cards'
"Methodology" sections).

Tensor arguments are any object with the attributes ``rows, cols, d, bits, K,
n_experts, codebook (uint16 [K, d]), codes (uint32 [n_stored, wpr]), scales
(uint16 [n_stored, cols/64])`` and ``row_map`` (int32 [n_experts*rows] or
None).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "vq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

X_F32, X_BF16, X_F64 = 0, 1, 2
_ERRORS = {1: "bad argument", 2: "code >= K", 3: "bad row map", 4: "out of memory"}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP over independent output rows)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", "-fopenmp",
               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Tensor(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("d", ctypes.c_int32),
        ("bits", ctypes.c_int32), ("K", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("n_stored", ctypes.c_int64),
        ("codebook", ctypes.c_void_p), ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p), ("row_map", ctypes.c_void_p),
    ]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        lib.vqo_half_to_double.restype = ctypes.c_double
        lib.vqo_half_to_double.argtypes = [ctypes.c_uint16]
        lib.vqo_bf16_to_double.restype = ctypes.c_double
        lib.vqo_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.vqo_words_per_row.restype = ctypes.c_int64
        lib.vqo_words_per_row.argtypes = [ctypes.c_int32] * 3
        lib.vqo_code.restype = ctypes.c_uint32
        lib.vqo_code.argtypes = [P, ctypes.c_int32, ctypes.c_int64]
        lib.vqo_unpack_row.restype = None
        lib.vqo_unpack_row.argtypes = [P, ctypes.c_int32, ctypes.c_int64, P]
        lib.vqo_check.restype = ctypes.c_int
        lib.vqo_check.argtypes = [P]
        lib.vqo_decode.restype = ctypes.c_int
        lib.vqo_decode.argtypes = [P, ctypes.c_int32, P]
        lib.vqo_gather.restype = ctypes.c_int
        lib.vqo_gather.argtypes = [P, ctypes.c_int64, P, P]
        lib.vqo_linear.restype = ctypes.c_int
        lib.vqo_linear.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32, P]
        lib.vqo_moe_ffn.restype = ctypes.c_int
        lib.vqo_moe_ffn.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32,
                                    P, P, ctypes.c_int32, P, P]
        lib.vqo_moe_stack.restype = ctypes.c_int
        lib.vqo_moe_stack.argtypes = [ctypes.c_int32, P, P, P, ctypes.c_int32, ctypes.c_int32,
                                      P, P, P]
        I64, I32 = ctypes.c_int64, ctypes.c_int32
        lib.vqo_float_to_half.restype = ctypes.c_uint16
        lib.vqo_float_to_half.argtypes = [ctypes.c_float]
        lib.vqo_fit_scales.restype = ctypes.c_int
        lib.vqo_fit_scales.argtypes = [I64, I32, P, P]
        lib.vqo_kmeans.restype = ctypes.c_int
        lib.vqo_kmeans.argtypes = [I64, I32, I32, I32, P, P, I64, P, P, I32, P]
        lib.vqo_encode.restype = ctypes.c_int
        lib.vqo_encode.argtypes = [I64, I32, I32, I32, I32, P, P, P, P]
        lib.vqo_fit.restype = ctypes.c_int
        lib.vqo_fit.argtypes = [I64, I32, I32, I32, I32, P, I64, P, P, I32, P, P, P]
        lib.vqo_set_threads.restype = None
        lib.vqo_set_threads.argtypes = [ctypes.c_int32]
        lib.vqo_threads.restype = ctypes.c_int32
        lib.vqo_threads.argtypes = []
        lib.vqo_swiglu.restype = ctypes.c_double
        lib.vqo_swiglu.argtypes = [ctypes.c_double, ctypes.c_double]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class _Pinned:
    """Keeps the contiguous arrays alive while the C structure points at them."""

    def __init__(self, T):
        self.codebook = _c(T.codebook, np.uint16)
        self.codes = _c(T.codes, np.uint32)
        self.scales = _c(T.scales, np.uint16)
        self.row_map = _c(T.row_map, np.int32)
        n_stored = self.scales.shape[0] if self.scales.ndim == 2 else 0
        self.struct = _Tensor(T.rows, T.cols, T.d, T.bits, T.K, T.n_experts, n_stored,
                              _ptr(self.codebook), _ptr(self.codes), _ptr(self.scales),
                              _ptr(self.row_map))

    @property
    def ref(self):
        return ctypes.byref(self.struct)


def _raise(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def _x_arg(x):
    """Activations as raw bit patterns: float32 values, bf16 bit patterns in a
    uint16 array, or float64 values."""
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), X_F32
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), X_BF16
    if x.dtype == np.float64:
        return np.ascontiguousarray(x), X_F64
    raise TypeError("x must be float32, float64 or uint16 (bf16 bit patterns)")


def half_to_double(h: int) -> float:
    return _load().vqo_half_to_double(h)


def bf16_to_double(h: int) -> float:
    return _load().vqo_bf16_to_double(h)


def words_per_row(cols: int, d: int, bits: int) -> int:
    return _load().vqo_words_per_row(cols, d, bits)


def unpack_row(words: np.ndarray, bits: int, n: int) -> np.ndarray:
    words = np.ascontiguousarray(words, dtype=np.uint32)
    out = np.zeros(max(n, 1), dtype=np.uint32)
    _load().vqo_unpack_row(_ptr(words), bits, n, _ptr(out))
    return out[:n]


def check(T) -> None:
    p = _Pinned(T)
    _raise(_load().vqo_check(p.ref), "check")


def decode(T, expert: int) -> np.ndarray:
    """Dense fp32 weights [rows, cols] of one expert."""
    p = _Pinned(T)
    W = np.zeros((T.rows, T.cols), dtype=np.float32)
    _raise(_load().vqo_decode(p.ref, expert, _ptr(W)), "decode")
    return W


def gather(T, ids: np.ndarray) -> np.ndarray:
    """fp32 rows [n, cols]: row i is logical row ids[i] of the stacked tensor
    (id = expert*rows + r); dead rows zero, out-of-range ids NaN."""
    p = _Pinned(T)
    ids = np.ascontiguousarray(ids, dtype=np.int64).ravel()
    Y = np.zeros((len(ids), T.cols), dtype=np.float32)
    _raise(_load().vqo_gather(p.ref, len(ids), _ptr(ids) if len(ids) else None,
                              _ptr(Y) if len(ids) else None), "gather")
    return Y


def linear(T, expert: int, x: np.ndarray) -> np.ndarray:
    """fp64 y[n, r] = sum_c W[r, c] x[n, c] for x of shape [n_tok, cols]."""
    p = _Pinned(T)
    xa, dt = _x_arg(x)
    n_tok = xa.shape[0]
    y = np.zeros((n_tok, T.rows), dtype=np.float64)
    _raise(_load().vqo_linear(p.ref, expert, n_tok, _ptr(xa), dt, _ptr(y)), "linear")
    return y


def moe_ffn(gate, up, down, x: np.ndarray, ids: np.ndarray, weights: np.ndarray,
            tokens=None) -> np.ndarray:
    """fp64 routed SwiGLU FFN output for the selected tokens (all by default)."""
    pg, pu, pd = _Pinned(gate), _Pinned(up), _Pinned(down)
    xa, dt = _x_arg(x)
    n_tok = xa.shape[0]
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.ascontiguousarray(weights, dtype=np.float32)
    top_k = ids.shape[1]
    if tokens is None:
        tokens = np.arange(n_tok, dtype=np.int32)
    tokens = np.ascontiguousarray(tokens, dtype=np.int32)
    y = np.zeros((len(tokens), gate.cols), dtype=np.float64)
    rc = _load().vqo_moe_ffn(pg.ref, pu.ref, pd.ref, n_tok, top_k, _ptr(xa), dt,
                             _ptr(ids), _ptr(w), len(tokens), _ptr(tokens), _ptr(y))
    _raise(rc, "moe_ffn")
    return y


def moe_stack(layers, x: np.ndarray) -> np.ndarray:
    """fp64 hidden state after h <- h + FFN_l(h) over the layers (gate, up,
    down, ids, weights), starting from x [n_tok, hidden] (any float dtype)."""
    h = np.ascontiguousarray(x, dtype=np.float64).copy()
    n_tok = h.shape[0]
    L = len(layers)
    pins = [(_Pinned(g), _Pinned(u), _Pinned(d)) for g, u, d, _, _ in layers]
    ids = [np.ascontiguousarray(l[3], dtype=np.int32) for l in layers]
    ws = [np.ascontiguousarray(l[4], dtype=np.float32) for l in layers]
    top_k = ids[0].shape[1] if L else 1
    TP = ctypes.POINTER(_Tensor)
    arr = lambda k: (TP * max(L, 1))(*[ctypes.pointer(p[k].struct) for p in pins])
    ga, ua, da = arr(0), arr(1), arr(2)
    ia = (ctypes.c_void_p * max(L, 1))(*[a.ctypes.data for a in ids])
    wa = (ctypes.c_void_p * max(L, 1))(*[a.ctypes.data for a in ws])
    rc = _load().vqo_moe_stack(L, ctypes.cast(ga, ctypes.c_void_p), ctypes.cast(ua, ctypes.c_void_p),
                               ctypes.cast(da, ctypes.c_void_p), n_tok, top_k,
                               ctypes.cast(ia, ctypes.c_void_p), ctypes.cast(wa, ctypes.c_void_p),
                               _ptr(h))
    _raise(rc, "moe_stack")
    return h


# ---- fitting the format -------------------------------------------------

def float_to_half(f: float) -> int:
    """fp16 bits of an fp32 value, round to nearest even."""
    return int(_load().vqo_float_to_half(f))


def fit_scales(w: np.ndarray) -> np.ndarray:
    """fp16 bits [n_rows, cols/64]: max |w| per group, w bf16 bits [n_rows, cols]."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    sc = np.zeros((w.shape[0], w.shape[1] // 64), dtype=np.uint16)
    _raise(_load().vqo_fit_scales(w.shape[0], w.shape[1], _ptr(w), _ptr(sc)), "fit_scales")
    return sc


def kmeans(w: np.ndarray, scales: np.ndarray, d: int, K: int, sample, init,
           iters: int) -> np.ndarray:
    """fp32 centroids [K, d] after `iters` Lloyd iterations on the normalised
    subvectors named by `sample`, from those named by `init`."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    sample = np.ascontiguousarray(sample, dtype=np.int64)
    init = np.ascontiguousarray(init, dtype=np.int64)
    C = np.zeros((K, d), dtype=np.float32)
    rc = _load().vqo_kmeans(w.shape[0], w.shape[1], d, K, _ptr(w), _ptr(scales), len(sample),
                            _ptr(sample) if len(sample) else None, _ptr(init), iters, _ptr(C))
    _raise(rc, "kmeans")
    return C


def encode(w: np.ndarray, scales: np.ndarray, codebook: np.ndarray, d: int,
           bits: int) -> np.ndarray:
    """Packed codes [n_rows, wpr]: every subvector's nearest fp16 entry."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    cb = np.ascontiguousarray(codebook, dtype=np.uint16)
    codes = np.zeros((w.shape[0], words_per_row(w.shape[1], d, bits)), dtype=np.uint32)
    rc = _load().vqo_encode(w.shape[0], w.shape[1], d, bits, cb.shape[0], _ptr(w), _ptr(scales),
                            _ptr(cb), _ptr(codes))
    _raise(rc, "encode")
    return codes


def fit(w: np.ndarray, d: int, bits: int, K: int, sample, init, iters: int):
    """The whole fit: (codebook fp16 bits [K, d], scales fp16 bits
    [n_rows, cols/64], packed codes [n_rows, wpr])."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    sample = np.ascontiguousarray(sample, dtype=np.int64)
    init = np.ascontiguousarray(init, dtype=np.int64)
    n_rows, cols = w.shape
    cb = np.zeros((K, d), dtype=np.uint16)
    sc = np.zeros((n_rows, cols // 64), dtype=np.uint16)
    codes = np.zeros((n_rows, words_per_row(cols, d, bits)), dtype=np.uint32)
    rc = _load().vqo_fit(n_rows, cols, d, bits, K, _ptr(w), len(sample),
                         _ptr(sample) if len(sample) else None, _ptr(init), iters, _ptr(cb),
                         _ptr(sc), _ptr(codes))
    _raise(rc, "fit")
    return cb, sc, codes


def swiglu(g: float, u: float) -> float:
    return _load().vqo_swiglu(g, u)


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's row loops (timing only; results do
    not depend on it)."""
    _load().vqo_set_threads(int(n))


def threads() -> int:
    return int(_load().vqo_threads())
