"""Python binding of the VQ MoE expert matmul library (MI355X / gfx950).

Thin ctypes layer over the C ABI in ``include/vq.h``: it marshals torch
device tensors into ``vq_tensor`` descriptors and raw pointers, passes the
current HIP stream, allocates outputs and workspaces with torch, and raises
``VQError`` on a non-zero status.  Every step of the computation runs in the
HIP kernels of ``libvqmm.so``; there is no CPU or PyTorch fallback, and
loading fails loudly when the library is missing or no GPU is present.

Names follow the C ABI: ``vq_dequantize``, ``vq_row_gather``, ``vq_expert_gemv``,
``vq_expert_gemm``, ``vq_moe_ffn`` and their workspace-size queries.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libvqmm.so")

VQ_OK, VQ_ERR_INVALID_ARGUMENT, VQ_ERR_UNSUPPORTED, VQ_ERR_WORKSPACE, VQ_ERR_HIP = range(5)
VQ_F32, VQ_BF16 = 0, 1


class VQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class _CTensor(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32), ("cols", ctypes.c_int32), ("d", ctypes.c_int32),
        ("bits", ctypes.c_int32), ("K", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("n_stored", ctypes.c_int64),
        ("codebook", ctypes.c_void_p), ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p), ("row_map", ctypes.c_void_p),
    ]


class _CLayer(ctypes.Structure):
    _fields_ = [
        ("gate", ctypes.POINTER(_CTensor)), ("up", ctypes.POINTER(_CTensor)),
        ("down", ctypes.POINTER(_CTensor)),
        ("topk_ids", ctypes.c_void_p), ("topk_weights", ctypes.c_void_p),
    ]


_lib = None


def build() -> str:
    """Compile libvqmm.so for gfx950 with hipcc (in-tree)."""
    from . import _build
    return _build.build()


def load_library():
    """Load libvqmm.so (building it first only if it does not exist)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    T = ctypes.POINTER(_CTensor)
    sigs = {
        "vq_abi_version": (I32, []),
        "vq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "vq_last_error": (ctypes.c_char_p, []),
        "vq_validate": (ctypes.c_int, [T]),
        "vq_dequantize": (ctypes.c_int, [T, I32, P, P]),
        "vq_row_gather": (ctypes.c_int, [T, I64, P, P, P]),
        "vq_fit_workspace_size": (SZ, [I32, I32, I64]),
        "vq_fit": (ctypes.c_int, [I64, I32, I32, I32, I32, P, I64, P, P, I32, P, P, P, P, SZ, P]),
        "vq_expert_gemv": (ctypes.c_int, [T, I32, I32, P, ctypes.c_int, P, P]),
        "vq_expert_gemm_workspace_size": (SZ, [T, I32]),
        "vq_expert_gemm": (ctypes.c_int, [T, I32, P, ctypes.c_int, P, P, P, SZ, P]),
        "vq_moe_ffn_workspace_size": (SZ, [T, T, T, I32, I32]),
        "vq_moe_ffn_engine": (ctypes.c_int, [T, T, T, I32, I32, P]),
        "vq_probe_read": (ctypes.c_int, [P, SZ, I32, P, P]),
        "vq_probe_mfma": (ctypes.c_int, [I32, I32, P, P]),
        "vq_moe_ffn": (ctypes.c_int, [T, T, T, I32, I32, P, ctypes.c_int, P, P, P, P, SZ, P]),
        "vq_moe_ffn_noalloc": (ctypes.c_int, [T, T, T, I32, I32, P, ctypes.c_int, P, P, P, P]),
        "vq_moe_gate_up": (ctypes.c_int, [T, T, I32, I32, P, ctypes.c_int, P, P, P]),
        "vq_moe_down": (ctypes.c_int, [T, I32, I32, P, P, P, P]),
        "vq_moe_combine": (ctypes.c_int, [I32, I32, I32, P, P, P, P]),
        "vq_set_kernel_events": (ctypes.c_int, [P, P]),
        "vq_moe_stack_workspace_size": (SZ, [ctypes.POINTER(_CLayer), I32, I32, I32]),
        "vq_moe_stack": (ctypes.c_int, [ctypes.POINTER(_CLayer), I32, I32, I32, P, P, SZ, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    names = {0: "VQ_OK", 1: "VQ_ERR_INVALID_ARGUMENT", 2: "VQ_ERR_UNSUPPORTED",
             3: "VQ_ERR_WORKSPACE", 4: "VQ_ERR_HIP"}
    return names.get(status, f"status {status}")


def _check(status: int):
    if status != VQ_OK:
        msg = load_library().vq_last_error().decode()
        raise VQError(status, msg)


def _require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("vq_dequant_matmul_amd needs a ROCm GPU (gfx950); none is visible")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


@dataclass
class VQTensor:
    """One VQ linear tensor stacked over experts, resident on the GPU.

    codebook: int16 [K, d] (fp16 bit patterns); codes: int32 [n_stored, wpr]
    (uint32 words); scales: int16 [n_stored, cols // 64] (fp16 bit patterns);
    row_map: int32 [n_experts * rows] (stored row or -1) or None (dense).
    """

    rows: int
    cols: int
    d: int
    bits: int
    K: int
    n_experts: int
    codebook: torch.Tensor
    codes: torch.Tensor
    scales: torch.Tensor
    row_map: Optional[torch.Tensor] = None

    @property
    def n_stored(self) -> int:
        return int(self.scales.shape[0])

    @classmethod
    def from_arrays(cls, *, rows, cols, d, bits, K, n_experts, codebook, codes, scales,
                    row_map=None, device="cuda"):
        """Upload numpy arrays (uint16 codebook/scales, uint32 codes, int32
        row map) to the device."""
        import numpy as np

        def up(a, dt):
            return torch.from_numpy(np.ascontiguousarray(a).view(dt)).to(device)
        return cls(rows, cols, d, bits, K, n_experts,
                   up(codebook, np.int16), up(codes, np.int32), up(scales, np.int16),
                   None if row_map is None else up(row_map, np.int32))

    @classmethod
    def from_host(cls, h, device="cuda"):
        """From any host object with the same attribute names (numpy arrays)."""
        return cls.from_arrays(rows=h.rows, cols=h.cols, d=h.d, bits=h.bits, K=h.K,
                               n_experts=h.n_experts, codebook=h.codebook, codes=h.codes,
                               scales=h.scales, row_map=h.row_map, device=device)

    def clone(self) -> "VQTensor":
        """A copy at new device addresses (same contents)."""
        return VQTensor(self.rows, self.cols, self.d, self.bits, self.K, self.n_experts,
                        self.codebook.clone(), self.codes.clone(), self.scales.clone(),
                        None if self.row_map is None else self.row_map.clone())

    def c(self) -> _CTensor:
        for t in (self.codebook, self.codes, self.scales, self.row_map):
            if t is not None and (not t.is_cuda or not t.is_contiguous()):
                raise ValueError("VQTensor arrays must be contiguous device tensors")
        return _CTensor(self.rows, self.cols, self.d, self.bits, self.K, self.n_experts,
                        self.n_stored, self.codebook.data_ptr(), self.codes.data_ptr(),
                        self.scales.data_ptr(),
                        None if self.row_map is None else self.row_map.data_ptr())

    def stored_bytes(self) -> int:
        n = self.codes.numel() * 4 + self.scales.numel() * 2
        if self.row_map is not None:
            n += self.row_map.numel() * 4
        return n


def _x_dtype(x: torch.Tensor) -> int:
    if x.dtype == torch.float32:
        return VQ_F32
    if x.dtype == torch.bfloat16:
        return VQ_BF16
    raise TypeError("activations must be float32 or bfloat16")


def vq_validate(W: VQTensor) -> None:
    c = W.c()
    _check(load_library().vq_validate(ctypes.byref(c)))


def vq_dequantize(W: VQTensor, expert: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _require_gpu()
    lib = load_library()
    if out is None:
        out = torch.empty((W.rows, W.cols), dtype=torch.float32, device=W.codes.device)
    c = W.c()
    _check(lib.vq_dequantize(ctypes.byref(c), expert, _ptr(out), _stream()))
    return out


def vq_row_gather(W: VQTensor, ids: torch.Tensor,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rows ids[i] = e*rows + r of the stacked tensor, decoded to fp32
    [n, cols]; dead rows +0.0, out-of-range ids NaN rows."""
    _require_gpu()
    lib = load_library()
    if ids.dtype != torch.int64 or not ids.is_cuda:
        raise TypeError("ids must be an int64 device tensor")
    ids = ids.contiguous().view(-1)
    n = ids.numel()
    if out is None:
        out = torch.empty((n, W.cols), dtype=torch.float32, device=ids.device)
    c = W.c()
    _check(lib.vq_row_gather(ctypes.byref(c), n, _ptr(ids), _ptr(out), _stream()))
    return out


def vq_fit(w: torch.Tensor, d: int, bits: int, K: int, sample: torch.Tensor,
           init: torch.Tensor, iters: int, workspace: Optional[torch.Tensor] = None):
    """Fit the format to bf16 weights w [n_rows, cols]: returns (codebook
    int16 [K, d] fp16 bits, scales int16 [n_rows, cols/64] fp16 bits, codes
    int32 [n_rows, wpr]), a dense tensor's arrays (see vq.h, vq_fit)."""
    _require_gpu()
    lib = load_library()
    if w.dtype != torch.bfloat16 or w.dim() != 2 or not w.is_contiguous():
        raise TypeError("w must be a contiguous 2-D bfloat16 device tensor")
    for name, t in (("sample", sample), ("init", init)):
        if t.dtype != torch.int64 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous int64 device tensor")
    n_rows, cols = w.shape
    wpr = ((cols // d + 31) // 32) * bits
    dev = w.device
    codebook = torch.empty((K, d), dtype=torch.int16, device=dev)
    scales = torch.empty((n_rows, cols // 64), dtype=torch.int16, device=dev)
    codes = torch.empty((n_rows, wpr), dtype=torch.int32, device=dev)
    if workspace is None:
        ws = lib.vq_fit_workspace_size(d, K, sample.numel())
        workspace = torch.empty(max(int(ws), 256), dtype=torch.uint8, device=dev)
    _check(lib.vq_fit(n_rows, cols, d, bits, K, _ptr(w), sample.numel(), _ptr(sample),
                      _ptr(init), iters, _ptr(codebook), _ptr(scales), _ptr(codes),
                      _ptr(workspace), workspace.numel(), _stream()))
    return codebook, scales, codes


def vq_expert_gemv(W: VQTensor, expert: int, x: torch.Tensor,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _require_gpu()
    lib = load_library()
    x = x.contiguous()
    n = x.shape[0]
    if out is None:
        out = torch.empty((n, W.rows), dtype=torch.float32, device=x.device)
    c = W.c()
    _check(lib.vq_expert_gemv(ctypes.byref(c), expert, n, _ptr(x), _x_dtype(x), _ptr(out),
                              _stream()))
    return out


def vq_expert_gemm_workspace_size(W: VQTensor, n_x_rows: int) -> int:
    c = W.c()
    return int(load_library().vq_expert_gemm_workspace_size(ctypes.byref(c), n_x_rows))


def vq_expert_gemm(W: VQTensor, x: torch.Tensor, expert_offsets: torch.Tensor,
                   out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    _require_gpu()
    lib = load_library()
    x = x.contiguous()
    n = x.shape[0]
    if out is None:
        out = torch.empty((n, W.rows), dtype=torch.float32, device=x.device)
    ws_bytes = vq_expert_gemm_workspace_size(W, n)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=x.device)
    c = W.c()
    _check(lib.vq_expert_gemm(ctypes.byref(c), n, _ptr(x), _x_dtype(x),
                              _ptr(expert_offsets.contiguous()), _ptr(out), _ptr(workspace),
                              0 if workspace is None else workspace.numel(), _stream()))
    return out


def vq_moe_ffn_workspace_size(gate: VQTensor, up: VQTensor, down: VQTensor, n_tokens: int,
                              top_k: int) -> int:
    g, u, d = gate.c(), up.c(), down.c()
    return int(load_library().vq_moe_ffn_workspace_size(ctypes.byref(g), ctypes.byref(u),
                                                        ctypes.byref(d), n_tokens, top_k))


VQ_ENGINE_DECODE = 0
VQ_ENGINE_MFMA = 1


def vq_moe_ffn_engine(gate: VQTensor, up: VQTensor, down: VQTensor, n_tokens: int,
                      top_k: int) -> int:
    """VQ_ENGINE_DECODE or VQ_ENGINE_MFMA: the engine vq_moe_ffn runs for
    this batch (host only)."""
    g, u, d = gate.c(), up.c(), down.c()
    eng = ctypes.c_int32(-1)
    _check(load_library().vq_moe_ffn_engine(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                            n_tokens, top_k, ctypes.byref(eng)))
    return int(eng.value)


def vq_probe_read(buf: torch.Tensor, n_workgroups: int, out: torch.Tensor) -> None:
    """Streaming-read ceiling probe over buf (device, any dtype); out: device
    uint32/int32 of n_workgroups*256 entries."""
    _check(load_library().vq_probe_read(_ptr(buf), buf.numel() * buf.element_size(),
                                        n_workgroups, _ptr(out), _stream()))


def vq_probe_mfma(n_workgroups: int, iters: int, out: torch.Tensor) -> None:
    """MFMA-only ceiling probe: iters x 4 v_mfma_f32_32x32x16_f16 per wave;
    out: device fp32 of n_workgroups*256 entries."""
    _check(load_library().vq_probe_mfma(n_workgroups, iters, _ptr(out), _stream()))


def vq_moe_ffn(gate: VQTensor, up: VQTensor, down: VQTensor, x: torch.Tensor,
               topk_ids: torch.Tensor, topk_weights: torch.Tensor,
               out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    _require_gpu()
    lib = load_library()
    x = x.contiguous()
    n, k = topk_ids.shape
    if out is None:
        out = torch.empty((n, gate.cols), dtype=torch.float32, device=x.device)
    if workspace is None:
        ws = vq_moe_ffn_workspace_size(gate, up, down, n, k)
        workspace = torch.empty(max(ws, 1), dtype=torch.uint8, device=x.device)
    g, u, d = gate.c(), up.c(), down.c()
    _check(lib.vq_moe_ffn(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), n, k, _ptr(x),
                          _x_dtype(x), _ptr(topk_ids.contiguous()),
                          _ptr(topk_weights.contiguous()), _ptr(out), _ptr(workspace),
                          workspace.numel(), _stream()))
    return out


def vq_moe_ffn_noalloc(gate: VQTensor, up: VQTensor, down: VQTensor, x: torch.Tensor,
                       topk_ids: torch.Tensor, topk_weights: torch.Tensor,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """vq_moe_ffn with its workspace in the library's static device array
    (no workspace argument; raises VQError for batches that need more)."""
    _require_gpu()
    lib = load_library()
    x = x.contiguous()
    n, k = topk_ids.shape
    if out is None:
        out = torch.empty((n, gate.cols), dtype=torch.float32, device=x.device)
    g, u, dn = gate.c(), up.c(), down.c()
    _check(lib.vq_moe_ffn_noalloc(ctypes.byref(g), ctypes.byref(u), ctypes.byref(dn), n, k,
                                  _ptr(x), _x_dtype(x), _ptr(topk_ids.contiguous()),
                                  _ptr(topk_weights.contiguous()), _ptr(out), _stream()))
    return out


class _StackArgs:
    """The C layer array and the descriptors it points at, kept alive together."""

    def __init__(self, layers):
        self.tensors = []
        self.arr = (_CLayer * max(len(layers), 1))()
        for i, (g, u, d, ids, w) in enumerate(layers):
            if ids.dtype != torch.int32 or w.dtype != torch.float32:
                raise TypeError("topk_ids must be int32 and topk_weights float32")
            if not (ids.is_contiguous() and w.is_contiguous()):
                raise ValueError("topk_ids and topk_weights must be contiguous")
            cs = (g.c(), u.c(), d.c())
            self.tensors.append(cs)
            self.arr[i] = _CLayer(ctypes.pointer(cs[0]), ctypes.pointer(cs[1]),
                                  ctypes.pointer(cs[2]), ids.data_ptr(), w.data_ptr())


def vq_moe_stack_workspace_size(layers, n_tokens: int, top_k: int) -> int:
    a = _StackArgs(layers)
    return int(load_library().vq_moe_stack_workspace_size(a.arr, len(layers), n_tokens, top_k))


def vq_moe_stack(layers, hidden: torch.Tensor,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hidden <- hidden + FFN_l(hidden) for each layer (gate, up, down,
    topk_ids, topk_weights) in order; fp32 [n_tokens, hidden], in place."""
    _require_gpu()
    lib = load_library()
    if hidden.dtype != torch.float32 or not hidden.is_contiguous():
        raise TypeError("hidden must be a contiguous float32 device tensor")
    n = hidden.shape[0]
    k = layers[0][3].shape[1] if layers else 1
    a = _StackArgs(layers)
    if workspace is None:
        ws = lib.vq_moe_stack_workspace_size(a.arr, len(layers), n, k)
        workspace = torch.empty(max(int(ws), 1), dtype=torch.uint8, device=hidden.device)
    _check(lib.vq_moe_stack(a.arr, len(layers), n, k, _ptr(hidden), _ptr(workspace),
                            workspace.numel(), _stream()))
    return hidden


def vq_moe_gate_up(gate: VQTensor, up: VQTensor, x: torch.Tensor, topk_ids: torch.Tensor,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """h[t*top_k + s] = silu(W_gate_e x_t) * (W_up_e x_t), e = topk_ids[t, s]."""
    _require_gpu()
    lib = load_library()
    x = x.contiguous()
    n, k = topk_ids.shape
    if out is None:
        out = torch.empty((n * k, gate.rows), dtype=torch.float32, device=x.device)
    g, u = gate.c(), up.c()
    _check(lib.vq_moe_gate_up(ctypes.byref(g), ctypes.byref(u), n, k, _ptr(x), _x_dtype(x),
                              _ptr(topk_ids.contiguous()), _ptr(out), _stream()))
    return out


def vq_moe_down(down: VQTensor, h: torch.Tensor, topk_ids: torch.Tensor,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """z[q] = W_down_e h[q] for every (token, slot) pair q."""
    _require_gpu()
    lib = load_library()
    n, k = topk_ids.shape
    if out is None:
        out = torch.empty((n * k, down.rows), dtype=torch.float32, device=h.device)
    dc = down.c()
    _check(lib.vq_moe_down(ctypes.byref(dc), n, k, _ptr(h.contiguous()),
                           _ptr(topk_ids.contiguous()), _ptr(out), _stream()))
    return out


def vq_moe_combine(z: torch.Tensor, topk_weights: torch.Tensor,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y[t] = sum over slots s of topk_weights[t, s] * z[t*top_k + s]."""
    _require_gpu()
    lib = load_library()
    n, k = topk_weights.shape
    hidden = z.shape[1]
    if out is None:
        out = torch.empty((n, hidden), dtype=torch.float32, device=z.device)
    _check(lib.vq_moe_combine(n, k, hidden, _ptr(z.contiguous()),
                              _ptr(topk_weights.contiguous()), _ptr(out), _stream()))
    return out


def vq_set_kernel_events(start, stop) -> None:
    """Record HIP events `start` / `stop` (raw hipEvent_t handles, or None to
    clear) around the dominant kernel of the following calls on this thread."""
    _check(load_library().vq_set_kernel_events(start, stop))


__all__ = [
    "VQError", "VQTensor", "build", "load_library", "vq_validate", "vq_dequantize",
    "vq_row_gather", "vq_fit",
    "vq_expert_gemv", "vq_expert_gemm", "vq_expert_gemm_workspace_size", "vq_moe_ffn",
    "vq_moe_ffn_workspace_size", "vq_moe_ffn_noalloc", "vq_moe_ffn_engine",
    "VQ_ENGINE_DECODE", "VQ_ENGINE_MFMA", "vq_moe_gate_up", "vq_moe_down", "vq_moe_combine",
    "vq_probe_read", "vq_probe_mfma",
    "vq_set_kernel_events", "vq_moe_stack", "vq_moe_stack_workspace_size",
    "VQ_F32", "VQ_BF16",
]
