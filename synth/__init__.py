"""Seeded synthetic inputs for the VQ MoE expert matmul.

Both the oracle-based tests and the GPU path draw their inputs from here; this
module holds none of the method's arithmetic (no unpacking, no decoding, no
matmul).  It only draws random numbers and writes them in the storage format:

* codebook: fp16 entries ~ N(0, 1), shape [K, d];
* scales: fp16 ~ U(0.01, 0.05), one per (stored row, 64-column group);
* codes: uniform on [0, K), written LSB-first into row-local uint32 streams,
  each row padded to whole 32-code blocks (padding bits are zero).  When
  K == 2**bits a uniform code is a uniform b-bit field, so the stream is drawn
  directly as random words and only the padding is cleared;
* skip-zero: a fixed number of dead rows per (expert, projection), chosen
  uniformly without replacement; dead rows have no codes or scales and the
  row map sends them to -1;
* activations ~ N(0, 1), kept as float32 or rounded to bf16;
* routes: expert ids uniform without replacement per token, gate weights the
  softmax of top_k N(0, 1) logits.

The model cards measure on real checkpoints (Qwen3.5-397B-A17B, Qwen3.8-Flash-
Next, gemma-4-26b-a4b-it, GLM-5.3-Flash); these seeded layers stand in for
them with the cards' geometries, expert counts and skip-zero fraction.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class VQTensorHost:
    """One VQ linear tensor stacked over experts, in host memory."""

    rows: int
    cols: int
    d: int
    bits: int
    K: int
    n_experts: int
    codebook: np.ndarray            # uint16 fp16 bits [K, d]
    codes: np.ndarray               # uint32 [n_stored, wpr]
    scales: np.ndarray              # uint16 fp16 bits [n_stored, cols // 64]
    row_map: Optional[np.ndarray]   # int32 [n_experts * rows], -1 = dead; None = dense
    raw_codes: Optional[np.ndarray] = None  # int codes [n_stored, n_sub] when kept

    @property
    def n_stored(self) -> int:
        return int(self.scales.shape[0])

    @property
    def n_sub(self) -> int:
        return self.cols // self.d

    @property
    def wpr(self) -> int:
        return words_per_row(self.cols, self.d, self.bits)

    @property
    def groups(self) -> int:
        return self.cols // 64

    def stored_bytes(self) -> int:
        """Bytes of codes + scales + row map as stored."""
        n = self.codes.nbytes + self.scales.nbytes
        if self.row_map is not None:
            n += self.row_map.nbytes
        return n

    def expert_stored_rows(self, e: int) -> int:
        if self.row_map is None:
            return self.rows
        return int((self.row_map[e * self.rows:(e + 1) * self.rows] >= 0).sum())


def words_per_row(cols: int, d: int, bits: int) -> int:
    """Row-local 32-code blocks of b words each."""
    n_sub = cols // d
    return ((n_sub + 31) // 32) * bits


def rng_for(seed: int, *stream: int) -> np.random.Generator:
    """Independent PCG64 stream per (seed, stream ids)."""
    return np.random.default_rng(np.random.SeedSequence([int(seed), *[int(s) for s in stream]]))


def to_half_bits(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16).view(np.uint16)


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Write integer codes [n_rows, n_sub] as LSB-first row streams of uint32
    words, each row padded with zero bits to whole 32-code blocks."""
    codes = np.asarray(codes, dtype=np.uint32)
    n_rows, n_sub = codes.shape
    wpr = ((n_sub + 31) // 32) * bits
    if bits == 0 or n_rows == 0:
        return np.zeros((n_rows, wpr), dtype=np.uint32)
    shifts = np.arange(bits, dtype=np.uint32)
    stream = ((codes[:, :, None] >> shifts) & 1).astype(np.uint8).reshape(n_rows, n_sub * bits)
    padded = np.zeros((n_rows, wpr * 32), dtype=np.uint8)
    padded[:, : n_sub * bits] = stream
    packed = np.packbits(padded, axis=1, bitorder="little")
    return np.ascontiguousarray(packed).view("<u4").astype(np.uint32).reshape(n_rows, wpr)


def _padding_mask(n_sub: int, bits: int) -> Optional[np.ndarray]:
    """uint32 mask per word of a row: 1 where the bit belongs to a real code."""
    wpr = ((n_sub + 31) // 32) * bits
    used = n_sub * bits
    if used == wpr * 32:
        return None
    mask = np.zeros(wpr, dtype=np.uint64)
    for w in range(wpr):
        lo, hi = 32 * w, 32 * w + 32
        n = max(0, min(hi, used) - lo)
        mask[w] = (1 << n) - 1
    return mask.astype(np.uint32)


def make_tensor(seed: int, stream: int, *, rows: int, cols: int, d: int, bits: int,
                K: Optional[int] = None, n_experts: int = 1, dead_rows: int = 0,
                keep_codes: bool = False, scale_range=(0.01, 0.05)) -> VQTensorHost:
    """A seeded VQ tensor.  ``dead_rows`` rows of every expert are dead
    (skip-zero).  ``keep_codes`` also returns the integer codes."""
    K = (1 << bits) if K is None else K
    if cols % 64 or cols % d:
        raise ValueError("cols must be a multiple of 64 and of d")
    if not 1 <= K <= (1 << bits):
        raise ValueError("need 1 <= K <= 2**bits")
    if not 0 <= dead_rows <= rows:
        raise ValueError("dead_rows out of range")
    g_cb, g_sc, g_code, g_dead = (rng_for(seed, stream, i) for i in range(4))
    codebook = to_half_bits(g_cb.standard_normal((K, d)))

    row_map = None
    n_stored = n_experts * rows
    if dead_rows:
        row_map = np.full(n_experts * rows, -1, dtype=np.int32)
        nxt = 0
        for e in range(n_experts):
            dead = g_dead.choice(rows, size=dead_rows, replace=False)
            live = np.ones(rows, dtype=bool)
            live[dead] = False
            idx = np.nonzero(live)[0]
            row_map[e * rows + idx] = np.arange(nxt, nxt + len(idx), dtype=np.int32)
            nxt += len(idx)
        n_stored = nxt

    scales = to_half_bits(g_sc.uniform(*scale_range, size=(n_stored, cols // 64)))
    n_sub = cols // d
    wpr = words_per_row(cols, d, bits)
    raw = None
    if K == (1 << bits) and bits > 0 and not keep_codes:
        codes = g_code.integers(0, 1 << 32, size=(n_stored, wpr), dtype=np.uint32)
        mask = _padding_mask(n_sub, bits)
        if mask is not None:
            codes &= mask[None, :]
    else:
        raw = g_code.integers(0, K, size=(n_stored, n_sub), dtype=np.uint32)
        codes = pack_codes(raw, bits)
    return VQTensorHost(rows, cols, d, bits, K, n_experts, codebook,
                        np.ascontiguousarray(codes), scales, row_map, raw)


def make_x(seed: int, stream: int, n_tok: int, cols: int, dtype: str = "bf16") -> np.ndarray:
    """Activations ~ N(0, 1): float32 values or bf16 bit patterns (uint16)."""
    x = rng_for(seed, stream).standard_normal((n_tok, cols)).astype(np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return to_bf16_bits(x)
    raise ValueError(dtype)


def make_routes(seed: int, stream: int, n_tok: int, n_experts: int, top_k: int):
    """Expert ids uniform without replacement per token, gate weights the
    softmax of top_k N(0, 1) logits (float32)."""
    g = rng_for(seed, stream)
    keys = g.random((n_tok, n_experts))
    ids = np.argsort(keys, axis=1)[:, :top_k].astype(np.int32)
    logits = g.standard_normal((n_tok, top_k))
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    w = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    return np.ascontiguousarray(ids), np.ascontiguousarray(w)


# --------------------------------------------------------------------------
# The workloads: shapes and geometries of the model cards' MoE layers.
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class MoEWorkload:
    name: str
    n_experts: int
    top_k: int
    hidden: int
    inter: int
    d: int
    bits: int
    n_tok: int
    dead_frac: float = 0.0
    seed: int = 1234

    def dead_rows(self, rows: int) -> int:
        return int(round(self.dead_frac * rows))


WORKLOADS = {
    # 128 experts, top-8 (the gemma-4 card's routing), d=4/K=512 9-bit
    # (the Qwen3.5-397B 2.6bpw and GLM-5.3 base geometry), one token.
    "moe_decode_e128_h2048_i768_d4k512_b1": MoEWorkload(
        "moe_decode_e128_h2048_i768_d4k512_b1", 128, 8, 2048, 768, 4, 9, 1, seed=1235),
    # 10 of 512 experts (the Qwen3.8-Flash-Next card), d=2/K=256 8-bit.
    "moe_decode_e512_h4096_i1024_d2k256_b1": MoEWorkload(
        "moe_decode_e512_h4096_i1024_d2k256_b1", 512, 10, 4096, 1024, 2, 8, 1, seed=1236),
    "moe_decode_e512_h4096_i1024_d2k256_b8": MoEWorkload(
        "moe_decode_e512_h4096_i1024_d2k256_b8", 512, 10, 4096, 1024, 2, 8, 8, seed=1236),
    # Its promoted layers: d=2/K=1024, 10-bit packed.
    "moe_decode_e512_h4096_i1024_d2k1024_b1": MoEWorkload(
        "moe_decode_e512_h4096_i1024_d2k1024_b1", 512, 10, 4096, 1024, 2, 10, 1, seed=1237),
    "moe_decode_e512_h4096_i1024_d2k1024_b8": MoEWorkload(
        "moe_decode_e512_h4096_i1024_d2k1024_b8", 512, 10, 4096, 1024, 2, 10, 8, seed=1237),
    # Batches between decode and prefill (multi-token verify steps, short
    # prompts): the decode geometries at 17, 32 and 64 tokens, and the 128-
    # expert one up to 128 tokens (4 routed pairs per expert at 64 tokens);
    # 16 tokens is the last batch the decode kernels take by count alone.
    **{f"moe_batch_e512_h4096_i1024_d2k256_t{t}": MoEWorkload(
        f"moe_batch_e512_h4096_i1024_d2k256_t{t}", 512, 10, 4096, 1024, 2, 8, t, seed=1240 + t)
       for t in (16, 17, 32, 64)},
    **{f"moe_batch_e128_h2048_i768_d4k512_t{t}": MoEWorkload(
        f"moe_batch_e128_h2048_i768_d4k512_t{t}", 128, 8, 2048, 768, 4, 9, t, seed=1240 + t)
       for t in (17, 32, 64, 128)},
    # Prefill: 2048 tokens, 128 experts top-8, d=4/K=2048 11-bit.
    "moe_prefill_e128_h2816_i704_d4k2048_t2048": MoEWorkload(
        "moe_prefill_e128_h2816_i704_d4k2048_t2048", 128, 8, 2816, 704, 4, 11, 2048, seed=1238),
    # Prefill: 4096 tokens, 512 experts top-10, d=2/K=256, 12.43 % dead groups.
    "moe_prefill_e512_h4096_i1024_d2k256_t4096_sz": MoEWorkload(
        "moe_prefill_e512_h4096_i1024_d2k256_t4096_sz", 512, 10, 4096, 1024, 2, 8, 4096,
        dead_frac=0.1243, seed=1239),
}

# The single-linear case: weight 256x512 at d=2/K=256, fp32 activations, 1 token.
LINEAR_256x512 = dict(rows=256, cols=512, d=2, bits=8, n_experts=1, seed=1233)


def make_moe_layer(wl: MoEWorkload, layer: int = 0, n_experts: Optional[int] = None,
                   down_scale_range=(0.01, 0.05)):
    """gate, up, down tensors of one MoE layer (one codebook per projection,
    shared by the layer's experts)."""
    E = wl.n_experts if n_experts is None else n_experts
    gate = make_tensor(wl.seed, 100 * layer + 1, rows=wl.inter, cols=wl.hidden, d=wl.d,
                       bits=wl.bits, n_experts=E, dead_rows=wl.dead_rows(wl.inter))
    up = make_tensor(wl.seed, 100 * layer + 2, rows=wl.inter, cols=wl.hidden, d=wl.d,
                     bits=wl.bits, n_experts=E, dead_rows=wl.dead_rows(wl.inter))
    down = make_tensor(wl.seed, 100 * layer + 3, rows=wl.hidden, cols=wl.inter, d=wl.d,
                       bits=wl.bits, n_experts=E, dead_rows=wl.dead_rows(wl.hidden),
                       scale_range=down_scale_range)
    return gate, up, down


def make_moe_inputs(wl: MoEWorkload, step: int = 0, n_experts: Optional[int] = None):
    """Activations (bf16 bit patterns) and routes for one batch."""
    E = wl.n_experts if n_experts is None else n_experts
    x = make_x(wl.seed, 10_000 + step, wl.n_tok, wl.hidden, "bf16")
    ids, w = make_routes(wl.seed, 20_000 + step, wl.n_tok, E, wl.top_k)
    return x, ids, w


# --------------------------------------------------------------------------
# Row gather from VQ embedding tables.  The card "Qwen3.8-Flash-Next-VQ-4.4bpw"
# stores its per-layer n-gram embedding (PLE) tables at d=2/K=256 and reads
# them by hashed row; it gives the total (51.2B parameters over its 40
# layers) but not the table shapes.  Stand-in: one table per layer, 2^18 rows
# of 256 columns (1.4 GB of codes for the 40 tables, several times the
# 256 MB Infinity Cache), and one uniformly random row per (token, layer) in
# place of the model's hash.
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class GatherWorkload:
    name: str
    tables: int
    rows: int
    cols: int
    d: int
    bits: int
    n_tok: int
    seed: int = 1240

    @property
    def n_ids(self) -> int:
        return self.n_tok * self.tables


GATHER_WORKLOADS = {
    "ple_gather_d2k256_tables40_rows262144_cols256_t4096": GatherWorkload(
        "ple_gather_d2k256_tables40_rows262144_cols256_t4096", 40, 1 << 18, 256, 2, 8, 4096),
    "ple_gather_d2k256_tables40_rows262144_cols256_t1": GatherWorkload(
        "ple_gather_d2k256_tables40_rows262144_cols256_t1", 40, 1 << 18, 256, 2, 8, 1),
}


def make_gather_table(wl: GatherWorkload) -> VQTensorHost:
    """The stacked tables: table l is expert l of one VQ tensor."""
    return make_tensor(wl.seed, 1, rows=wl.rows, cols=wl.cols, d=wl.d, bits=wl.bits,
                       n_experts=wl.tables)


def make_gather_ids(wl: GatherWorkload, step: int = 0) -> np.ndarray:
    """int64 ids, token-major: ids[t*tables + l] = l*rows + (row of token t in
    table l), the row uniform on [0, rows)."""
    g = rng_for(wl.seed, 30_000 + step)
    r = g.integers(0, wl.rows, size=(wl.n_tok, wl.tables), dtype=np.int64)
    return np.ascontiguousarray((r + np.arange(wl.tables, dtype=np.int64) * wl.rows).ravel())


# --------------------------------------------------------------------------
# Stacks of MoE layers with promoted layers.  "GLM-5.3-Flash-VQ-2.7bpw" fits
# its 42 expert layers (L3-L44, "Methodology") at d=4/K=512 and promotes
# layers 20, 27, 29, 31, 33, 34, 35 and 39 to d=4/K=2048;
# "Qwen3.8-Flash-Next-VQ-4.4bpw" keeps d=2/K=256 and promotes layers 0, 1, 2,
# 16, 24, 31 and 39 (of 40) to d=2/K=1024 (both opening summaries).  The
# layer shapes are the decode workloads' above.  A layer adds its FFN output to the running state, and an
# FFN of random weights grows about quadratically with its input, so forty
# of them at the experts' usual scales overflow fp32.  In the stacks the down
# projections' scales are drawn 64 times smaller (U(0.01, 0.05) / 64), which
# keeps the state bounded over 40 layers (the layers then change it by 8 %
# and 14 % in L2 for the two stacks below); a real model bounds it with the
# norms between blocks, which are not part of this path.
# --------------------------------------------------------------------------

STACK_DOWN_SCALES = (0.01 / 64, 0.05 / 64)

@dataclass(frozen=True)
class StackWorkload:
    name: str
    n_layers: int
    promoted: tuple            # model layer numbers
    base: MoEWorkload          # shapes, routing and the base geometry
    promoted_bits: int         # same d, wider code
    first_layer: int = 0       # model layer number of stack position 0

    def layer_bits(self, layer: int) -> int:
        """Code width at stack position `layer`."""
        return self.promoted_bits if layer + self.first_layer in self.promoted else self.base.bits

    def layer_workload(self, layer: int) -> MoEWorkload:
        b = self.base
        bits = self.layer_bits(layer)
        return MoEWorkload(f"{self.name}_l{layer}", b.n_experts, b.top_k, b.hidden, b.inter,
                           b.d, bits, b.n_tok, b.dead_frac, b.seed + (17 if bits != b.bits else 0))


STACK_WORKLOADS = {
    "moe_stack42_e128_h2048_i768_d4k512_p8k2048_b1": StackWorkload(
        "moe_stack42_e128_h2048_i768_d4k512_p8k2048_b1", 42, (20, 27, 29, 31, 33, 34, 35, 39),
        WORKLOADS["moe_decode_e128_h2048_i768_d4k512_b1"], 11, first_layer=3),
    "moe_stack40_e512_h4096_i1024_d2k256_p7k1024_b1": StackWorkload(
        "moe_stack40_e512_h4096_i1024_d2k256_p7k1024_b1", 40, (0, 1, 2, 16, 24, 31, 39),
        WORKLOADS["moe_decode_e512_h4096_i1024_d2k256_b1"], 10),
}


def make_stack_inputs(sw: StackWorkload, step: int = 0, n_experts: Optional[int] = None):
    """The step's hidden state (float32 [n_tok, hidden]) and every layer's
    routes (ids int32 [n_layers, n_tok, top_k], weights float32 alike)."""
    b = sw.base
    E = b.n_experts if n_experts is None else n_experts
    x = make_x(b.seed, 40_000 + step, b.n_tok, b.hidden, "f32")
    ids, ws = [], []
    for layer in range(sw.n_layers):
        i, w = make_routes(b.seed, 50_000 + 1000 * step + layer, b.n_tok, E, b.top_k)
        ids.append(i)
        ws.append(w)
    return x, np.stack(ids), np.stack(ws)


def make_stack_layer(sw: StackWorkload, layer: int):
    """gate, up, down of stack layer `layer` (layers of one geometry share
    their values)."""
    return make_moe_layer(sw.layer_workload(layer), down_scale_range=STACK_DOWN_SCALES)


# --------------------------------------------------------------------------
# Weights to fit the format to.  The cards fit real bf16 checkpoints; these
# stand in for them: N(0, 0.02) with 2 % of the weights four times larger
# (a heavier tail, as trained weights have), rounded to bf16.
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class FitWorkload:
    name: str
    n_rows: int
    cols: int
    d: int
    bits: int
    K: int
    n_sample: int
    iters: int
    seed: int = 1234          # the seed the GLM and Flash-Next cards fit with

    def draws(self):
        """The fit set (sorted subvector indices, without replacement) and the
        K initial subvectors, drawn with the workload's seed."""
        g = rng_for(self.seed, 70_000)
        N = self.n_rows * (self.cols // self.d)
        sample = np.sort(g.choice(N, self.n_sample, replace=False)).astype(np.int64)
        init = g.choice(N, self.K, replace=False).astype(np.int64)
        return sample, init


FIT_WORKLOADS = {
    # one gate projection of the 128-expert layer (128 x 768 rows of 2048),
    # d=4/K=512, a 2^20-subvector fit set, 10 Lloyd iterations
    "fit_e128_gate_h2048_i768_d4k512": FitWorkload(
        "fit_e128_gate_h2048_i768_d4k512", 128 * 768, 2048, 4, 9, 512, 1 << 20, 10),
}


def make_fit_weights(seed: int, n_rows: int, cols: int) -> np.ndarray:
    """bf16 bit patterns [n_rows, cols]."""
    g = rng_for(seed, 60_000)
    w = g.standard_normal((n_rows, cols)).astype(np.float32) * np.float32(0.02)
    w *= np.where(g.random((n_rows, cols)) < 0.02, np.float32(4.0), np.float32(1.0))
    return to_bf16_bits(w)
