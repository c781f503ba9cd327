"""Seeded synthetic inputs for the SDM write/read and decode step.

This module holds no part of the method's arithmetic: it only draws random tensors and rounds them to their dtype.
Both the tests' oracle calls and the HIP path take their inputs from here.

Generator: numpy's Philox4x32-10 (a counter-based generator, Salmon et al., SC 2011) keyed by (seed, tensor id),
so any tensor (and any per-stream block of the bank) can be regenerated on its own. Distributions follow the
workload descriptions: queries, write keys, sub-keys and values ~ N(0, 1); forget and input gates =
sigmoid(N(0, 1)); initial bank ~ N(0, 0.02^2). Values are drawn in float32 and rounded to nearest-even bfloat16
where the dtype is bf16; they are returned as float32 arrays holding dtype-exact values.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

# tensor ids of the Philox key
_T_WKEYS, _T_RQ, _T_VALUES, _T_ALPHA, _T_BETA, _T_SUBKEYS, _T_BANK = 1, 2, 3, 4, 5, 6, 7
_T_X, _T_WIN, _T_WOUT, _T_ALOG, _T_DT = 8, 9, 10, 11, 12


@dataclass(frozen=True)
class Shape:
    """One SDM workload: B streams of T tokens over H heads, F product-key factors."""

    batch: int
    tokens: int
    heads: int
    widths: tuple
    subkey_dim: int
    head_dim: int
    num_writes: int
    num_reads: int
    chunk_size: int
    act: str = "f32"      # "f32" | "bf16"
    bank: str = "f32"     # "f32" | "bf16"
    bank_rows: int = 0    # 0 -> exactly N rows per stream
    name: str = field(default="", compare=False)

    @property
    def slots(self) -> int:
        n = 1
        for w in self.widths:
            n *= int(w)
        return n

    @property
    def rows(self) -> int:
        return self.bank_rows or self.slots

    @property
    def streams(self) -> int:
        return self.batch * self.heads

    def with_(self, **kw) -> "Shape":
        return replace(self, **kw)


# The five workloads the method is exercised on (sizes as described for each).
WORKLOADS = {
    # batch 1, 256 tokens, 1 head, 2 factors of 32 (1024 slots), dk 16, d 64, W=R=4, chunk 64, fp32
    "tiny_1k": Shape(1, 256, 1, (32, 32), 16, 64, 4, 4, 64, "f32", "f32", name="tiny_1k"),
    # batch 2, 4096 tokens, 2 heads of 1024, 2 factors of 256 (65536 slots), dk 64, W=R=64, chunk 64,
    # bf16 activations on a float32 bank
    "layer_65k": Shape(2, 4096, 2, (256, 256), 64, 1024, 64, 64, 64, "bf16", "f32", name="layer_65k"),
    # 128 independent streams, one token per step, 2 heads of 256, 2 factors of 32 (1024 slots), dk 32, W=R=64, fp32
    "decode_b128": Shape(128, 1, 2, (32, 32), 32, 256, 64, 64, 1, "f32", "f32", name="decode_b128"),
    # batch 1, 32768 tokens, 4 heads of 256, factors (64, 32, 32) (65536 slots), dk 32, W=R=64, chunk 128, bf16 bank
    "three_factor_65k": Shape(1, 32768, 4, (64, 32, 32), 32, 256, 64, 64, 128, "bf16", "bf16",
                              name="three_factor_65k"),
    # batch 4, 8192 tokens, 4 heads of 512, 2 factors of 1024 (1,048,576 slots), dk 64, W=R=64, chunk 64,
    # bf16 activations on a float32 bank
    "large_1m": Shape(4, 8192, 4, (1024, 1024), 64, 512, 64, 64, 64, "bf16", "f32", name="large_1m"),
}


def round_bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even), returned as float32 (finite inputs)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _rng(seed: int, tensor: int, sub: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=[int(seed) & (2**64 - 1), (tensor << 40) | int(sub)]))


def _normal(seed, tensor, shape, scale=1.0, sub=0) -> np.ndarray:
    a = _rng(seed, tensor, sub).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        a *= np.float32(scale)
    return a


def _as(a: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16_rne(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def _gate(seed, tensor, shape, sub=0) -> np.ndarray:
    z = _rng(seed, tensor, sub).standard_normal(size=shape, dtype=np.float32).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def make_step_inputs(s: Shape, seed: int = 0, step: int = 0) -> dict:
    """Per-token tensors of one call (one decode step uses step > 0 for fresh draws)."""
    B, T, H = s.batch, s.tokens, s.heads
    F = len(s.widths)
    qk = (B, T, H, F * s.subkey_dim)
    return {
        "wkeys": _as(_normal(seed, _T_WKEYS, qk, sub=step), s.act),
        "rq": _as(_normal(seed, _T_RQ, qk, sub=step), s.act),
        "values": _as(_normal(seed, _T_VALUES, (B, T, H, s.head_dim), sub=step), s.act),
        "alpha": _as(_gate(seed, _T_ALPHA, (B, T, H), sub=step), s.act),
        "beta": _as(_gate(seed, _T_BETA, (B, T, H), sub=step), s.act),
    }


def make_subkeys(s: Shape, seed: int = 0) -> np.ndarray:
    return _as(_normal(seed, _T_SUBKEYS, (s.heads, int(sum(s.widths)), s.subkey_dim)), s.act)


def make_bank_stream(s: Shape, b: int, h: int, seed: int = 0) -> np.ndarray:
    """Initial bank rows [bank_rows, d] of stream (b, h) ~ N(0, 0.02^2), in the bank dtype."""
    return _as(_normal(seed, _T_BANK, (s.rows, s.head_dim), scale=0.02, sub=b * s.heads + h), s.bank)


def make_bank(s: Shape, seed: int = 0, threads: int = 8) -> np.ndarray:
    """Initial bank [B, H, bank_rows, d]; streams are drawn independently (in parallel threads)."""
    from concurrent.futures import ThreadPoolExecutor

    out = np.empty((s.batch, s.heads, s.rows, s.head_dim), dtype=np.float32)

    def one(bh):
        b, h = bh
        out[b, h] = make_bank_stream(s, b, h, seed)

    pairs = [(b, h) for b in range(s.batch) for h in range(s.heads)]
    with ThreadPoolExecutor(max_workers=max(1, min(threads, len(pairs)))) as ex:
        list(ex.map(one, pairs))
    return out


def fill_bank_stream_device(rows_view, s: Shape, b: int, h: int, seed: int = 0) -> None:
    """Fills the device bank rows [rows, d] of stream (b, h) (torch view, any row pitch) with N(0, 0.02^2) drawn by
    torch's device generator seeded with seed * 1000003 + b * heads + h, rounded to the view's dtype.

    For banks too large to draw on the host (the 1,048,576-slot workload: 32 GiB); the same seed always gives the
    same values on the same device type."""
    import torch

    g = torch.Generator(device=rows_view.device)
    g.manual_seed(int(seed) * 1000003 + b * s.heads + h)
    z = torch.randn(tuple(rows_view.shape), generator=g, device=rows_view.device, dtype=torch.float32)
    rows_view.copy_((z * 0.02).to(rows_view.dtype))


def fill_bank_device(bank, s: Shape, seed: int = 0) -> None:
    """Fills a device bank view [B, H, rows, d] stream by stream (fill_bank_stream_device)."""
    for b in range(bank.shape[0]):
        for h in range(bank.shape[1]):
            fill_bank_stream_device(bank[b, h], s, b, h, seed)


def make_inputs(s: Shape, seed: int = 0) -> dict:
    d = make_step_inputs(s, seed)
    d["subkeys"] = make_subkeys(s, seed)
    d["bank"] = make_bank(s, seed)
    return d


def make_layer_inputs(s: Shape, model_dim: int, seed: int = 0) -> dict:
    """Inputs of the layer around the op (all bf16 values as float32 except the per-head gate parameters):
    x [B, T, Dm] ~ N(0, 1); w_in [2 H F dk + H d + 2 H, Dm] and w_out [Dm, H d] ~ N(0, 1 / fan_in) (so projections
    and outputs are O(1)); the gate parameters drawn as in FLA's Gated DeltaNet initialisation: A ~ U(0, 16),
    a_log = log A; dt = exp(U(log 0.001, log 0.1)) clamped at 1e-4, dt_bias = dt + log(-expm1(-dt)) (the inverse of
    softplus at dt); sub-keys ~ N(0, 1); the initial bank as for the op."""
    B, T, H, F = s.batch, s.tokens, s.heads, len(s.widths)
    n_in = 2 * H * F * s.subkey_dim + H * s.head_dim + 2 * H
    Dm = int(model_dim)
    u = _rng(seed, _T_ALOG).uniform(0.0, 16.0, size=H)
    dt = np.exp(_rng(seed, _T_DT).uniform(np.log(0.001), np.log(0.1), size=H))
    dt = np.maximum(dt, 1e-4)
    return {
        "x": round_bf16_rne(_normal(seed, _T_X, (B, T, Dm))),
        "w_in": round_bf16_rne(_normal(seed, _T_WIN, (n_in, Dm), scale=1.0 / np.sqrt(Dm))),
        "w_out": round_bf16_rne(_normal(seed, _T_WOUT, (Dm, H * s.head_dim), scale=1.0 / np.sqrt(H * s.head_dim))),
        "a_log": np.log(u).astype(np.float32),
        "dt_bias": (dt + np.log(-np.expm1(-dt))).astype(np.float32),
        "subkeys": make_subkeys(s, seed),
        "bank": make_bank(s, seed),
    }
