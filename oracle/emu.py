"""Rounding-point emulator: the oracle's projector with values rounded where a
16-bit MFMA implementation stores them.

TEST INFRASTRUCTURE ONLY, like the rest of this package.  It imports nothing
from the GPU path and repeats no GPU code: it is the oracle's own algorithm
(ref.py, in the pages' order, [KVA] "What the hell?") with a rounding applied
to each intermediate that a 16-bit implementation has to store, everything
else in float64.  Its purpose is to say how much of a measured GPU-vs-oracle
difference the storage precision alone explains, one rounding point at a
time:

  point   value rounded                                     format
  ------  ------------------------------------------------  ------------------
  w       trunk weights (bf16/fp32 storage -> MFMA operand)  fp16
  wh      head weights                                       bf16 (fp16 for q8_0/q4_0)
  in      input times its norm gain, x * g (the row's 1/RMS  fp16
          then scales the input Linear's output)
  a1      attention-norm output                              fp16
  q       Q times log2(e)/sqrt(128) (scores in base 2; the   fp16
          factor itself as a binary32 constant)
  kv      K and V                                            fp16
  p       softmax numerators 2^(s - row max)                 fp16 (the row sum is not rounded)
  o       attention output                                   fp16
  a2      FFN-norm output                                    fp16
  act     silu(gate) * up                                    fp16
  z       final-norm output                                  bf16 (fp16 for q8_0/q4_0)

The accumulations (GEMMs, softmax sums) stay float64 by default, so a
residual difference between this emulation and the GPU is accumulation
order and fp32 rounding, not a storage decision.  With arith=np.float32 and
no rounding point the same steps run in float32 NumPy (sgemm): the
benchmark's float32 CPU baseline.
"""
from __future__ import annotations

import math

import numpy as np

from . import ref

ALL_POINTS = frozenset({"w", "wh", "in", "a1", "q", "kv", "p", "o", "a2", "act", "z"})
# log2(e) / sqrt(128), and the binary32 constant a float32 implementation
# multiplies by (used with the "q" point)
Q_SCALE = math.log2(math.e) / math.sqrt(128.0)
Q_SCALE_F32 = float(np.float32(Q_SCALE))


def f16(x: np.ndarray) -> np.ndarray:
    """Nearest-even binary16 value of x (float64 in, float64 out)."""
    return ref.f16_bits_to_f64(ref.f64_to_f16_bits(x))


def bf16(x: np.ndarray) -> np.ndarray:
    """Nearest-even bf16 value of x (float64 in, float64 out)."""
    return ref.bf16_bits_to_f64(ref.f64_to_bf16_bits(x))


def _r(points, name, fn, x):
    return fn(x).astype(x.dtype) if name in points else x


def _rmsnorm(x, g, eps):
    """ref.rmsnorm in the dtype of x."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def _silu(x):
    return x / (1.0 + np.exp(-x))


def attention_base2(q2: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int, head_dim: int,
                    points=ALL_POINTS) -> np.ndarray:
    """Causal attention over one block with q2 = q * log2(e) / sqrt(head_dim):
    scores are then in base-2 units, p = 2^(s - rowmax), o = (p V) / sum(p).
    With no rounding this equals ref.causal_attention(q, k, v) up to the
    float64 rounding of the rescaled scores."""
    T = q2.shape[0]
    out = np.empty((T, n_heads * head_dim), dtype=q2.dtype)
    allowed = np.tril(np.ones((T, T), dtype=bool))
    for h in range(n_heads):
        c = slice(h * head_dim, (h + 1) * head_dim)
        s = np.where(allowed, q2[:, c] @ k[:, c].T, -np.inf)
        p = np.exp2(s - np.max(s, axis=1, keepdims=True))
        l = np.sum(p, axis=1, keepdims=True)
        out[:, c] = (_r(points, "p", f16, p) @ v[:, c]) / l
    return out


def project(cfg: dict, weights: dict, x: np.ndarray, points=ALL_POINTS, which=None, arith=np.float64) -> dict:
    """Per-head outputs {head: [T, out_dim]} of the projector with the given
    rounding points applied (ALL_POINTS: every storage rounding of a 16-bit
    implementation; an empty set reproduces ref.project up to float64
    rounding), computed in `arith` (float64 or float32)."""
    points = frozenset(points)
    unknown = points - ALL_POINTS
    if unknown:
        raise ValueError(f"unknown rounding points {sorted(unknown)}")
    dt = cfg["weight_dtype"]
    quant = dt in ("q8_0", "q4_0")
    d, f, n_in = cfg["d_model"], cfg["d_ffn"], cfg["n_in"]
    H, hd = cfg["n_heads"], cfg["head_dim"]
    eps = cfg["eps"]

    ar = np.dtype(arith)

    def wt(w, o, i):
        return _r(points, "w", f16, ref.weight_f64(w, dt, o, i)).astype(ar)

    x = np.asarray(x, dtype=ar)
    g_in = weights["in_norm"].astype(ar)
    w_in = wt(weights["in_proj"], d, n_in)
    blocks = []
    for b in weights["blocks"]:
        blocks.append({k: wt(b[k], *shape) for k, shape in
                       (("wq", (H * hd, d)), ("wk", (H * hd, d)), ("wv", (H * hd, d)), ("wo", (d, H * hd)),
                        ("w_gate", (f, d)), ("w_up", (f, d)), ("w_down", (d, f)))})
        blocks[-1]["attn_norm"] = b["attn_norm"].astype(ar)
        blocks[-1]["ffn_norm"] = b["ffn_norm"].astype(ar)
    g_out = weights["out_norm"].astype(ar)
    z_round = f16 if quant else bf16

    z = np.empty((x.shape[0], d), dtype=ar)
    for s, e in ref.block_ranges(x.shape[0], cfg["attn_block"]):
        if "in" in points:
            # a 16-bit implementation that folds the norm into the GEMM rounds
            # x * g and applies the row's 1/RMS to the product afterwards
            xb = x[s:e]
            rin = 1.0 / np.sqrt(np.mean(xb * xb, axis=-1, keepdims=True) + eps)
            h = (f16(xb * g_in).astype(ar) @ w_in.T) * rin
        else:
            h = _rmsnorm(x[s:e], g_in, eps) @ w_in.T
        for b in blocks:
            a = _r(points, "a1", f16, _rmsnorm(h, b["attn_norm"], eps))
            q2 = (a @ b["wq"].T) * ar.type(Q_SCALE_F32 if "q" in points else Q_SCALE)
            q2 = _r(points, "q", f16, q2)
            k = _r(points, "kv", f16, a @ b["wk"].T)
            v = _r(points, "kv", f16, a @ b["wv"].T)
            o = _r(points, "o", f16, attention_base2(q2, k, v, H, hd, points))
            h = h + o @ b["wo"].T
            a = _r(points, "a2", f16, _rmsnorm(h, b["ffn_norm"], eps))
            act = _r(points, "act", f16, _silu(a @ b["w_gate"].T) * (a @ b["w_up"].T))
            h = h + act @ b["w_down"].T
        z[s:e] = _r(points, "z", z_round, _rmsnorm(h, g_out, eps))

    out = {}
    which = range(len(cfg["heads"])) if which is None else which
    for i in which:
        hdesc = cfg["heads"][i]
        W = ref.weight_f64(weights["heads"][i]["w"], dt, hdesc["out_dim"], d)
        W = _r(points, "wh", f16 if quant else bf16, W).astype(ar)
        y = z @ W.T
        if weights["heads"][i]["b"] is not None:
            y = y + np.asarray(weights["heads"][i]["b"], dtype=ar)
        out[i] = y
    return out
