"""Seeded synthetic inputs for the KVA projector: configs, weights, residuals.

This module only *draws* numbers and stores them in the formats the projector
consumes (fp32, bf16 bit patterns, q8_0 blocks).  It performs none of the
projector's arithmetic, so the CPU oracle and the GPU path can both take their
inputs from here without sharing any of the computation under test.

Shapes follow the Qwen3.8-27B-KVA model card ("What the hell?" and the r2/r3
table beneath it): a 5120-wide layer-31 residual in, a trunk of width d with
3 causal blocks of multi-head attention (heads of 128) and SwiGLU, and one
linear head per late layer: 24 gated-DeltaNet heads predicting qkv 10240 + a 48
+ b 48, and 8 full-attention heads predicting k 1024 + v 1024.  r3 adds the
drafter heads kva.res.34, kva.res.48, kva.res.62 and kva.final (5120 each).

Distributions: weights N(0, 1/fan_in) rounded once to the stored dtype; norm
gains 1 + 0.02 N(0, 1); head biases N(0, 1/fan_in); residuals N(0, 1) per
element, rescaled per token to an RMS of 4 for the full-size projectors.
q8_0 weights: int8 codes uniform in [-127, 127] and one fp16 scale per block of
32 inputs, |N(0, 1)| / (127 sqrt(fan_in)).  q4_0 weights (the card's other
projector quantisation): 4-bit codes uniform in [0, 15] and one fp16 scale
per block of 32 inputs, |N(0, 1)| / (8 sqrt(fan_in)).
"""
from __future__ import annotations

import copy
import math

import numpy as np

N_IN = 5120  # width of the base model's residual stream

# ---------------------------------------------------------------- configs

def _late_layer_heads(with_drafters: bool):
    """Late layers 32..63: 24 gated-DeltaNet and 8 full-attention layers.

    The card gives only the counts; which late layers are attention layers is
    not stated.  We place attention at every fourth layer (layer % 4 == 3),
    which gives 8 of 32 late layers and 16 of 64 overall, as the card says.
    """
    heads = []
    for layer in range(32, 64):
        if layer % 4 == 3:
            heads.append({"name": f"kva.attn.{layer}", "kind": "attn", "layer": layer,
                          "out_dim": 2048, "segments": [["k", 1024], ["v", 1024]]})
        else:
            heads.append({"name": f"kva.dn.{layer}", "kind": "deltanet", "layer": layer,
                          "out_dim": 10336,
                          "segments": [["qkv", 10240], ["a", 48], ["b", 48]]})
    if with_drafters:
        for layer in (34, 48, 62):
            heads.append({"name": f"kva.res.{layer}", "kind": "draft", "layer": layer,
                          "out_dim": 5120, "segments": [["res", 5120]]})
        heads.append({"name": "kva.final", "kind": "draft", "layer": 64,
                      "out_dim": 5120, "segments": [["final", 5120]]})
    return heads


_CONFIGS = {
    "tiny": {
        "n_in": 512, "d_model": 256, "n_blocks": 3, "n_heads": 2, "head_dim": 128,
        "d_ffn": 704, "attn_block": 1024, "eps": 1e-6, "weight_dtype": "f32",
        "has_head_bias": True, "seed": 0, "n_tokens": 64, "input_rms": None,
        "heads": [
            {"name": "kva.dn.a", "kind": "deltanet", "layer": 32, "out_dim": 1040,
             "segments": [["qkv", 1024], ["a", 8], ["b", 8]]},
            {"name": "kva.dn.b", "kind": "deltanet", "layer": 33, "out_dim": 1040,
             "segments": [["qkv", 1024], ["a", 8], ["b", 8]]},
            {"name": "kva.attn.c", "kind": "attn", "layer": 35, "out_dim": 256,
             "segments": [["k", 128], ["v", 128]]},
        ],
    },
    "r2": {
        "n_in": N_IN, "d_model": 2560, "n_blocks": 3, "n_heads": 20, "head_dim": 128,
        "d_ffn": 7040, "attn_block": 1024, "eps": 1e-6, "weight_dtype": "bf16",
        "has_head_bias": True, "seed": 1, "n_tokens": 1024, "input_rms": 4.0,
        "heads": _late_layer_heads(False),
    },
    "r3": {
        "n_in": N_IN, "d_model": 3072, "n_blocks": 3, "n_heads": 24, "head_dim": 128,
        "d_ffn": 8448, "attn_block": 1024, "eps": 1e-6, "weight_dtype": "bf16",
        "has_head_bias": True, "seed": 2, "n_tokens": 8192, "input_rms": 4.0,
        "heads": _late_layer_heads(True),
    },
}
_CONFIGS["r3_q8_0"] = dict(copy.deepcopy(_CONFIGS["r3"]), weight_dtype="q8_0", seed=3,
                           n_tokens=65536)
_CONFIGS["r3_kv"] = dict(copy.deepcopy(_CONFIGS["r3"]), seed=4, n_tokens=65536)
_CONFIGS["r3_q4_0"] = dict(copy.deepcopy(_CONFIGS["r3"]), weight_dtype="q4_0", seed=5,
                           n_tokens=8192)


def config(name: str, **overrides) -> dict:
    """A deep copy of a named projector config, optionally with fields replaced."""
    cfg = copy.deepcopy(_CONFIGS[name])
    cfg["name"] = name
    cfg.update(overrides)
    return cfg


def config_names():
    return sorted(_CONFIGS)


# ---------------------------------------------------------------- storage formats

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (storage only)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        r[nan] = 0x7FC0
    return r


Q8_0_BLOCK = 32          # int8 codes per block
Q8_0_BYTES = 2 + 32      # fp16 scale followed by the codes


def pack_q8_0(codes: np.ndarray, scales_f16: np.ndarray) -> np.ndarray:
    """Pack int8 codes [rows, cols] and fp16 scales [rows, cols/32] into
    34-byte blocks: little-endian fp16 scale, then 32 int8 codes."""
    rows, cols = codes.shape
    nb = cols // Q8_0_BLOCK
    out = np.empty((rows, nb, Q8_0_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(scales_f16, dtype=np.float16).view(np.uint8).reshape(rows, nb, 2)
    out[:, :, 2:] = codes.reshape(rows, nb, Q8_0_BLOCK).view(np.uint8)
    return out.reshape(rows, nb * Q8_0_BYTES)


Q4_0_BYTES = 2 + 16      # fp16 scale followed by 32 4-bit codes


def pack_q4_0(codes: np.ndarray, scales_f16: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes [rows, cols] (values 0..15) and fp16 scales
    [rows, cols/32] into 18-byte blocks: little-endian fp16 scale, then 16
    bytes whose byte j holds code j in its low nibble and code j + 16 in its
    high nibble (the ggml q4_0 layout)."""
    rows, cols = codes.shape
    nb = cols // Q8_0_BLOCK
    c = np.asarray(codes, dtype=np.uint8).reshape(rows, nb, Q8_0_BLOCK)
    out = np.empty((rows, nb, Q4_0_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = np.ascontiguousarray(scales_f16, dtype=np.float16).view(np.uint8).reshape(rows, nb, 2)
    out[:, :, 2:] = (c[:, :, :16] & 0xF) | ((c[:, :, 16:] & 0xF) << 4)
    return out.reshape(rows, nb * Q4_0_BYTES)


# ---------------------------------------------------------------- weights

def _linear(rng, out_dim, in_dim, dtype):
    if dtype == "q8_0":
        assert in_dim % Q8_0_BLOCK == 0
        codes = rng.integers(-127, 128, size=(out_dim, in_dim), dtype=np.int8)
        sc = np.abs(rng.standard_normal((out_dim, in_dim // Q8_0_BLOCK), dtype=np.float32))
        sc = (sc.astype(np.float64) / (127.0 * math.sqrt(in_dim))).astype(np.float16)
        return pack_q8_0(codes, sc)
    if dtype == "q4_0":
        assert in_dim % Q8_0_BLOCK == 0
        codes = rng.integers(0, 16, size=(out_dim, in_dim), dtype=np.uint8)
        sc = np.abs(rng.standard_normal((out_dim, in_dim // Q8_0_BLOCK), dtype=np.float32))
        sc = (sc.astype(np.float64) / (8.0 * math.sqrt(in_dim))).astype(np.float16)
        return pack_q4_0(codes, sc)
    w = rng.standard_normal((out_dim, in_dim), dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(in_dim))
    if dtype == "f32":
        return w
    if dtype == "bf16":
        return f32_to_bf16_bits(w)
    raise ValueError(dtype)


def _gain(rng, n):
    return (1.0 + 0.02 * rng.standard_normal(n, dtype=np.float32)).astype(np.float32)


def make_weights(cfg: dict, seed: int | None = None) -> dict:
    """Draw every projector tensor in a fixed order from PCG64(seed).

    Order: in_norm, in_proj, blocks 0..n-1 {attn_norm, wq, wk, wv, wo, ffn_norm,
    w_gate, w_up, w_down}, out_norm, then each head's weight and bias.
    Linear weights are [out][in] row-major in the config's weight dtype.
    """
    rng = np.random.default_rng(cfg["seed"] if seed is None else seed)
    dt = cfg["weight_dtype"]
    d, f, n_in = cfg["d_model"], cfg["d_ffn"], cfg["n_in"]
    hd = cfg["n_heads"] * cfg["head_dim"]
    w = {"in_norm": _gain(rng, n_in), "in_proj": _linear(rng, d, n_in, dt), "blocks": []}
    for _ in range(cfg["n_blocks"]):
        b = {}
        b["attn_norm"] = _gain(rng, d)
        b["wq"] = _linear(rng, hd, d, dt)
        b["wk"] = _linear(rng, hd, d, dt)
        b["wv"] = _linear(rng, hd, d, dt)
        b["wo"] = _linear(rng, d, hd, dt)
        b["ffn_norm"] = _gain(rng, d)
        b["w_gate"] = _linear(rng, f, d, dt)
        b["w_up"] = _linear(rng, f, d, dt)
        b["w_down"] = _linear(rng, d, f, dt)
        w["blocks"].append(b)
    w["out_norm"] = _gain(rng, d)
    w["heads"] = []
    for h in cfg["heads"]:
        W = _linear(rng, h["out_dim"], d, dt)
        bias = None
        if cfg["has_head_bias"]:
            bias = (rng.standard_normal(h["out_dim"], dtype=np.float32)
                    * np.float32(1.0 / math.sqrt(d))).astype(np.float32)
        w["heads"].append({"w": W, "b": bias})
    return w


def make_input(cfg: dict, n_tokens: int | None = None, seed: int | None = None) -> np.ndarray:
    """Layer-31 residuals [n_tokens, n_in] fp32 from PCG64(seed + 1000).

    Full-size configs rescale each token to an RMS of cfg['input_rms'] (4),
    the magnitude of a real residual stream; the tiny config keeps N(0, 1)."""
    n = cfg["n_tokens"] if n_tokens is None else n_tokens
    rng = np.random.default_rng((cfg["seed"] if seed is None else seed) + 1000)
    x = rng.standard_normal((n, cfg["n_in"]), dtype=np.float32)
    if cfg.get("input_rms"):
        x64 = x.astype(np.float64)
        s = cfg["input_rms"] / np.sqrt(np.mean(x64 * x64, axis=1, keepdims=True))
        x = (x64 * s).astype(np.float32)
    return np.ascontiguousarray(x)


# ---------------------------------------------------------------- KV-cache write inputs

KV_PAGE = 256        # tokens per KV-cache page
KV_HEADS = 4         # KV heads per attention layer of the base model
KV_HEAD_DIM = 256    # their width
KV_ROT = 64          # rotary dims per KV head
ROPE_BASE = 1.0e7


def make_kv_write_inputs(n_tokens: int, n_layers: int = 8, seed: int = 4,
                         n_pages: int | None = None, head_dim: int = KV_HEAD_DIM):
    """k_norm gains (one [head_dim] gain per attention layer) and a page table
    that is a seeded permutation of the pages the prompt needs."""
    rng = np.random.default_rng(seed + 2000)
    gains = (1.0 + 0.02 * rng.standard_normal((n_layers, head_dim), dtype=np.float32)).astype(np.float32)
    need = -(-n_tokens // KV_PAGE)
    n_pages = need if n_pages is None else n_pages
    ptab = rng.permutation(n_pages)[:need].astype(np.int32)
    return gains, ptab, n_pages


def make_kv_rows(n_tokens: int, width: int = 2 * KV_HEADS * KV_HEAD_DIM, seed: int = 4,
                 scale: float = 1.0) -> np.ndarray:
    """Stand-alone f32 k|v rows [n_tokens, 2048] for exercising the cache write."""
    rng = np.random.default_rng(seed + 3000)
    return (rng.standard_normal((n_tokens, width), dtype=np.float32) * np.float32(scale))


# ---------------------------------------------------------------- DeltaNet layer inputs

DN_QKV, DN_HEADS_V, DN_HEAD_DIM, DN_CONV = 10240, 48, 128, 4


def make_deltanet_params(n_layers: int, seed: int = 6):
    """Per DeltaNet layer, the parameters the state update uses that the
    projector does not produce, drawn like a freshly initialised layer:
    depthwise conv weights [10240][4] ~ U(-1/2, 1/2); decay rates
    A = exp(A_log) log-uniform in [0.01, 16]; dt_bias = softplus^-1(dt) with
    dt log-uniform in [1e-3, 0.1].  fp32."""
    rng = np.random.default_rng(seed + 4000)
    conv_w = rng.uniform(-0.5, 0.5, (n_layers, DN_QKV, DN_CONV)).astype(np.float32)
    a_log = rng.uniform(math.log(0.01), math.log(16.0), (n_layers, DN_HEADS_V)).astype(np.float32)
    dt = np.exp(rng.uniform(math.log(1e-3), math.log(0.1), (n_layers, DN_HEADS_V)))
    dt_bias = (dt + np.log(-np.expm1(-dt))).astype(np.float32)
    return conv_w, a_log, dt_bias


def make_deltanet_state(n_layers: int, seed: int = 6, scale: float = 0.05):
    """Carried state before a ubatch: conv state [3][10240] (raw rows like the
    projector's outputs) and recurrent states [48][128][128] ~ N(0, scale^2)."""
    rng = np.random.default_rng(seed + 5000)
    conv = rng.standard_normal((n_layers, DN_CONV - 1, DN_QKV), dtype=np.float32)
    S = (rng.standard_normal((n_layers, DN_HEADS_V, DN_HEAD_DIM, DN_HEAD_DIM), dtype=np.float32)
         * np.float32(scale))
    return conv, S


def make_deltanet_rows(n_tokens: int, seed: int = 6, width: int = DN_QKV + 2 * DN_HEADS_V) -> np.ndarray:
    """Stand-alone DeltaNet head outputs [n_tokens][qkv | a | b] ~ N(0, 1), fp32
    (the projector's outputs have unit scale)."""
    rng = np.random.default_rng(seed + 6000)
    return rng.standard_normal((n_tokens, width), dtype=np.float32)


# ---------------------------------------------------------------- single-map projector

def map_layers(start_layer: int, n_layers: int = 64) -> int:
    """Maps a start layer needs: one per later layer (start+1 .. n_layers-1)."""
    return n_layers - 1 - start_layer


def make_map_weights(n_in: int, n_maps: int, dtype: str = "bf16", seed: int = 8, bias: bool = True):
    """n_maps square maps [n_in][n_in] ~ N(0, 1/n_in) in the storage format of
    `dtype` (q8_0 / q4_0: random codes and scales of that scale), and fp32
    biases ~ N(0, 1/n_in), drawn map by map from PCG64(seed + 7000)."""
    rng = np.random.default_rng(seed + 7000)
    maps, biases = [], []
    for _ in range(n_maps):
        maps.append(_linear(rng, n_in, n_in, dtype))
        if bias:
            biases.append((rng.standard_normal(n_in, dtype=np.float32) / np.float32(math.sqrt(n_in))))
    return maps, (biases if bias else None)


def make_map_input(n_tokens: int, n_in: int, seed: int = 8, rms: float = 4.0) -> np.ndarray:
    """Start-layer residuals [n_tokens][n_in]: N(0, 1) rows rescaled to RMS `rms`."""
    rng = np.random.default_rng(seed + 8000)
    x = rng.standard_normal((n_tokens, n_in), dtype=np.float32).astype(np.float64)
    x *= rms / np.sqrt(np.mean(x * x, axis=1, keepdims=True))
    return x.astype(np.float32)
