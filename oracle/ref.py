"""CPU oracle for the KVA projector and its attention-layer KV-cache write.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module; only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It is written to be read against the pages, not to be fast:
plain NumPy in float64, one library matmul per Linear, no fusion, no blocking.

Sources (titles of the pages the method is described on):
  [KVA]  "Qwen3.8-27B-KVA: late-layer KV approximation" (model card)
  [MLA]  "Qwen3.8-27B-MLA" (model card; used only for the base model's
         attention geometry and rotary frequency law)

What the oracle computes, in the pages' order ([KVA] "What the hell?"):
  residual of layer 31 -> RMSNorm -> Linear(5120 -> d) -> 3 x causal
  transformer block -> RMSNorm -> one Linear head per late layer,
with attention confined to the block (ubatch) of at most 1024 consecutive
tokens a call is split into, so nothing depends on prompt length.

Readings where the pages leave a step open are listed with each function.
Every function here is pinned by tests against the pages' printed values,
library special cases, closed forms, invariants or brute force, except the
points marked "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

# --------------------------------------------------------------------------
# stored formats -> float64


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern = upper 16 bits of an IEEE binary32 value."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> float64 (subnormals included)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


Q8_0_BLOCK = 32
Q8_0_BYTES = 34      # fp16 scale + 32 int8 codes
Q4_0_BYTES = 18      # fp16 scale + 32 4-bit codes


def dequant_q8_0(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """q8_0 (ggml's 8-bit block format, named on [KVA] "Projector quantization
    and flash-attn"): each run of 32 consecutive inputs of a weight row is one
    block holding a fp16 scale d and 32 int8 codes q; the weight is d * q.
    The product of a fp16 value and an int8 has at most 11 + 8 significant
    bits, so float64 (and float32) hold it exactly."""
    nb = cols // Q8_0_BLOCK
    blk = np.asarray(packed, dtype=np.uint8).reshape(rows, nb, Q8_0_BYTES)
    d = f16_bits_to_f64(np.ascontiguousarray(blk[:, :, 0:2]).view(np.uint16)[:, :, 0])
    q = np.ascontiguousarray(blk[:, :, 2:]).view(np.int8).astype(np.float64)
    return (d[:, :, None] * q).reshape(rows, cols)


def dequant_q4_0(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """q4_0 (ggml's 4-bit block format, the card's smaller projector file on
    [KVA] "Projector quantization and flash-attn"): each run of 32 inputs is
    one 18-byte block, a fp16 scale d then 16 bytes of 4-bit codes n; the
    weight is d * (n - 8).  The pages fix only the block size (the 525 MB
    file); the code order (byte j: input j in the low nibble, input j + 16
    in the high nibble) and the offset 8 are ggml's.  d * (n - 8) has at
    most 11 + 4 significant bits: exact in float64."""
    nb = cols // Q8_0_BLOCK
    blk = np.asarray(packed, dtype=np.uint8).reshape(rows, nb, Q4_0_BYTES)
    d = f16_bits_to_f64(np.ascontiguousarray(blk[:, :, 0:2]).view(np.uint16)[:, :, 0])
    qs = blk[:, :, 2:].astype(np.int64)
    n = np.concatenate([qs & 0xF, qs >> 4], axis=2).astype(np.float64)   # inputs 0..15, then 16..31
    return (d[:, :, None] * (n - 8.0)).reshape(rows, cols)


def weight_f64(w: np.ndarray, dtype: str, out_dim: int, in_dim: int) -> np.ndarray:
    """A stored Linear weight [out][in] as float64 values."""
    if dtype == "f32":
        return np.asarray(w, dtype=np.float32).astype(np.float64).reshape(out_dim, in_dim)
    if dtype == "bf16":
        return bf16_bits_to_f64(w).reshape(out_dim, in_dim)
    if dtype == "q8_0":
        return dequant_q8_0(w, out_dim, in_dim)
    if dtype == "q4_0":
        return dequant_q4_0(w, out_dim, in_dim)
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# float64 -> bf16 (single rounding, nearest even)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values once to the nearest bf16 (ties to even) and return
    the bit patterns.  bf16 keeps 8 significant bits and binary32's exponent
    range; below 2^-126 the spacing stays 2^-133 (subnormals)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    fin = np.isfinite(x) & (x != 0)
    m, e = np.frexp(x[fin])                  # x = m * 2^e, 0.5 <= |m| < 1
    ulp_exp = np.maximum(e - 8, -133)        # 8 significant bits
    ulp = np.ldexp(1.0, ulp_exp)
    r = np.rint(x[fin] / ulp) * ulp          # rint rounds half to even
    out[fin] = r
    out[~fin] = x[~fin]
    with np.errstate(over="ignore"):
        f = out.astype(np.float32)           # exact: r has <= 8 significant bits
    big = np.abs(out) >= 2.0 ** 128          # rounded past the largest bf16
    f[big] = np.copysign(np.inf, out[big])
    bits = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(x)] = 0x7FC0
    return bits


def f64_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values once to the nearest IEEE binary16 (ties to even)
    and return the bit patterns.  binary16 keeps 11 significant bits; below
    2^-14 the spacing stays 2^-24 (subnormals); a result past 65504 is an
    infinity."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.float64)
    fin = np.isfinite(x) & (x != 0)
    m, e = np.frexp(x[fin])                  # x = m * 2^e, 0.5 <= |m| < 1
    ulp = np.ldexp(1.0, np.maximum(e - 11, -24))
    out[fin] = np.rint(x[fin] / ulp) * ulp   # rint rounds half to even
    out[~fin] = x[~fin]
    big = np.abs(out) > 65504.0              # rounded past the largest binary16
    with np.errstate(over="ignore"):
        h = out.astype(np.float16)           # exact: out has <= 11 significant bits
    h[big] = np.copysign(np.inf, out[big]).astype(np.float16)
    bits = h.view(np.uint16).copy()
    bits[np.isnan(x)] = 0x7E00
    return bits


def dequant_q4_0_f16_bits(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """q4_0 weights d * (n - 8) rounded once to the nearest binary16."""
    return f64_to_f16_bits(dequant_q4_0(packed, rows, cols))


def dequant_q8_0_f16_bits(packed: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """The fp16 weights an fp16 MFMA path feeds on for q8_0 weights: the exact
    product d * q (dequant_q8_0) rounded once to the nearest binary16."""
    return f64_to_f16_bits(dequant_q8_0(packed, rows, cols))


# --------------------------------------------------------------------------
# building blocks


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: x / sqrt(mean(x^2) + eps) times the stored
    gain.  [KVA] "What the hell?" names RMSNorm without its epsilon; eps sits
    inside the square root and is 1e-6 (reading)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                     n_heads: int, head_dim: int) -> np.ndarray:
    """Multi-head causal self-attention over ONE block of tokens.

    q, k, v: [T, n_heads*head_dim]; head j owns columns [j*head_dim, (j+1)*head_dim).
    Scores are q.k / sqrt(head_dim); key j > query i is excluded before the
    softmax (its weight is exactly zero).  No position encoding is applied:
    the card lists none for the projector and the parameter totals leave no
    room for a learned one (reading).  Returns [T, n_heads*head_dim]."""
    T = q.shape[0]
    out = np.empty((T, n_heads * head_dim), dtype=np.float64)
    allowed = np.tril(np.ones((T, T), dtype=bool))
    for h in range(n_heads):
        c = slice(h * head_dim, (h + 1) * head_dim)
        s = (q[:, c] @ k[:, c].T) / math.sqrt(head_dim)
        s = np.where(allowed, s, -np.inf)
        s = s - np.max(s, axis=1, keepdims=True)
        p = np.exp(s)
        p = p / np.sum(p, axis=1, keepdims=True)
        out[:, c] = p @ v[:, c]
    return out


# --------------------------------------------------------------------------
# the projector


def prepare(cfg: dict, weights: dict) -> dict:
    """float64 copies of the trunk weights (heads are converted on use)."""
    dt = cfg["weight_dtype"]
    d, f, n_in = cfg["d_model"], cfg["d_ffn"], cfg["n_in"]
    hd = cfg["n_heads"] * cfg["head_dim"]
    p = {"in_norm": weights["in_norm"].astype(np.float64),
         "in_proj": weight_f64(weights["in_proj"], dt, d, n_in),
         "out_norm": weights["out_norm"].astype(np.float64), "blocks": []}
    for b in weights["blocks"]:
        p["blocks"].append({
            "attn_norm": b["attn_norm"].astype(np.float64),
            "wq": weight_f64(b["wq"], dt, hd, d), "wk": weight_f64(b["wk"], dt, hd, d),
            "wv": weight_f64(b["wv"], dt, hd, d), "wo": weight_f64(b["wo"], dt, d, hd),
            "ffn_norm": b["ffn_norm"].astype(np.float64),
            "w_gate": weight_f64(b["w_gate"], dt, f, d), "w_up": weight_f64(b["w_up"], dt, f, d),
            "w_down": weight_f64(b["w_down"], dt, d, f)})
    p["_raw"] = weights
    return p


def block_forward(h: np.ndarray, b: dict, cfg: dict) -> np.ndarray:
    """One causal transformer block, pre-norm ([KVA] "What the hell?" and the
    r2/r3 table: attention of 128-wide heads, then a SwiGLU FFN; the
    parameter totals fix full multi-head Q/K/V/O and three FFN matrices).
    Reading: RMSNorm before each sub-layer, residual adds, no trunk biases,
    SwiGLU = silu(gate) * up, then down."""
    eps = cfg["eps"]
    a = rmsnorm(h, b["attn_norm"], eps)
    q, k, v = a @ b["wq"].T, a @ b["wk"].T, a @ b["wv"].T
    o = causal_attention(q, k, v, cfg["n_heads"], cfg["head_dim"])
    h = h + o @ b["wo"].T
    a = rmsnorm(h, b["ffn_norm"], eps)
    act = silu(a @ b["w_gate"].T) * (a @ b["w_up"].T)
    return h + act @ b["w_down"].T


def block_ranges(n_tokens: int, attn_block: int):
    """Consecutive attention blocks of `attn_block` tokens from token 0 of the
    call; the last one may be shorter ([KVA] "What the hell?": attention in
    the projector never looks past the ubatch a token arrived in; the card's
    evaluation uses 1536-token prompts, i.e. a full ubatch and a 512-token
    remainder)."""
    return [(s, min(s + attn_block, n_tokens)) for s in range(0, n_tokens, attn_block)]


def trunk(cfg: dict, prep: dict, x: np.ndarray) -> np.ndarray:
    """Final-normed trunk output z [T, d] for residuals x [T, n_in]."""
    x = np.asarray(x, dtype=np.float64)
    z = np.empty((x.shape[0], cfg["d_model"]), dtype=np.float64)
    for s, e in block_ranges(x.shape[0], cfg["attn_block"]):
        u = rmsnorm(x[s:e], prep["in_norm"], cfg["eps"])
        h = u @ prep["in_proj"].T
        for b in prep["blocks"]:
            h = block_forward(h, b, cfg)
        z[s:e] = rmsnorm(h, prep["out_norm"], cfg["eps"])
    return z


def head_weight(cfg: dict, prep: dict, i: int) -> np.ndarray:
    h = cfg["heads"][i]
    return weight_f64(prep["_raw"]["heads"][i]["w"], cfg["weight_dtype"], h["out_dim"], cfg["d_model"])


def heads(cfg: dict, prep: dict, z: np.ndarray, which=None, cols=None) -> dict:
    """Y_i = z W_i^T + b_i for each requested head i ([KVA] "What the hell?":
    one Linear head per late layer; the table there gives each head's output
    layout: gated DeltaNet qkv | a | b, attention k | v; drafter heads
    kva.res.N / kva.final from the r2/r3 table).  The per-head bias is a
    reading: it is the only choice whose parameter totals round to the card's.
    `cols[i]`, if given, selects output columns of head i."""
    which = range(len(cfg["heads"])) if which is None else which
    out = {}
    for i in which:
        W = head_weight(cfg, prep, i)
        b = prep["_raw"]["heads"][i]["b"]
        if cols is not None and i in cols:
            c = np.asarray(cols[i])
            W = W[c]
            b = None if b is None else b[c]
        y = z @ W.T
        if b is not None:
            y = y + np.asarray(b, dtype=np.float64)
        out[i] = y
    return out


def project(cfg: dict, weights_or_prep: dict, x: np.ndarray, which=None, cols=None) -> dict:
    """The whole projector: per-head outputs {head index: [T, out_dim]} float64."""
    prep = weights_or_prep if "_raw" in weights_or_prep else prepare(cfg, weights_or_prep)
    z = trunk(cfg, prep, x)
    return heads(cfg, prep, z, which, cols)


# --------------------------------------------------------------------------
# parameter accounting ([KVA] r2/r3 table; "Projector quantization")


def param_count(cfg: dict, head_bias: bool | None = None) -> dict:
    d, f, n_in = cfg["d_model"], cfg["d_ffn"], cfg["n_in"]
    hd = cfg["n_heads"] * cfg["head_dim"]
    bias = cfg["has_head_bias"] if head_bias is None else head_bias
    nb = cfg["n_blocks"]
    trunk_w = n_in * d + nb * (3 * hd * d + hd * d + 3 * d * f)
    trunk_g = n_in + nb * 2 * d + d
    mix = [h for h in cfg["heads"] if h["kind"] != "draft"]
    dra = [h for h in cfg["heads"] if h["kind"] == "draft"]
    mixer = sum(h["out_dim"] * (d + (1 if bias else 0)) for h in mix)
    drafter = sum(h["out_dim"] * (d + (1 if bias else 0)) for h in dra)
    return {"trunk": trunk_w + trunk_g, "trunk_linear": trunk_w, "mixer": mixer,
            "drafter": drafter, "total": trunk_w + trunk_g + mixer + drafter,
            "linear": trunk_w + sum(h["out_dim"] * d for h in cfg["heads"])}


def quantized_file_bytes(cfg: dict, bytes_per_block: int, block: int = 32) -> int:
    """Size of the projector with every Linear weight in a 32-element block
    format and norm gains / head biases kept as fp32."""
    pc = param_count(cfg)
    lin = pc["linear"]
    other = pc["total"] - lin
    assert lin % block == 0
    return lin // block * bytes_per_block + 4 * other


# --------------------------------------------------------------------------
# attention-layer KV-cache write ([KVA] "What the hell?": after projection the
# engine applies k_norm and RoPE and writes the KV cache for the attention
# layers; geometry and rotary law from [MLA] "What this is")


def rope_inv_freq(n_rot: int, base: float) -> np.ndarray:
    """Angular speed of rotary pair j: base^(-2j / n_rot), j < n_rot / 2."""
    j = np.arange(n_rot // 2, dtype=np.float64)
    return base ** (-2.0 * j / n_rot)


def rope_rotate(x: np.ndarray, pos: np.ndarray, n_rot: int, base: float) -> np.ndarray:
    """Rotate the first n_rot dims of x [T, ..., D] by position.  Pair j is
    (x[j], x[j + n_rot/2]) (rotate-half pairing: a reading; parity unpinned,
    the pages do not fix the pairing) turned by pos * inv_freq[j]; dims from
    n_rot on pass through."""
    x = np.array(x, dtype=np.float64, copy=True)
    half = n_rot // 2
    th = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(n_rot, base)[None, :]
    shape = (x.shape[0],) + (1,) * (x.ndim - 2) + (half,)
    c, s = np.cos(th).reshape(shape), np.sin(th).reshape(shape)
    a, b = x[..., :half].copy(), x[..., half:n_rot].copy()
    x[..., :half] = a * c - b * s
    x[..., half:n_rot] = a * s + b * c
    return x


def kv_write_values(kv: np.ndarray, gain: np.ndarray, pos0: int, n_kv_heads: int = 4,
                    head_dim: int = 256, n_rot: int = 64, base: float = 1.0e7,
                    eps: float = 1e-6):
    """float64 K and V rows [T, n_kv_heads, head_dim] as they go into the cache.

    kv: [T, 2 * n_kv_heads * head_dim], the attention head's k | v prediction
    (pre-k_norm, pre-RoPE).  K: RMSNorm per KV head over its head_dim values
    times the layer's k_norm gain, then RoPE at absolute position pos0 + t.
    V is stored as predicted (no norm, no rotation)."""
    kv = np.asarray(kv, dtype=np.float64)
    T = kv.shape[0]
    w = n_kv_heads * head_dim
    k = kv[:, :w].reshape(T, n_kv_heads, head_dim)
    v = kv[:, w:2 * w].reshape(T, n_kv_heads, head_dim)
    k = rmsnorm(k, gain, eps)
    k = rope_rotate(k, pos0 + np.arange(T), n_rot, base)
    return k, v


def kv_write(kv, gain, pos0, page_table, k_pool, v_pool, page_size: int = 256, **kw):
    """Write bf16 K and V into paged pools [n_pages][page_size][n_kv_heads][head_dim]
    (bit patterns, updated in place): token at position p goes to page
    page_table[p // page_size], slot p % page_size."""
    k, v = kv_write_values(kv, gain, pos0, **kw)
    kb, vb = f64_to_bf16_bits(k), f64_to_bf16_bits(v)
    for t in range(kb.shape[0]):
        p = pos0 + t
        pg, sl = int(page_table[p // page_size]), p % page_size
        k_pool[pg, sl] = kb[t]
        v_pool[pg, sl] = vb[t]
    return k_pool, v_pool


# --------------------------------------------------------------------------
# quantised KV cache with a Hadamard rotation ([KVA] "Other notes": q8_0 K and
# V caches are supported, and the approximated K and V go through the same
# Hadamard rotation as the exactly computed ones).
# Readings (the pages give no more than that sentence):
#  - the rotation is the orthonormal Walsh-Hadamard transform of Sylvester
#    order over each KV head's 256 dims, y = H x / 16 with
#    H[i][j] = (-1)^popcount(i & j), applied to K after k_norm and RoPE and
#    to V as predicted;
#  - each KV head's 256 rotated values are then 8 q8_0 blocks of 32
#    consecutive dims (ggml's block: fp16 scale d, 32 int8 codes q, value
#    d * q), laid out [n_pages][page_size][n_kv_heads][8 x 34 bytes];
#  - a block's quantisation is decided in binary32, the precision the rotated
#    values exist in: d = amax / 127, q = round-half-away(y / d) (q = 0 when
#    d = 0), clamped to [-127, 127]; the stored scale is d rounded once to
#    fp16 (nearest even).


def hadamard(n: int) -> np.ndarray:
    """Sylvester-order Hadamard matrix of order n (a power of two) from its
    definition H[i][j] = (-1)^(number of bits i and j share)."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    bits = np.bitwise_and(i, j)
    parity = np.zeros_like(bits)
    while np.any(bits):
        parity ^= bits & 1
        bits = bits >> 1
    return np.where(parity == 1, -1.0, 1.0)


def hadamard_rotate(x: np.ndarray) -> np.ndarray:
    """y = H x / sqrt(n) along the last axis (H symmetric and H H = n I, so
    this is an orthogonal involution)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    return x @ hadamard(n) / math.sqrt(n)


def q8_0_quantize(y: np.ndarray):
    """q8_0 blocks of the last axis (a multiple of 32), decided in binary32,
    by ggml's q8_0 block rule (the cache type the engine of [KVA] *Projector
    quantization and flash-attn* writes): d = amax / 127, the reciprocal
    1/d formed once per block, each code = round-half-away(y * (1/d)),
    0 for an all-zero block.  Returns (scale bits uint16 [..., nb], codes
    int8 [..., nb, 32])."""
    y32 = np.asarray(y, dtype=np.float64).astype(np.float32)
    blk = y32.reshape(y32.shape[:-1] + (y32.shape[-1] // Q8_0_BLOCK, Q8_0_BLOCK))
    amax = np.max(np.abs(blk), axis=-1)
    d = (amax / np.float32(127.0)).astype(np.float32)          # binary32 division
    safe = np.where(d == 0, np.float32(1.0), d)
    inv = (np.float32(1.0) / safe).astype(np.float32)          # binary32 reciprocal
    t = (blk * inv[..., None]).astype(np.float32)              # binary32 product
    t64 = t.astype(np.float64)                                  # exact
    q = np.sign(t64) * np.floor(np.abs(t64) + 0.5)              # half away from zero, exact in float64
    q = np.clip(q, -127, 127)
    q[d == 0] = 0
    return f64_to_f16_bits(d.astype(np.float64)), q.astype(np.int8)


def q8_0_block_bytes(d_bits: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Pack scales [..., nb] and codes [..., nb, 32] into [..., nb * 34] bytes
    (per block: the fp16 scale little-endian, then the 32 codes)."""
    nb = d_bits.shape[-1]
    out = np.zeros(d_bits.shape + (Q8_0_BYTES,), dtype=np.uint8)
    out[..., 0] = (d_bits & 0xFF).astype(np.uint8)
    out[..., 1] = (d_bits >> 8).astype(np.uint8)
    out[..., 2:] = q.view(np.uint8)
    return out.reshape(d_bits.shape[:-1] + (nb * Q8_0_BYTES,))


def q8_0_block_values(row_bytes: np.ndarray) -> np.ndarray:
    """Inverse of q8_0_block_bytes up to the values: [..., nb * 34] bytes ->
    float64 [..., nb * 32], each fp16(d) * q exactly."""
    b = np.asarray(row_bytes, dtype=np.uint8)
    nb = b.shape[-1] // Q8_0_BYTES
    blk = b.reshape(b.shape[:-1] + (nb, Q8_0_BYTES))
    d = f16_bits_to_f64(np.ascontiguousarray(blk[..., 0:2]).view(np.uint16)[..., 0])
    q = np.ascontiguousarray(blk[..., 2:]).view(np.int8).astype(np.float64)
    return (d[..., None] * q).reshape(b.shape[:-1] + (nb * Q8_0_BLOCK,))


def kv_write_q8_0_values(kv: np.ndarray, gain: np.ndarray, pos0: int, **kw):
    """float64 rotated K and V [T, n_kv_heads, head_dim] as they are quantised
    (k_norm and RoPE as in kv_write_values, then hadamard_rotate)."""
    k, v = kv_write_values(kv, gain, pos0, **kw)
    return hadamard_rotate(k), hadamard_rotate(v)


def kv_write_q8_0(kv, gain, pos0, page_table, k_pool, v_pool, page_size: int = 256, **kw):
    """Write q8_0 K and V rows into byte pools [n_pages][page_size][n_kv_heads]
    [head_dim / 32 * 34] (updated in place), token at position p on page
    page_table[p // page_size], slot p % page_size."""
    k, v = kv_write_q8_0_values(kv, gain, pos0, **kw)
    kb, vb = q8_0_block_bytes(*q8_0_quantize(k)), q8_0_block_bytes(*q8_0_quantize(v))
    for t in range(kb.shape[0]):
        p = pos0 + t
        pg, sl = int(page_table[p // page_size]), p % page_size
        k_pool[pg, sl] = kb[t]
        v_pool[pg, sl] = vb[t]
    return k_pool, v_pool


# --------------------------------------------------------------------------
# gated-DeltaNet state update ([KVA] "What the hell?": after projection the
# engine runs, for the DeltaNet layers, conv + silu, l2-norm and the DeltaNet
# scan over the approximated tokens; the table of predicted inputs gives
# in_proj_qkv (q, k, v before conv/silu) 10240, in_proj_a 48, in_proj_b 48).
# The pages name the steps but not their formulas.  Readings:
#  - widths: 48 value heads (one a and one b per value head) of 128 dims
#    (v = 6144), so q and k take 2048 each: 16 key heads of 128; value head h
#    reads key head h // 3 (consecutive grouping); qkv order q | k | v;
#  - conv: causal depthwise convolution of width 4 over the token axis on all
#    10240 qkv channels, per-channel weights w[c][0..3] (w[c][3] multiplies
#    the current token), no bias, the previous 3 tokens' raw qkv as the
#    carried conv state (zeros at the start of a sequence); then SiLU;
#  - l2-norm: k / sqrt(sum(k^2) + 1e-6) per key head (q likewise, but q only
#    feeds the layer's output, which the update does not produce);
#  - gates (the gated delta rule's Mamba-2-style decay): per value head and
#    token, log-decay g = -exp(A_log) * softplus(a + dt_bias), decay
#    alpha = exp(g), write strength beta = sigmoid(b);
#  - gated delta rule on the state S [d_v][d_k] (S maps a key to a value):
#    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T;
#  - the update's results are the state after the last token and the new
#    conv state (the last 3 raw qkv rows); per-token outputs are not formed.
# Parity for trained weights is unpinned (none of these formulas is on the
# pages); the pins below check the functions against their definitions.

DN_QKV, DN_NK, DN_NV, DN_HD, DN_CONV = 10240, 16, 48, 128, 4


def causal_conv_silu(x: np.ndarray, w: np.ndarray, conv_state: np.ndarray):
    """x [T, C] raw rows, w [C, W], conv_state [W-1, C] (oldest first).
    Returns (silu(conv) [T, C], new conv state [W-1, C])."""
    x = np.asarray(x, dtype=np.float64)
    W = w.shape[1]
    xp = np.concatenate([np.asarray(conv_state, dtype=np.float64), x], axis=0)
    T = x.shape[0]
    out = np.zeros_like(x)
    for tau in range(W):
        out += xp[tau:tau + T] * np.asarray(w, dtype=np.float64)[:, tau][None, :]
    return silu(out), xp[T:].copy()


def l2norm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def softplus(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return np.logaddexp(0.0, x)


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-x)), evaluated as exp(x) / (1 + exp(x)) for x < 0 so that
    neither branch overflows or cancels."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def deltanet_prepare(mixer_in: np.ndarray, conv_w: np.ndarray, a_log: np.ndarray, dt_bias: np.ndarray,
                     conv_state: np.ndarray, n_k: int = DN_NK, n_v: int = DN_NV, hd: int = DN_HD):
    """From one DeltaNet head's predicted inputs [T, qkv | a | b] to the scan's
    inputs: unit keys k [T, n_k, hd], values v [T, n_v, hd], decays alpha and
    strengths beta [T, n_v], and the new conv state."""
    m = np.asarray(mixer_in, dtype=np.float64)
    qkv_w = 2 * n_k * hd + n_v * hd
    act, new_conv = causal_conv_silu(m[:, :qkv_w], conv_w, conv_state)
    T = m.shape[0]
    k = l2norm(act[:, n_k * hd:2 * n_k * hd].reshape(T, n_k, hd))
    v = act[:, 2 * n_k * hd:].reshape(T, n_v, hd)
    a = m[:, qkv_w:qkv_w + n_v]
    b = m[:, qkv_w + n_v:qkv_w + 2 * n_v]
    g = -np.exp(np.asarray(a_log, dtype=np.float64))[None, :] * softplus(a + np.asarray(dt_bias)[None, :])
    return k, v, np.exp(g), sigmoid(b), new_conv


def gated_delta_scan(S0: np.ndarray, k: np.ndarray, v: np.ndarray, alpha: np.ndarray, beta: np.ndarray,
                     group: int = 3) -> np.ndarray:
    """S0 [n_v, dv, dk]; k [T, n_k, dk] (value head h reads key head h // group);
    v [T, n_v, dv]; alpha, beta [T, n_v].  Token by token:
    S <- alpha S (I - beta k k^T) + beta v k^T.  Returns the final state."""
    S = np.array(S0, dtype=np.float64, copy=True)
    kv_map = np.arange(S.shape[0]) // group
    for t in range(k.shape[0]):
        kk = k[t][kv_map]                                   # [n_v, dk]
        Sk = np.einsum("hvk,hk->hv", S, kk)                 # S k
        a, b = alpha[t][:, None, None], beta[t][:, None, None]
        S = a * S - a * b * Sk[:, :, None] * kk[:, None, :] + b * v[t][:, :, None] * kk[:, None, :]
    return S


def deltanet_update(mixer_in, conv_w, a_log, dt_bias, conv_state, S0, n_k: int = DN_NK,
                    n_v: int = DN_NV, hd: int = DN_HD):
    """One DeltaNet layer's state update over the rows of mixer_in.
    Returns (final state [n_v, hd, hd], new conv state [3, qkv])."""
    k, v, alpha, beta, new_conv = deltanet_prepare(mixer_in, conv_w, a_log, dt_bias, conv_state, n_k, n_v, hd)
    return gated_delta_scan(S0, k, v, alpha, beta, n_v // n_k), new_conv


# --------------------------------------------------------------------------
# single-map projector (the R9V forum post, "R9V Update: Created and adopted
# KVA projections ...": one full map per later layer, fitted by ridge
# regression, from the start layer's residual straight to each later layer's
# input; the start layer is variable).  Readings: each map is affine,
# y_l = W_l x + b_l, with W_l square (the residual width on both sides); the
# maps for a start layer s of an L-layer model are those of layers s+1..L-1.


def map_project(x: np.ndarray, maps, biases=None, dtype: str = "f32") -> list:
    """[x @ W_l^T + b_l] in float64 for every map (weights in their storage
    format, decoded by weight_f64)."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[1]
    out = []
    for i, w in enumerate(maps):
        y = x @ weight_f64(w, dtype, n, n).T
        if biases is not None:
            y = y + np.asarray(biases[i], dtype=np.float64)[None, :]
        out.append(y)
    return out
