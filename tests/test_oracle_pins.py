"""Pins for the CPU oracle against what the pages and the mathematics fix.

Each test ties one part of oracle/ref.py to something other than itself:
values printed on the pages (tests/golden/kva_card_facts.json), a library
routine for the special case it reduces to, brute force on tiny inputs,
closed forms, or invariants.  A mutation section at the end plants plausible
mistakes in (a copy of) the oracle and checks that some pin catches each.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from oracle import ref


# ------------------------------------------------------------------ shapes and sizes

@pytest.mark.parametrize("name", ["r2", "r3"])
def test_param_totals_match_card(golden, name):
    cfg = synth.config(name)
    pc = oracle.param_count(cfg)
    want = golden["params_millions"][name]
    assert round(pc["trunk"] / 1e6) == want["trunk"]
    assert round(pc["mixer"] / 1e6) == want["mixer"]
    assert round(pc["total"] / 1e6) == want["total"]


def test_exact_param_totals():
    assert oracle.param_count(synth.config("r2"))["total"] == 931_226_368
    assert oracle.param_count(synth.config("r3"))["total"] == 1_238_155_520


def test_head_bias_is_needed_for_r3_mixer(golden):
    # Without one bias per head output the r3 mixer total rounds to 812M, not
    # the card's 813M: the reading "heads carry a bias" is forced by the card.
    pc = oracle.param_count(synth.config("r3"), head_bias=False)
    assert round(pc["mixer"] / 1e6) == 812 != golden["params_millions"]["r3"]["mixer"]


def test_gqa_or_two_matrix_mlp_would_miss_trunk(golden):
    # Alternative block structures move the r2 trunk far from 254M.
    cfg = synth.config("r2")
    d, f = cfg["d_model"], cfg["d_ffn"]
    full = oracle.param_count(cfg)["trunk"]
    gqa = full - 3 * 2 * (d * d - d * 512)           # K/V with 4 KV heads of 128
    two_mlp = full - 3 * d * f                        # no gate matrix
    assert round(full / 1e6) == golden["params_millions"]["r2"]["trunk"]
    assert abs(gqa - 254e6) > 20e6 and abs(two_mlp - 254e6) > 20e6


@pytest.mark.parametrize("name", ["r2", "r3"])
def test_head_output_widths_match_card(golden, name):
    cfg = synth.config(name)
    lay = golden["late_layers"]
    dn = [h for h in cfg["heads"] if h["kind"] == "deltanet"]
    at = [h for h in cfg["heads"] if h["kind"] == "attn"]
    assert len(dn) == lay["late_deltanet"] and len(at) == lay["late_attention"]
    assert all([s[1] for s in h["segments"]] == lay["deltanet_out"] for h in dn)
    assert all([s[1] for s in h["segments"]] == lay["attention_out"] for h in at)
    assert all(h["out_dim"] == sum(s[1] for s in h["segments"]) for h in cfg["heads"])
    shp = golden["projector_shapes"][name]
    assert (cfg["d_model"], cfg["n_heads"], cfg["head_dim"], cfg["d_ffn"], cfg["n_blocks"]) == \
        (shp["d"], shp["heads"], shp["head_dim"], shp["ffn"], shp["blocks"])
    if name == "r3":
        assert [h["name"] for h in cfg["heads"] if h["kind"] == "draft"] == shp["drafters"]
    at_kv = golden["kv_geometry"]
    assert lay["attention_out"][0] == at_kv["kv_heads"] * at_kv["head_dim"]


def test_quantized_file_sizes_match_card(golden):
    cfg = synth.config("r2")
    mb = golden["projector_file_mb"]
    assert round(oracle.quantized_file_bytes(cfg, ref.Q8_0_BYTES) / 1e6) == mb["q8_0"]
    assert round(oracle.quantized_file_bytes(cfg, ref.Q4_0_BYTES) / 1e6) == mb["q4_0"]
    # a different block size law misses the card
    assert round(oracle.quantized_file_bytes(cfg, 33) / 1e6) != mb["q8_0"]


# ------------------------------------------------------------------ library special case

def _torch_projector(cfg, w, x):
    """The same network written with torch's own fp64 CPU operators."""
    dt = torch.float64
    t = lambda a: torch.tensor(np.asarray(a, dtype=np.float64), dtype=dt)
    H, hd, eps = cfg["n_heads"], cfg["head_dim"], cfg["eps"]
    X = t(x)
    T = X.shape[0]
    assert T <= cfg["attn_block"]
    h = F.linear(F.rms_norm(X, (cfg["n_in"],), weight=t(w["in_norm"]), eps=eps), t(w["in_proj"]))
    for b in w["blocks"]:
        a = F.rms_norm(h, (cfg["d_model"],), weight=t(b["attn_norm"]), eps=eps)
        q, k, v = (F.linear(a, t(b[n])).view(T, H, hd).transpose(0, 1) for n in ("wq", "wk", "wv"))
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        h = h + F.linear(o.transpose(0, 1).reshape(T, H * hd), t(b["wo"]))
        a = F.rms_norm(h, (cfg["d_model"],), weight=t(b["ffn_norm"]), eps=eps)
        h = h + F.linear(F.silu(F.linear(a, t(b["w_gate"]))) * F.linear(a, t(b["w_up"])), t(b["w_down"]))
    z = F.rms_norm(h, (cfg["d_model"],), weight=t(w["out_norm"]), eps=eps)
    return [F.linear(z, t(hh["w"]), t(hh["b"])).numpy() for hh in w["heads"]]


def test_tiny_matches_torch_library_ops():
    cfg = synth.config("tiny")
    w, x = synth.make_weights(cfg), synth.make_input(cfg)
    got = oracle.project(cfg, w, x)
    want = _torch_projector(cfg, w, x)
    for i, y in enumerate(want):
        err = np.max(np.abs(got[i] - y)) / np.sqrt(np.mean(y * y))
        assert err < 1e-12, (i, err)


# ------------------------------------------------------------------ brute force

def _micro_cfg():
    return {"n_in": 12, "d_model": 8, "n_blocks": 2, "n_heads": 2, "head_dim": 4, "d_ffn": 10,
            "attn_block": 4, "eps": 1e-6, "weight_dtype": "f32", "has_head_bias": True,
            "seed": 7, "n_tokens": 10, "input_rms": None,
            "heads": [{"name": "h0", "kind": "deltanet", "layer": 32, "out_dim": 5, "segments": [["x", 5]]},
                      {"name": "h1", "kind": "attn", "layer": 35, "out_dim": 3, "segments": [["k", 3]]}]}


def _brute(cfg, w, x):
    """Scalar loops over lists; the attention mask is written as the predicate
    'same block and key not after query' over the whole sequence."""
    eps, B = cfg["eps"], cfg["attn_block"]
    H, hd = cfg["n_heads"], cfg["head_dim"]
    X = [[float(v) for v in row] for row in x]
    T = len(X)

    def lin(A, W, b=None):
        W = [[float(v) for v in r] for r in np.asarray(W)]
        return [[sum(a[k] * W[o][k] for k in range(len(a))) + (float(b[o]) if b is not None else 0.0)
                 for o in range(len(W))] for a in A]

    def norm(A, g):
        out = []
        for a in A:
            r = math.sqrt(sum(v * v for v in a) / len(a) + eps)
            out.append([a[i] / r * float(g[i]) for i in range(len(a))])
        return out

    h = lin(norm(X, w["in_norm"]), w["in_proj"])
    for b in w["blocks"]:
        a = norm(h, b["attn_norm"])
        q, k, v = lin(a, b["wq"]), lin(a, b["wk"]), lin(a, b["wv"])
        o = [[0.0] * (H * hd) for _ in range(T)]
        for hh in range(H):
            for i in range(T):
                js = [j for j in range(T) if j // B == i // B and j <= i]
                s = {j: sum(q[i][hh * hd + c] * k[j][hh * hd + c] for c in range(hd)) / math.sqrt(hd) for j in js}
                m = max(s.values())
                e = {j: math.exp(s[j] - m) for j in js}
                tot = sum(e.values())
                for c in range(hd):
                    o[i][hh * hd + c] = sum(e[j] / tot * v[j][hh * hd + c] for j in js)
        ao = lin(o, b["wo"])
        h = [[h[i][c] + ao[i][c] for c in range(len(h[i]))] for i in range(T)]
        a = norm(h, b["ffn_norm"])
        g, u = lin(a, b["w_gate"]), lin(a, b["w_up"])
        act = [[g[i][c] / (1.0 + math.exp(-g[i][c])) * u[i][c] for c in range(len(g[i]))] for i in range(T)]
        dd = lin(act, b["w_down"])
        h = [[h[i][c] + dd[i][c] for c in range(len(h[i]))] for i in range(T)]
    z = norm(h, w["out_norm"])
    return [np.array(lin(z, hh["w"], hh["b"])) for hh in w["heads"]]


def test_brute_force_micro_with_ragged_blocks():
    cfg = _micro_cfg()
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg)
    assert ref.block_ranges(10, 4) == [(0, 4), (4, 8), (8, 10)]
    got = oracle.project(cfg, w, x)
    want = _brute(cfg, w, x)
    for i, y in enumerate(want):
        assert np.max(np.abs(got[i] - y)) <= 1e-12 * max(1.0, np.max(np.abs(y))), i


# ------------------------------------------------------------------ invariants

def test_causality_and_block_independence_bitwise():
    cfg = synth.config("tiny", attn_block=16)
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=40)
    prep = ref.prepare(cfg, w)
    y0 = ref.project(cfg, prep, x)
    j = 20                       # inside block [16, 32)
    x2 = x.copy()
    x2[j] += np.float32(0.5)
    y1 = ref.project(cfg, prep, x2)
    for i in y0:
        a, b = y0[i], y1[i]
        assert np.array_equal(a[:j], b[:j])          # earlier tokens
        assert np.array_equal(a[32:], b[32:])        # later blocks
        assert not np.array_equal(a[j], b[j])        # the token itself
        assert not np.array_equal(a[j + 1:32], b[j + 1:32])


def test_prompt_length_independence_bitwise():
    cfg = synth.config("tiny", attn_block=16)
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=48)
    prep = ref.prepare(cfg, w)
    whole = ref.project(cfg, prep, x)
    for s in (0, 16, 32):
        part = ref.project(cfg, prep, x[s:s + 16])
        for i in whole:
            assert np.array_equal(whole[i][s:s + 16], part[i])


def test_rmsnorm_scale_invariance():
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=8)
    prep = ref.prepare(cfg, w)
    y0 = ref.project(cfg, prep, x)
    y1 = ref.project(cfg, prep, x * 3.0)
    for i in y0:
        assert np.max(np.abs(y0[i] - y1[i])) < 1e-5 * np.max(np.abs(y0[i]))
    # closed form: a constant row c normalises to sign(c)/sqrt(1 + eps/c^2)
    v = ref.rmsnorm(np.full((1, 6), -2.0), np.ones(6), 1e-6)
    assert np.allclose(v, -1.0 / math.sqrt(1.0 + 1e-6 / 4.0), rtol=0, atol=1e-15)


def test_first_token_attends_only_to_itself():
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((5, 256)) for _ in range(3))
    o = ref.causal_attention(q, k, v, 2, 128)
    assert np.array_equal(o[0], v[0])                 # softmax over one key is exactly 1
    o2 = ref.causal_attention(q, k, np.ones_like(v), 2, 128)
    assert np.allclose(o2, 1.0, atol=1e-15)           # weights sum to one


def test_attention_scale_and_softmax_closed_form():
    # two tokens, one head: the second query weighs keys by exp(q.k / sqrt(hd))
    hd = 4
    q = np.array([[0.0] * hd, [1.0, 2.0, 0.0, 0.0]])
    k = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]])
    v = np.array([[1.0, 0.0, 0.0, 0.0], [0.0, 1.0, 0.0, 0.0]])
    o = ref.causal_attention(q, k, v, 1, hd)
    s0, s1 = 1.0 / 2.0, 2.0 / 2.0
    p1 = math.exp(s1) / (math.exp(s0) + math.exp(s1))
    assert np.allclose(o[1], [1 - p1, p1, 0, 0], atol=1e-15)


# ------------------------------------------------------------------ formats

def test_f16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32)
    s = np.where(bits >> 15, -1.0, 1.0)
    e = (bits >> 10) & 0x1F
    m = (bits & 0x3FF).astype(np.float64)
    want = np.where(e == 0, s * m * 2.0 ** -24, s * (1.0 + m / 1024.0) * np.exp2(e.astype(np.float64) - 15))
    got = ref.f16_bits_to_f64(bits.astype(np.uint16))
    fin = e != 31
    assert np.array_equal(got[fin], want[fin])
    assert np.all(np.isinf(got[(e == 31) & ((bits & 0x3FF) == 0)]))


def test_q8_0_dequant_hand_blocks():
    # block 0: scale 0.5, codes -128..-97; block 1: smallest subnormal scale 2^-24;
    # block 2: scale -0.0; block 3: largest fp16 65504 with codes +-1
    scales = np.array([0.5, 2.0 ** -24, -0.0, 65504.0], dtype=np.float16)
    codes = np.zeros((4, 32), dtype=np.int8)
    codes[0] = np.arange(-128, -96)
    codes[1] = np.arange(0, 32) * 4 - 64
    codes[2] = 77
    codes[3, ::2], codes[3, 1::2] = 1, -1
    packed = synth.pack_q8_0(codes.reshape(1, 128), scales.reshape(1, 4))
    assert packed.shape == (1, 4 * 34)
    v = ref.dequant_q8_0(packed, 1, 128).reshape(4, 32)
    assert np.array_equal(v[0], 0.5 * np.arange(-128, -96))
    assert np.array_equal(v[1], (np.arange(0, 32) * 4 - 64) * 2.0 ** -24)
    assert np.all(v[2] == 0.0)
    assert np.array_equal(v[3], np.tile([65504.0, -65504.0], 16))


def test_f16_rounding_hand_cases_and_torch():
    # ties to even, subnormal spacing 2^-24, overflow past 65504, signed zero
    cases = {1 + 2.0 ** -11: 0x3C00, 1 + 3 * 2.0 ** -11: 0x3C02, 2.0 ** -25: 0x0000,
             3 * 2.0 ** -26: 0x0001, 65519.0: 0x7BFF, 65520.0: 0x7C00, -0.0: 0x8000,
             -65536.0: 0xFC00, 2.0 ** -14: 0x0400, 1.0 / 3.0: 0x3555}
    got = ref.f64_to_f16_bits(np.array(list(cases)))
    assert [int(b) for b in got] == list(cases.values())
    # against torch's conversion on float32 inputs across the whole range
    rng = np.random.default_rng(6)
    x32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 20, 20000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ref.f64_to_f16_bits(x32.astype(np.float64)), want)
    # float64 inputs: one of the two binary16 neighbours, the nearer one
    x = rng.standard_normal(20000) * 64
    v = ref.f16_bits_to_f64(ref.f64_to_f16_bits(x))
    up = np.nextafter(x.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(x.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    assert np.all(np.abs(v - x) <= np.minimum(np.abs(up - x), np.abs(dn - x)) + 0.0)


def test_q8_0_f16_weights_hand_blocks():
    # exact products stay exact; a halfway product rounds to even; overflow -> inf
    scales = np.array([0.5, 2.0 ** -24, 1 + 2.0 ** -10, 65504.0], dtype=np.float16)
    codes = np.zeros((4, 32), dtype=np.int8)
    codes[0] = np.arange(-128, -96)
    codes[1, :] = 3
    codes[2, :] = 3
    codes[3, 0], codes[3, 1], codes[3, 2] = 1, -1, 2
    packed = synth.pack_q8_0(codes.reshape(1, 128), scales.reshape(1, 4))
    b = ref.dequant_q8_0_f16_bits(packed, 1, 128).reshape(4, 32)
    assert np.array_equal(ref.f16_bits_to_f64(b[0]), 0.5 * np.arange(-128, -96))
    assert np.all(b[1] == 0x0003)                      # 3 * 2^-24, a subnormal, exact
    assert np.all(b[2] == 0x4202)                      # 3 + 3*2^-10: halfway, to even 3 + 2^-8
    assert (b[3, 0], b[3, 1], b[3, 2], b[3, 3]) == (0x7BFF, 0xFBFF, 0x7C00, 0x0000)


def test_q4_0_dequant_hand_blocks_and_brute_force():
    # block 0: scale 0.5, codes 0..15 then 15..0; block 1: smallest subnormal
    # scale; block 2: scale -0.0; block 3: largest fp16 with codes 0 and 15
    scales = np.array([0.5, 2.0 ** -24, -0.0, 65504.0], dtype=np.float16)
    codes = np.zeros((4, 32), dtype=np.uint8)
    codes[0, :16], codes[0, 16:] = np.arange(16), np.arange(15, -1, -1)
    codes[1] = np.arange(32) % 16
    codes[2] = 9
    codes[3, ::2], codes[3, 1::2] = 0, 15
    packed = synth.pack_q4_0(codes.reshape(1, 128), scales.reshape(1, 4))
    assert packed.shape == (1, 4 * 18)
    v = ref.dequant_q4_0(packed, 1, 128).reshape(4, 32)
    assert np.array_equal(v[0], 0.5 * (codes[0].astype(np.float64) - 8))
    assert np.array_equal(v[1], (np.arange(32) % 16 - 8) * 2.0 ** -24)
    assert np.all(v[2] == 0.0)
    assert np.array_equal(v[3], np.tile([-8 * 65504.0, 7 * 65504.0], 16))
    # byte j of a block: input j in the low nibble, input j + 16 in the high one
    rng = np.random.default_rng(12)
    raw = rng.integers(0, 256, size=(3, 5 * 18), dtype=np.uint8)
    raw.reshape(3, 5, 18)[:, :, 0:2] = np.array([0.25], dtype=np.float16).view(np.uint8)   # finite scales
    v = ref.dequant_q4_0(raw, 3, 160)
    for r in range(3):
        for b in range(5):
            blk = raw[r, b * 18:(b + 1) * 18]
            d = float(blk[:2].view(np.float16)[0])
            for j in range(32):
                byte = int(blk[2 + (j % 16)])
                n = (byte & 15) if j < 16 else (byte >> 4)
                assert v[r, b * 32 + j] == d * (n - 8)
    # the fp16 weights: exact products stay exact; d * 7 may round
    b = ref.dequant_q4_0_f16_bits(packed, 1, 128).reshape(4, 32)
    assert np.array_equal(ref.f16_bits_to_f64(b[0]), 0.5 * (codes[0].astype(np.float64) - 8))
    assert b[3, 0] == 0xFC00 and b[3, 1] == 0x7C00        # -8 * 65504 and 7 * 65504 overflow


def test_bf16_rounding_matches_torch_and_neighbours():
    rng = np.random.default_rng(5)
    x32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-140, 100, 20000))).astype(np.float32)
    got = ref.f64_to_bf16_bits(x32.astype(np.float64))
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)
    # float64 inputs: the result is one of the two bf16 neighbours and the nearer one
    x = rng.standard_normal(20000) * 8
    b = ref.f64_to_bf16_bits(x)
    val = ref.bf16_bits_to_f64(b)
    up = ref.bf16_bits_to_f64((b.astype(np.int32) + 1).astype(np.uint16))
    dn = ref.bf16_bits_to_f64((b.astype(np.int32) - 1).astype(np.uint16))
    assert np.all(np.abs(val - x) <= np.abs(up - x)) and np.all(np.abs(val - x) <= np.abs(dn - x))
    # exact ties go to the even pattern: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert ref.f64_to_bf16_bits(np.array([1.0 + 2 ** -8]))[0] == 0x3F80
    assert ref.f64_to_bf16_bits(np.array([1.0 + 3 * 2 ** -8]))[0] == 0x3F82
    # a double-rounding trap: just above a bf16 tie, but an fp32 cast would land on the tie
    assert ref.f64_to_bf16_bits(np.array([1.0 + 2 ** -8 + 2 ** -40]))[0] == 0x3F81


# ------------------------------------------------------------------ RoPE and the cache write

def test_rope_low_frequency_angles_match_mla_card(golden):
    g = golden["rope_low_frequency_turn_degrees"]
    n_rot = golden["kv_geometry"]["rotary_dims"]
    inv = ref.rope_inv_freq(n_rot, 1.0e7)
    for tokens in (g["tokens"], 131000):
        deg = np.degrees(inv[-3:] * tokens)
        assert list(np.round(deg, g["printed_decimals"])) == g["degrees"]
    # base 1e6 or a 256-wide exponent denominator would not print these values
    assert list(np.round(np.degrees(ref.rope_inv_freq(n_rot, 1.0e6)[-3:] * g["tokens"]), 1)) != g["degrees"]
    inv256 = 1.0e7 ** (-2.0 * np.arange(32) / 256)
    assert list(np.round(np.degrees(inv256[-3:] * g["tokens"]), 1)) != g["degrees"]


def test_rope_rotation_properties():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 3, 256))
    pos = np.array([0, 1, 7, 1000, 65535, 131071])
    r = ref.rope_rotate(x, pos, 64, 1.0e7)
    assert np.array_equal(r[0], x[0])                         # position 0 is the identity
    assert np.array_equal(r[:, :, 64:], x[:, :, 64:])         # pass-through dims
    half = 32
    n0 = x[:, :, :half] ** 2 + x[:, :, half:64] ** 2
    n1 = r[:, :, :half] ** 2 + r[:, :, half:64] ** 2
    assert np.allclose(n0, n1, rtol=1e-12)                    # each pair keeps its norm
    # as complex numbers (a + i b) * exp(i theta)
    th = pos[:, None] * ref.rope_inv_freq(64, 1.0e7)[None, :]
    c = (x[:, :, :half] + 1j * x[:, :, half:64]) * np.exp(1j * th)[:, None, :]
    assert np.allclose(r[:, :, :half], c.real, atol=1e-12) and np.allclose(r[:, :, half:64], c.imag, atol=1e-12)
    # <R(p) q, R(p') k> depends only on p - p'
    q, k = rng.standard_normal((1, 256)), rng.standard_normal((1, 256))
    def dot(p, pp):
        return float(np.sum(ref.rope_rotate(q, np.array([p]), 64, 1e7) * ref.rope_rotate(k, np.array([pp]), 64, 1e7)))
    assert abs(dot(100, 37) - dot(1063, 1000)) < 1e-10


def test_k_norm_unit_gain_rms():
    rng = np.random.default_rng(2)
    kv = rng.standard_normal((5, 2048)) * 3.0
    k, v = ref.kv_write_values(kv, np.ones(256), pos0=0)
    ms = np.mean(kv[:, :1024].reshape(5, 4, 256) ** 2, axis=-1)
    rms = np.sqrt(np.mean(k ** 2, axis=-1))
    assert np.allclose(rms, np.sqrt(ms / (ms + 1e-6)), rtol=1e-12)   # RoPE keeps the RMS
    assert np.array_equal(v, kv[:, 1024:].reshape(5, 4, 256))


def test_paged_write_gathers_back_and_fills_each_slot_once():
    n_tok = 600
    gains, ptab, n_pages = synth.make_kv_write_inputs(n_tok, n_layers=1, n_pages=5)
    kv = synth.make_kv_rows(n_tok)
    poison = 0xFFFF
    kp = np.full((n_pages, 256, 4, 256), poison, dtype=np.uint16)
    vp = kp.copy()
    ref.kv_write(kv, gains[0], 0, ptab, kp, vp)
    k, v = ref.kv_write_values(kv, gains[0], 0)
    pos = np.arange(n_tok)
    assert np.array_equal(kp[ptab[pos // 256], pos % 256], ref.f64_to_bf16_bits(k))
    assert np.array_equal(vp[ptab[pos // 256], pos % 256], ref.f64_to_bf16_bits(v))
    used = np.zeros((n_pages, 256), dtype=bool)
    used[ptab[pos // 256], pos % 256] = True
    assert np.all(kp[~used] == poison) and not np.any(np.all(kp[used] == poison, axis=-1))


# ------------------------------------------------------------------ quantised KV cache (Hadamard + q8_0)

def test_hadamard_is_scipys_sylvester_matrix_and_an_orthogonal_involution():
    import scipy.linalg
    for n in (2, 8, 32, 256):
        H = ref.hadamard(n)
        assert np.array_equal(H, scipy.linalg.hadamard(n))          # library special case
        assert np.array_equal(H @ H.T, n * np.eye(n))
    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, 4, 256))
    y = ref.hadamard_rotate(x)
    assert np.allclose(ref.hadamard_rotate(y), x, rtol=0, atol=1e-13)     # involution
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
    # basis vectors: e_0 -> all 1/16, e_j -> row j of H / 16 (Sylvester order)
    e = np.zeros(256)
    e[0] = 1.0
    assert np.array_equal(ref.hadamard_rotate(e), np.full(256, 1.0 / 16))
    e[:] = 0
    e[5] = 1.0
    want = np.array([(-1.0) ** bin(i & 5).count("1") for i in range(256)]) / 16
    assert np.array_equal(ref.hadamard_rotate(e), want)
    # dot products survive the rotation (what lets attention use rotated K with rotated Q)
    a, b = rng.standard_normal(256), rng.standard_normal(256)
    assert abs(ref.hadamard_rotate(a) @ ref.hadamard_rotate(b) - a @ b) < 1e-12


def test_q8_0_quantize_hand_blocks():
    # amax 127 -> d = 1 exactly: the codes are the values rounded half away from zero
    y = np.zeros(64)
    y[:9] = [127, -127, 63.5, -63.5, 0.49, -2.5, 0.5, -0.5, 1.5]
    y[32:35] = [-3.0, 1.5, 0.75]            # second block: amax 3, d = 3/127
    d, q = ref.q8_0_quantize(y)
    assert d[0] == 0x3C00                    # fp16 1.0
    assert q[0, :9].tolist() == [127, -127, 64, -64, 0, -3, 1, -1, 2]
    assert not q[0, 9:].any()
    d1 = np.float32(3.0) / np.float32(127.0)
    assert d[1] == ref.f64_to_f16_bits(np.array([float(d1)]))[0]
    assert q[1, :3].tolist() == [-127, 64, 32]   # 1.5/d1 = 63.5 -> 64; 0.75/d1 = 31.75 -> 32
    # the code is decided on y times the block's reciprocal, not on y / d: with
    # amax 3 and y one ulp below fl32(2.5 d), y / d rounds to 2.5 but
    # y * fl32(1/d) = 2.4999998 in binary32, so the code is 2, not 3
    d3 = np.float32(3.0) / np.float32(127.0)
    y2 = np.zeros(32, np.float32)
    y2[0], y2[1] = 3.0, np.nextafter(np.float32(2.5) * d3, np.float32(0.0))
    assert y2[1] / d3 == np.float32(2.5) and y2[1] * (np.float32(1.0) / d3) < np.float32(2.5)
    _, q = ref.q8_0_quantize(y2.astype(np.float64))
    assert q[0, :2].tolist() == [127, 2]
    # an all-zero block has d = 0 and codes 0
    d, q = ref.q8_0_quantize(np.zeros(32))
    assert d[0] == 0 and not q.any()
    # packing: scale little-endian, then the codes as bytes; values d*q back
    d, q = ref.q8_0_quantize(y)
    b = ref.q8_0_block_bytes(d, q)
    assert b.shape == (68,) and b[0] == 0x00 and b[1] == 0x3C and b[2] == 127 and b[3] == 0x81
    vals = ref.q8_0_block_values(b)
    assert vals[0] == 127.0 and vals[3] == -64.0


def test_q8_0_quantize_error_bound_and_extremes():
    rng = np.random.default_rng(12)
    y = rng.standard_normal((400, 256)) * np.exp2(rng.integers(-6, 6, (400, 1)))
    d, q = ref.q8_0_quantize(y)
    blk = y.reshape(400, 8, 32)
    amax = np.abs(blk).max(-1)
    # the block's largest magnitude always maps to +-127
    assert np.all(np.abs(q).max(-1) == 127)
    # |fp16(d) q - y| <= d/2 (rounding) + |fp16(d) - d| * 127 (scale storage) + fp32 slack
    d32 = amax / 127.0
    d16 = ref.f16_bits_to_f64(d)
    err = np.abs(d16[..., None] * q - blk)
    bound = 0.5 * d32 + np.abs(d16 - d32) * 127 + 1e-6 * amax
    assert np.all(err <= bound[..., None])


def test_q8_0_kv_write_layout_and_rotation():
    n_tok = 300
    gains, ptab, n_pages = synth.make_kv_write_inputs(n_tok, n_layers=1, n_pages=3)
    kv = synth.make_kv_rows(n_tok)
    kp = np.full((n_pages, 256, 4, 8 * 34), 0xFF, dtype=np.uint8)
    vp = kp.copy()
    ref.kv_write_q8_0(kv, gains[0], 10, ptab, kp, vp)
    k, v = ref.kv_write_values(kv, gains[0], 10)
    pos = 10 + np.arange(n_tok)
    gk = ref.q8_0_block_values(kp[ptab[pos // 256], pos % 256])
    gv = ref.q8_0_block_values(vp[ptab[pos // 256], pos % 256])
    # rotating the dequantised rows back gives K and V within the q8_0 error
    for got, want in ((gk, k), (gv, v)):
        back = ref.hadamard_rotate(got)
        rms = np.sqrt(np.mean(want * want))
        assert np.max(np.abs(back - want)) / rms < 0.05
        assert np.sqrt(np.mean((back - want) ** 2)) / rms < 0.01
    used = np.zeros((n_pages, 256), dtype=bool)
    used[ptab[pos // 256], pos % 256] = True
    assert np.all(kp[~used] == 0xFF)


# ------------------------------------------------------------------ gated-DeltaNet state update

def test_deltanet_conv_matches_torch_conv1d():
    rng = np.random.default_rng(31)
    T, C = 9, 40
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, 4))
    st = rng.standard_normal((3, C))
    got, new = ref.causal_conv_silu(x, w, st)
    xp = torch.from_numpy(np.concatenate([st, x]).T[None])             # [1, C, T+3]
    conv = F.conv1d(xp, torch.from_numpy(w)[:, None, :], groups=C)     # library special case
    assert np.allclose(got, F.silu(conv)[0].T.numpy(), rtol=1e-13, atol=1e-13)
    assert np.array_equal(new, x[-3:])
    # fewer tokens than the window: the new state keeps older rows
    got2, new2 = ref.causal_conv_silu(x[:2], w, st)
    assert np.array_equal(new2, np.concatenate([st[2:], x[:2]]))


def test_deltanet_gates_and_norm_match_torch():
    rng = np.random.default_rng(32)
    z = rng.standard_normal(1000) * 30
    sp = F.softplus(torch.from_numpy(z)).numpy()        # torch returns x itself above x = 20
    lo = z <= 20
    assert np.allclose(ref.softplus(z[lo]), sp[lo], rtol=1e-13, atol=1e-300)
    assert np.all(np.abs(ref.softplus(z[~lo]) - z[~lo]) <= np.exp(-z[~lo]) + 1e-14 * z[~lo])
    assert np.allclose(ref.sigmoid(z), torch.sigmoid(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-300)
    k = rng.standard_normal((20, 16, 128))
    n = np.linalg.norm(ref.l2norm(k), axis=-1)
    assert np.allclose(n, 1.0, atol=1e-9)
    assert np.allclose(ref.l2norm(k), F.normalize(torch.from_numpy(k), dim=-1, eps=0).numpy(), rtol=1e-6)


def _random_scan_inputs(rng, T, n_v=6, n_k=2, d=8):
    k = ref.l2norm(rng.standard_normal((T, n_k, d)))
    v = rng.standard_normal((T, n_v, d))
    alpha = rng.uniform(0.5, 1.0, (T, n_v))
    beta = rng.uniform(0.0, 1.0, (T, n_v))
    S0 = rng.standard_normal((n_v, d, d))
    return S0, k, v, alpha, beta


def test_gated_delta_scan_equals_product_of_transitions():
    """Closed form of the recurrence: S_T = S_0 M_1 ... M_T + sum_t beta_t v_t
    k_t^T M_{t+1} ... M_T with M_t = alpha_t (I - beta_t k_t k_t^T), built by
    explicit matrix products (value head h reads key head h // 3)."""
    rng = np.random.default_rng(33)
    T, d = 7, 8
    S0, k, v, alpha, beta = _random_scan_inputs(rng, T, d=d)
    got = ref.gated_delta_scan(S0, k, v, alpha, beta, group=3)
    for h in range(6):
        M = [alpha[t, h] * (np.eye(d) - beta[t, h] * np.outer(k[t, h // 3], k[t, h // 3])) for t in range(T)]
        want = S0[h].copy()
        for t in range(T):
            want = want @ M[t]
        for t in range(T):
            tail = np.eye(d)
            for s in range(t + 1, T):
                tail = tail @ M[s]
            want += beta[t, h] * np.outer(v[t, h], k[t, h // 3]) @ tail
        assert np.allclose(got[h], want, rtol=1e-12, atol=1e-12)


def test_gated_delta_scan_closed_cases():
    rng = np.random.default_rng(34)
    S0, k, v, alpha, beta = _random_scan_inputs(rng, 5)
    # beta = 0: pure decay
    got = ref.gated_delta_scan(S0, k, v, alpha, np.zeros_like(beta))
    assert np.allclose(got, S0 * np.prod(alpha, axis=0)[:, None, None], rtol=1e-13)
    # alpha = beta = 1 with orthonormal keys from a zero state: the state
    # stores every association exactly, S k_i = v_i
    d, n = 16, 10
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Q[:n][:, None, :]                                 # [n, 1 key head, d]
    vals = rng.standard_normal((n, 3, d))
    S = ref.gated_delta_scan(np.zeros((3, d, d)), keys, vals, np.ones((n, 3)), np.ones((n, 3)))
    for i in range(n):
        assert np.allclose(S @ keys[i, 0], vals[i], atol=1e-12)
    # one token: S_1 = alpha S_0 - alpha beta S_0 k k^T + beta v k^T
    one = ref.gated_delta_scan(S0, k[:1], v[:1], alpha[:1], beta[:1])
    kk = k[0][np.arange(6) // 3]
    want = (alpha[0][:, None, None] * (S0 - beta[0][:, None, None] * np.einsum("hvk,hk,hj->hvj", S0, kk, kk))
            + beta[0][:, None, None] * np.einsum("hv,hk->hvk", v[0], kk))
    assert np.allclose(one, want, rtol=1e-13, atol=1e-13)


def test_deltanet_update_splits_at_any_token():
    """Carrying the conv state and the recurrent state across calls gives the
    same result as one call (the update is a sequential recurrence)."""
    conv_w, a_log, dt_bias = synth.make_deltanet_params(1)
    conv0, S0 = synth.make_deltanet_state(1)
    rows = synth.make_deltanet_rows(40)
    S_all, c_all = ref.deltanet_update(rows, conv_w[0], a_log[0], dt_bias[0], conv0[0], S0[0])
    S_a, c_a = ref.deltanet_update(rows[:17], conv_w[0], a_log[0], dt_bias[0], conv0[0], S0[0])
    S_b, c_b = ref.deltanet_update(rows[17:], conv_w[0], a_log[0], dt_bias[0], c_a, S_a)
    assert np.allclose(S_b, S_all, rtol=1e-12, atol=1e-14) and np.array_equal(c_b, c_all)
    # widths: q | k | v = 2048 | 2048 | 6144 and a, b = 48 each
    assert ref.DN_QKV == 2 * ref.DN_NK * ref.DN_HD + ref.DN_NV * ref.DN_HD == 10240
    assert rows.shape[1] == 10240 + 48 + 48


def _prepare_by_loops(m, conv_w, a_log, dt_bias, conv_state, n_k, n_v, hd):
    """The DeltaNet preparation written out element by element from its
    definition (the readings in the oracle's DeltaNet section): columns
    q | k | v | a | b; a width-4 causal depthwise conv over the raw q|k|v rows
    (the carried rows first), SiLU, each key head divided by
    sqrt(|k|^2 + 1e-6), value heads as they are, and per value head
    alpha = exp(-exp(A_log) * ln(1 + e^(a + dt_bias))), beta = 1 / (1 + e^-b)."""
    T = m.shape[0]
    C = (2 * n_k + n_v) * hd
    W = conv_w.shape[1]
    rows = [list(map(float, r)) for r in conv_state] + [list(map(float, r[:C])) for r in m]
    act = [[0.0] * C for _ in range(T)]
    for t in range(T):
        for c in range(C):
            acc = 0.0
            for tau in range(W):
                acc += float(conv_w[c][tau]) * rows[t + tau][c]
            act[t][c] = acc / (1.0 + math.exp(-acc))
    k = np.zeros((T, n_k, hd))
    v = np.zeros((T, n_v, hd))
    alpha = np.zeros((T, n_v))
    beta = np.zeros((T, n_v))
    for t in range(T):
        for j in range(n_k):
            col0 = n_k * hd + j * hd
            nrm = math.sqrt(sum(act[t][col0 + e] ** 2 for e in range(hd)) + 1e-6)
            for e in range(hd):
                k[t, j, e] = act[t][col0 + e] / nrm
        for h in range(n_v):
            for e in range(hd):
                v[t, h, e] = act[t][2 * n_k * hd + h * hd + e]
            a = float(m[t, C + h])
            b = float(m[t, C + n_v + h])
            alpha[t, h] = math.exp(-math.exp(float(a_log[h])) * math.log1p(math.exp(a + float(dt_bias[h]))))
            beta[t, h] = 1.0 / (1.0 + math.exp(-b))
    new_conv = np.array(rows[T:], dtype=np.float64)
    return k, v, alpha, beta, new_conv


def _small_deltanet_case(seed=71, T=6, n_k=2, n_v=6, hd=4):
    rng = np.random.default_rng(seed)
    C = (2 * n_k + n_v) * hd
    m = rng.standard_normal((T, C + 2 * n_v)) * 2.0
    conv_w = rng.standard_normal((C, 4)) * 0.5
    a_log = rng.uniform(-2.0, 1.0, n_v)
    dt_bias = rng.standard_normal(n_v)
    conv_state = rng.standard_normal((3, C))
    return m, conv_w, a_log, dt_bias, conv_state, n_k, n_v, hd


def _prepare_deviation(fn, case):
    got = fn(*case)
    want = _prepare_by_loops(*case)
    return max(float(np.max(np.abs(np.asarray(g, dtype=np.float64) - w))) for g, w in zip(got, want))


def test_deltanet_prepare_matches_elementwise_definition():
    """Slices (q | k | v | a | b), conv, norm and gates against the scalar
    definition on a small layer (2 key heads, 6 value heads of 4 dims)."""
    case = _small_deltanet_case()
    assert _prepare_deviation(ref.deltanet_prepare, case) < 1e-12


def test_deltanet_prepare_hand_values():
    """Gates at hand-computable points: a + dt_bias = 0 makes softplus ln 2, so
    alpha = 2^(-exp(A_log)): 1/2 at A_log = 0, 1/4 at A_log = ln 2; beta is
    1/2 at b = 0 and 3/4 at b = ln 3.  With conv weights (0, 0, 0, 1) the
    conv is the identity, so k is the l2-normed SiLU of the k columns alone
    (q columns hold other values) and v the SiLU of the v columns."""
    n_k, n_v, hd, T = 1, 2, 4, 2
    C = (2 * n_k + n_v) * hd
    m = np.zeros((T, C + 2 * n_v))
    m[:, :hd] = 7.0                                          # q: must not leak into k
    m[:, hd:2 * hd] = [[1.0, 2.0, 3.0, 4.0], [-1.0, 0.5, 0.0, 2.0]]
    m[:, 2 * hd:C] = np.arange(T * n_v * hd).reshape(T, n_v * hd) / 10.0 - 1.0
    dt_bias = np.array([0.3, -1.2])
    m[:, C:C + n_v] = -dt_bias                               # a + dt_bias = 0
    m[0, C + n_v:] = [0.0, math.log(3.0)]
    m[1, C + n_v:] = [math.log(3.0), 0.0]
    conv_w = np.tile([0.0, 0.0, 0.0, 1.0], (C, 1))
    a_log = np.array([0.0, math.log(2.0)])
    k, v, alpha, beta, new_conv = ref.deltanet_prepare(m, conv_w, a_log, dt_bias, np.zeros((3, C)), n_k, n_v, hd)
    assert np.allclose(alpha, [[0.5, 0.25], [0.5, 0.25]], rtol=1e-14)
    assert np.allclose(beta, [[0.5, 0.75], [0.75, 0.5]], rtol=1e-14)
    silu = lambda z: z / (1.0 + np.exp(-z))
    kk = silu(m[:, hd:2 * hd])
    assert np.allclose(k[:, 0, :], kk / np.sqrt(np.sum(kk ** 2, axis=1, keepdims=True) + 1e-6), rtol=1e-14)
    assert np.allclose(v.reshape(T, -1), silu(m[:, 2 * hd:C]), rtol=1e-14)
    assert np.array_equal(new_conv[1:], m[:, :C]) and np.array_equal(new_conv[0], np.zeros(C))


def _prep_swapped_ab(m, conv_w, a_log, dt_bias, conv_state, n_k, n_v, hd):
    C = (2 * n_k + n_v) * hd
    m2 = m.copy()
    m2[:, C:C + n_v], m2[:, C + n_v:C + 2 * n_v] = m[:, C + n_v:C + 2 * n_v], m[:, C:C + n_v]
    return ref.deltanet_prepare(m2, conv_w, a_log, dt_bias, conv_state, n_k, n_v, hd)


def _prep_gate_sign(*case):
    k, v, alpha, beta, c = ref.deltanet_prepare(*case)
    return k, v, 1.0 / alpha, beta, c                       # exp(+exp(A_log) softplus(.))


def _prep_k_from_q(m, conv_w, a_log, dt_bias, conv_state, n_k, n_v, hd):
    m2, cs2, w2 = m.copy(), conv_state.copy(), conv_w.copy()
    m2[:, n_k * hd:2 * n_k * hd] = m[:, :n_k * hd]
    cs2[:, n_k * hd:2 * n_k * hd] = conv_state[:, :n_k * hd]
    w2[n_k * hd:2 * n_k * hd] = conv_w[:n_k * hd]
    k, v, alpha, beta, _ = ref.deltanet_prepare(m2, w2, a_log, dt_bias, cs2, n_k, n_v, hd)
    return k, v, alpha, beta, ref.deltanet_prepare(m, conv_w, a_log, dt_bias, conv_state, n_k, n_v, hd)[4]


@pytest.mark.parametrize("mutant", [_prep_swapped_ab, _prep_gate_sign, _prep_k_from_q])
def test_deltanet_prepare_planted_mistakes_are_caught(mutant):
    """a and b swapped, the sign of the log-decay flipped, k read from the q
    columns: each moves some output far off the elementwise definition."""
    assert _prepare_deviation(mutant, _small_deltanet_case()) > 1e-3


# ------------------------------------------------------------------ single-map projector

def test_map_project_matches_torch_linear_and_closed_cases():
    rng = np.random.default_rng(51)
    n = 64
    maps, biases = synth.make_map_weights(n, 3, "f32")
    x = synth.make_map_input(10, n)
    got = ref.map_project(x, maps, biases)
    for i in range(3):                                            # library special case
        want = F.linear(torch.from_numpy(x.astype(np.float64)), torch.from_numpy(maps[i].astype(np.float64)),
                        torch.from_numpy(biases[i].astype(np.float64))).numpy()
        assert np.allclose(got[i], want, rtol=1e-12, atol=1e-12)
    # zero input gives the bias; the identity map gives the input back
    z = ref.map_project(np.zeros((2, n)), maps, biases)
    assert all(np.array_equal(z[i], np.tile(biases[i].astype(np.float64), (2, 1))) for i in range(3))
    eye = ref.map_project(x, [np.eye(n, dtype=np.float32)])[0]
    assert np.array_equal(eye, x.astype(np.float64))
    # stored formats decode through the weight readers: a bf16 map equals its decoded values
    wb = synth.make_map_weights(n, 1, "bf16", bias=False)[0][0]
    assert np.allclose(ref.map_project(x, [wb], dtype="bf16")[0],
                       x.astype(np.float64) @ ref.bf16_bits_to_f64(wb).reshape(n, n).T, rtol=1e-13)
    assert synth.map_layers(12) == 51 and synth.map_layers(24) == 39


# ------------------------------------------------------------------ planted mistakes

def _mutants():
    orig_attn, orig_norm = ref.causal_attention, ref.rmsnorm

    def no_mask(q, k, v, H, hd):
        out = np.empty_like(q)
        for h in range(H):
            c = slice(h * hd, (h + 1) * hd)
            s = q[:, c] @ k[:, c].T / math.sqrt(hd)
            p = np.exp(s - s.max(1, keepdims=True))
            out[:, c] = (p / p.sum(1, keepdims=True)) @ v[:, c]
        return out

    def doubled_scale(q, k, v, H, hd):
        return orig_attn(q * 2.0, k, v, H, hd)

    def sum_not_mean(x, g, eps):
        x = np.asarray(x, dtype=np.float64)
        return x / np.sqrt(np.sum(x * x, -1, keepdims=True) + eps) * g

    def norm_no_gain(x, g, eps):
        return orig_norm(x, np.ones_like(g), eps)

    def silu_sign(x):
        return x / (1.0 + np.exp(x))

    return {"unmasked attention": ("causal_attention", no_mask),
            "doubled score scale": ("causal_attention", doubled_scale),
            "norm uses sum": ("rmsnorm", sum_not_mean),
            "norm without gain": ("rmsnorm", norm_no_gain),
            "silu sign": ("silu", silu_sign)}


@pytest.mark.parametrize("which", list(_mutants()))
def test_planted_mistakes_are_caught(monkeypatch, which):
    name, fn = _mutants()[which]
    monkeypatch.setattr(ref, name, fn)
    cfg = synth.config("tiny")
    w, x = synth.make_weights(cfg), synth.make_input(cfg, n_tokens=24)
    got = ref.project(cfg, w, x)
    want = _torch_projector(cfg, w, x)
    worst = max(np.max(np.abs(got[i] - y)) / np.sqrt(np.mean(y * y)) for i, y in enumerate(want))
    assert worst > 1e-6, which


def test_planted_transposed_weight_is_caught(monkeypatch):
    orig = ref.prepare

    def transposed(cfg, w):
        p = orig(cfg, w)
        p["blocks"][1]["wq"] = p["blocks"][1]["wq"].T.copy()
        return p
    monkeypatch.setattr(ref, "prepare", transposed)
    cfg = synth.config("tiny")
    w, x = synth.make_weights(cfg), synth.make_input(cfg, n_tokens=24)
    got = ref.project(cfg, w, x)
    want = _torch_projector(cfg, w, x)
    assert max(np.max(np.abs(got[i] - y)) for i, y in enumerate(want)) > 1e-6
