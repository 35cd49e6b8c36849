"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/kva.h declares, validates configs, and its host-side
weight conversion and head packing are right."""
import ctypes

import numpy as np
import pytest

import learned_kv_approximation_amd as kva
import synth
from oracle import ref


def test_library_exports_every_declared_function():
    names = kva.header_exports()
    assert {"kva_create", "kva_project_ubatch", "kva_destroy", "kva_attn_kv_write"} <= set(names)
    L = kva.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(kva._SIGS), "binding signatures out of step with the header"


def test_status_strings_and_null_safety():
    L = kva.lib()
    for s in range(8):
        assert L.kva_status_str(s).decode().startswith("KVA_")
    assert kva.lib().kva_destroy(None) == kva.KVA_OK
    assert L.kva_project_ubatch(None, None, 1, None, None) == kva.KVA_ERR_ARG
    assert b"NULL" in L.kva_last_error()


@pytest.mark.parametrize("name", ["tiny", "r2", "r3"])
def test_validate_accepts_page_configs(name):
    c, keep = kva.make_config(synth.config(name))
    assert kva.kva_validate_config(c) == kva.KVA_OK


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, kva.KVA_ERR_SHAPE),
    ("n_heads", 3, kva.KVA_ERR_SHAPE),
    ("d_ffn", 7000, kva.KVA_ERR_SHAPE),
    ("attn_block", 1000, kva.KVA_ERR_SHAPE),
    ("max_tokens", 0, kva.KVA_ERR_SHAPE),
    ("weight_dtype", 9, kva.KVA_ERR_DTYPE),
    ("n_out_heads", 0, kva.KVA_ERR_SHAPE),
    ("n_out_heads", 65, kva.KVA_ERR_SHAPE),
    ("has_head_bias", 2, kva.KVA_ERR_ARG),
])
def test_validate_rejects(field, value, status):
    c, keep = kva.make_config(synth.config("r2"))
    setattr(c, field, value)
    assert kva.kva_validate_config(c) == status
    assert kva.lib().kva_last_error()


def test_validate_rejects_bad_head():
    cfg = synth.config("tiny")
    cfg["heads"][1]["out_dim"] = 0
    c, keep = kva.make_config(cfg)
    assert kva.kva_validate_config(c) == kva.KVA_ERR_SHAPE


@pytest.mark.parametrize("name", ["tiny", "r2", "r3"])
def test_head_plan_is_a_tiled_bijection(name):
    cfg = synth.config(name)
    c, keep = kva.make_config(cfg)
    head, idx = kva.kva_debug_head_plan(c)
    assert head.size % 256 == 0
    seen = set()
    for h, i in zip(head.tolist(), idx.tolist()):
        if h < 0:
            continue
        assert 0 <= i < cfg["heads"][h]["out_dim"]
        seen.add((h, i))
    assert len(seen) == sum(h["out_dim"] for h in cfg["heads"])
    assert np.count_nonzero(head >= 0) == len(seen)
    # every 256-column tile outside the tail belongs to a single head
    tiles = head.reshape(-1, 256)
    full = [t for t in tiles if np.all(t == t[0]) and t[0] >= 0]
    assert len(full) == sum(h["out_dim"] // 256 for h in cfg["heads"])
    if name == "r2":
        assert head.size == 264448 + 0   # 24 * 96 a|b columns fill 9 tiles exactly


def test_host_f16_conversion_matches_numpy():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-30, 17, 200000))).astype(np.float32)
    x = x[np.abs(x) < 65504]
    st, got = kva.kva_debug_host_to_f16(x, "f32")
    assert st == kva.KVA_OK
    assert np.array_equal(got, x.astype(np.float16).view(np.uint16))
    b = synth.f32_to_bf16_bits(x[np.abs(x) < 65280])   # bf16 rounding must stay finite in fp16
    st, got = kva.kva_debug_host_to_f16(b, "bf16")
    bf = (b.astype(np.uint32) << 16).view(np.float32)
    assert st == kva.KVA_OK and np.array_equal(got, bf.astype(np.float16).view(np.uint16))
    # ties and the overflow edge
    edge = np.array([65504.0, 65519.99, 65520.0, -70000.0, 2.0 ** -25, 3 * 2.0 ** -26, 1.0 + 2 ** -11],
                    dtype=np.float32)
    st, got = kva.kva_debug_host_to_f16(edge, "f32")
    assert st == kva.KVA_ERR_RANGE
    with np.errstate(over="ignore"):
        assert np.array_equal(got, edge.astype(np.float16).view(np.uint16))


def test_create_without_device_fails_cleanly():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    cfg = synth.config("tiny")
    w = synth.make_weights(cfg)
    c, k1 = kva.make_config(cfg)
    s, k2 = kva.make_weights(cfg, w)
    out = ctypes.c_void_p()
    st = kva.lib().kva_create(ctypes.byref(c), ctypes.byref(s), 0, ctypes.byref(out))
    assert st in (kva.KVA_ERR_HIP, kva.KVA_ERR_OOM) and out.value is None


def test_truncating_round_half_away_identity():
    """The q8_0 KV kernels round t = y * (1/d) half away from zero as
    trunc(t + copysign(pred(1/2), t)) in binary32 (one add, no roundf): check
    that identity against an exact rounding on every binary32 value near the
    half-integers of [-128, 128] (each k + 1/2 and 40 neighbours either side),
    on the values just below 1/2, and on random draws."""
    h = np.nextafter(np.float32(0.5), np.float32(0.0))
    pts = []
    for k in range(-128, 128):
        c = np.float32(k + 0.5)
        v = c
        for _ in range(40):
            v = np.nextafter(v, np.float32(-np.inf))
            pts.append(v)
        v = c
        for _ in range(40):
            v = np.nextafter(v, np.float32(np.inf))
            pts.append(v)
        pts.append(c)
    x = np.concatenate([np.array(pts, np.float32),
                        np.float32([h, -h, 0.0, -0.0, 1e-30, -1e-30, 0.25, 0.75]),
                        np.random.default_rng(3).uniform(-128, 128, 200000).astype(np.float32)])
    got = np.trunc((x + np.copysign(h, x)).astype(np.float32)).astype(np.float64)
    xd = x.astype(np.float64)
    want = np.sign(xd) * np.floor(np.abs(xd) + 0.5)       # exact in float64
    assert np.array_equal(got, want)


def test_build_commands_keep_packed_fp32_off():
    """Every HIP source is compiled for gfx950 with the packed fp32 VALU
    feature disabled (the compiler would otherwise form packed adds and
    multiplies from scalar float code); only the attention source asks for
    VGPR-form MFMAs, and the link step names every object."""
    from learned_kv_approximation_amd import _build
    objs = []
    for src in _build.SOURCES:
        cmd = _build.compile_command(src, src + ".o")
        assert "--offload-arch=gfx950" in cmd and "-O3" in cmd and "-c" in cmd
        i = cmd.index("-packed-fp32-ops")
        assert cmd[i - 3:i] == ["-Xclang", "-target-feature", "-Xclang"]
        assert ("-amdgpu-mfma-vgpr-form" in cmd) == (src == "kva_attn.hip")
        objs.append(src + ".o")
    link = _build.link_command(objs, "lib.so")
    assert "-shared" in link and all(o in link for o in objs) and link[-2:] == ["-o", "lib.so"]


# ------------------------------------------------------------------ weight packing (host only)

def _t32_index(r, k, K):
    """Element index of (row r, K-value k) in the 16-bit device layout: 256-row
    groups, 32-wide K slabs, 64-byte rows, 16-byte chunk c at c ^ ((r >> 2) & 3)."""
    nb, rr, kt = r // 256, r % 256, k // 32
    c, e = (k % 32) // 8, k % 8
    return ((nb * (K // 32) + kt) * 256 + rr) * 32 + ((c ^ ((rr >> 2) & 3)) * 8) + e


@pytest.mark.parametrize("target", ["f16", "bf16"])
def test_pack_weight_16bit_layout(target):
    rng = np.random.default_rng(61)
    rows, K = 300, 96
    w = (rng.standard_normal((rows, K)) * 0.1).astype(np.float32)
    st, out, _ = kva.kva_debug_pack_weight(w, "f32", rows, K, target)
    assert st == kva.KVA_OK
    got = out.view(np.uint16)
    want = (np.float16 if target == "f16" else None)
    r, k = np.meshgrid(np.arange(512), np.arange(K), indexing="ij")
    idx = _t32_index(r, k, K)
    assert np.unique(idx).size == idx.size == got.size            # a permutation of the buffer
    if target == "f16":
        vals = np.zeros((512, K), dtype=np.float16)
        vals[:rows] = w.astype(np.float16)
        assert np.array_equal(got[idx], vals.view(np.uint16))
    else:
        bits = np.zeros((512, K), dtype=np.uint16)
        bits[:rows] = synth.f32_to_bf16_bits(w)
        assert np.array_equal(got[idx], bits)


def test_pack_weight_q8_0_planes():
    rng = np.random.default_rng(62)
    rows, K = 260, 64
    codes = rng.integers(-128, 128, size=(rows, K), dtype=np.int8)
    sc = (np.abs(rng.standard_normal((rows, K // 32))) * 1e-3).astype(np.float16)
    blocks = synth.pack_q8_0(codes, sc)
    st, out, scales = kva.kva_debug_pack_weight(blocks, "q8_0", rows, K, "q8_0")
    assert st == kva.KVA_OK
    for r in (0, 1, 5, 37, 255, 256, 259, 300, 511):
        for b in range(K // 32):
            nb, rr = r // 256, r % 256
            si = (nb * (K // 32) + b) * 256 + rr
            want_d = sc[r, b].view(np.uint16) if r < rows else 0
            assert scales[si] == want_d, (r, b)
            for c in range(4):
                off = ((nb * (K // 32) + b) * 256 + rr) * 32 + ((c ^ ((rr >> 2) & 3)) * 8)
                chunk = out[off:off + 8]
                q = codes[r, b * 32 + 8 * c: b * 32 + 8 * c + 8] if r < rows else np.zeros(8, np.int8)
                biased = (q.view(np.uint8) ^ 0x80)
                # each 32-bit half holds codes 4j, 4j+2, 4j+1, 4j+3 in its bytes
                order = [0, 2, 1, 3, 4, 6, 5, 7]
                assert np.array_equal(chunk, biased[order]) if r < rows else np.all(chunk == 0), (r, b, c)


def test_pack_weight_q4_0_planes_and_range():
    rng = np.random.default_rng(63)
    rows, K = 256, 64
    n = rng.integers(0, 16, size=(rows, K)).astype(np.uint8)
    sc = (np.abs(rng.standard_normal((rows, K // 32))) * 1e-3).astype(np.float16)
    blocks = synth.pack_q4_0(n, sc)
    st, out, scales = kva.kva_debug_pack_weight(blocks, "q4_0", rows, K, "q4_0")
    assert st == kva.KVA_OK
    for r in (0, 3, 8, 100, 255):
        for b in range(K // 32):
            for c in range(4):
                off = ((b) * 256 + r) * 16 + ((c ^ ((r >> 3) & 3)) * 4)
                wv = int(out[off:off + 4].view(np.uint32)[0])
                for e in range(8):
                    h, hi = e // 2, e % 2
                    got = (wv >> (16 * hi + 4 * h)) & 0xF
                    assert got == n[r, b * 32 + 8 * c + e], (r, b, c, e)
    # a scale whose weights overflow fp16 is refused
    bad = blocks.copy().reshape(rows, -1)
    bad[7, 0:2] = np.array([0x7BFF], dtype=np.uint16).view(np.uint8)
    bad[7, 2] = 0x00                                  # code 0 -> n - 8 = -8
    st, _, _ = kva.kva_debug_pack_weight(bad, "q4_0", rows, K, "q4_0")
    assert st == kva.KVA_ERR_RANGE


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0"])
def test_pack_weight_quantised_expanded_to_fp16(fmt):
    """Contexts of more than 256 tokens per call hold q8_0 / q4_0 weights
    expanded to fp16 at create: every value must be the oracle's fp16(d * code)
    (the weight the in-register dequantisation forms), in the 16-bit layout,
    including subnormal and zero scales, q = -128 and padding rows."""
    rng = np.random.default_rng(64)
    rows, K = 300, 96
    nb = K // 32
    sc = (np.abs(rng.standard_normal((rows, nb))) * 1e-3).astype(np.float16)
    sc[3, 0] = np.float16(3e-7)                       # subnormal scale
    sc[4, 1] = np.float16(0.0)
    sc[5, 2] = np.float16(-0.02)
    if fmt == "q8_0":
        codes = rng.integers(-128, 128, size=(rows, K), dtype=np.int8)
        codes[6, :32] = -128
        blocks = synth.pack_q8_0(codes, sc)
        want16 = ref.dequant_q8_0_f16_bits(blocks, rows, K)
    else:
        n = rng.integers(0, 16, size=(rows, K)).astype(np.uint8)
        blocks = synth.pack_q4_0(n, sc)
        want16 = ref.dequant_q4_0_f16_bits(blocks, rows, K)
    st, out, _ = kva.kva_debug_pack_weight(blocks, fmt, rows, K, "f16")
    assert st == kva.KVA_OK
    got = out.view(np.uint16)
    r, k = np.meshgrid(np.arange(512), np.arange(K), indexing="ij")
    bits = np.zeros((512, K), dtype=np.uint16)
    bits[:rows] = np.asarray(want16, dtype=np.uint16).reshape(rows, K)
    assert np.array_equal(got[_t32_index(r, k, K)], bits)
