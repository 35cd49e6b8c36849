"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bar (per head): max|y_gpu - y_oracle| <= 2e-2 * RMS(y_oracle) for 16-bit
weights, and bitwise equality for the block-structure invariants (a block's
outputs do not depend on other blocks or on later tokens), the q8_0
dequantisation hook, and determinism.  The KV-cache write must land within
one bf16 ulp of the oracle's correctly rounded value plus the fp32
rotation's absolute error (2^-20 of the rotary pair's norm); V bit-exact.
"""
import concurrent.futures
import os

import numpy as np
import pytest
import torch

import learned_kv_approximation_amd as kva
import oracle
import synth
from oracle import emu, ref

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(proj, x):
    outs = proj.project(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def _errs(got, want):
    out = {}
    for i, y in want.items():
        g = got[i].astype(np.float64)
        rms = np.sqrt(np.mean(y * y))
        out[i] = (float(np.max(np.abs(g - y)) / rms), float(np.sqrt(np.mean((g - y) ** 2)) / rms))
    return out


def _check(cfg, got, want, tol=TOL, label=""):
    errs = _errs(got, want)
    worst = max(e[0] for e in errs.values())
    print(f"{label} worst max|err|/rms {worst:.4e}; sigma max {max(e[1] for e in errs.values()):.4e}", flush=True)
    bad = {cfg["heads"][i]["name"]: e for i, e in errs.items() if not e[0] <= tol}
    assert not bad, bad


# ------------------------------------------------------------------ tiny config

@pytest.fixture(scope="module")
def tiny():
    cfg = synth.config("tiny")
    return cfg, synth.make_weights(cfg)


def test_tiny_parity(tiny):
    cfg, w = tiny
    x = synth.make_input(cfg)
    proj = kva.Projector(cfg, w, max_tokens=64)
    _check(cfg, _run(proj, x), oracle.project(cfg, w, x), label="tiny")
    proj.close()


def test_tiny_trunk_state_matches_oracle(tiny):
    cfg, w = tiny
    x = synth.make_input(cfg)
    proj = kva.Projector(cfg, w, max_tokens=64)
    _run(proj, x)
    z = proj.copy_z(64).cpu().numpy().view(np.uint16)
    zg = ref.bf16_bits_to_f64(z)
    zr = ref.trunk(cfg, ref.prepare(cfg, w), x)
    err = np.max(np.abs(zg - zr)) / np.sqrt(np.mean(zr ** 2))
    print("tiny z max|err|/rms", err)
    assert err < 2e-2
    proj.close()


@pytest.mark.parametrize("dtype", ["f32", "q8_0", "q4_0"])
def test_tiny_skinny_context(dtype):
    """A context of at most 32 tokens per call runs every trunk GEMM on the
    skinny kernel (K split over the waves of a workgroup, the N = d GEMMs
    also over 4 workgroups; half its waves get no K slab at the tiny
    widths): oracle parity (the q8_0 / q4_0 bar for quantised weights) and
    a call's rows bit for bit those of a longer call."""
    cfg = synth.config("tiny", weight_dtype=dtype)
    w = synth.make_weights(cfg)
    proj = kva.Projector(cfg, w, max_tokens=32)
    x = synth.make_input(cfg, n_tokens=32, seed=41)
    full = _run(proj, x)
    _check(cfg, full, oracle.project(cfg, w, x), tol=TOL if dtype == "f32" else 5e-2, label=f"tiny {dtype} skinny")
    for n in (1, 17):
        part = _run(proj, np.ascontiguousarray(x[:n]))
        for i in range(len(part)):
            assert np.array_equal(part[i], full[i][:n]), (dtype, n, i)
    proj.close()


@pytest.mark.parametrize("n", [1, 63, 65, 200])
def test_tiny_ragged_blocks(tiny, n):
    cfg, w = tiny
    cfg = dict(cfg, attn_block=64)
    x = synth.make_input(cfg, n_tokens=n, seed=11)
    proj = kva.Projector(cfg, w, max_tokens=256)
    _check(cfg, _run(proj, x), oracle.project(cfg, w, x), label=f"tiny n={n}")
    proj.close()


def _jitter_spread(cfg, w, x, base, trials=3, rel=1e-7):
    """How far the emulator moves when its input moves by fp32-size noise:
    the worst (max|diff|/rms, rms diff/rms) over `trials` relative jitters of
    x by rel * N(0, 1)."""
    rng = np.random.default_rng(1234)
    mx, sd = 0.0, 0.0
    for _ in range(trials):
        xj = x.astype(np.float64) * (1.0 + rel * rng.standard_normal(x.shape))
        e = _errs(emu.project(cfg, w, xj), base)
        mx = max(mx, max(v[0] for v in e.values()))
        sd = max(sd, max(v[1] for v in e.values()))
    return mx, sd


@pytest.mark.parametrize("scale", [1.0, 3.0])
def test_tiny_long_block_peaked_scores(tiny, scale):
    """1024 tokens in one attention block (16 key tiles per query tile) with
    the Q and K weights scaled by `scale` (scores x scale^2).  At 3 the
    running maximum of a query jumps by several units between key tiles, so
    the softmax rescale of the output accumulators runs on non-empty state
    (with unscaled weights it runs only on the first tile).

    Bar at scale 1: the projector's (max|err| <= 2e-2 RMS against the
    oracle).  At scale 3 the block is numerically chaotic: the rounding-point
    emulator (oracle/emu.py: every intermediate the kernels store rounded to
    its format, float64 arithmetic otherwise) is 0.195 RMS away from the
    oracle at most (the GPU: 0.190), and it moves by 0.03-0.04 RMS when its
    input is jittered by 1e-7 relative, the size of fp32 arithmetic noise.
    So at scale 3 the GPU is held to the emulator within 1.5x that measured
    spread (max and RMS; a rescale that dropped or misapplied its factor
    would move whole rows by O(1)), and to the oracle by the RMS error
    (<= 2e-2)."""
    cfg, w = tiny
    cfg = dict(cfg, attn_block=1024)
    w = dict(w, blocks=[dict(b, wq=b["wq"] * np.float32(scale), wk=b["wk"] * np.float32(scale))
                        for b in w["blocks"]])
    x = synth.make_input(cfg, n_tokens=1024, seed=12)
    proj = kva.Projector(cfg, w, max_tokens=1024)
    got, want = _run(proj, x), oracle.project(cfg, w, x)
    proj.close()
    emulated = emu.project(cfg, w, x)
    ee = _errs(got, emulated)
    gm, gs = max(e[0] for e in ee.values()), max(e[1] for e in ee.values())
    print(f"tiny 1024 tokens, qk scale {scale}: vs emulator worst max|err|/rms {gm:.4e}, rms {gs:.4e}", flush=True)
    if scale == 1.0:
        _check(cfg, got, want, label="tiny 1024 tokens")
        _check(cfg, got, emulated, label="tiny 1024 tokens vs emulator")
        return
    errs = _errs(got, want)
    print(f"tiny 1024 tokens, qk scale {scale}: vs oracle worst max|err|/rms "
          f"{max(e[0] for e in errs.values()):.4e}; rms err/rms {max(e[1] for e in errs.values()):.4e}", flush=True)
    assert all(e[1] <= 2e-2 for e in errs.values()), errs
    sm, ss = _jitter_spread(cfg, w, x, emulated)
    print(f"  emulator spread under 1e-7 input jitter: max {sm:.4e}, rms {ss:.4e}", flush=True)
    assert gm <= max(TOL, 1.5 * sm) and gs <= 1.5 * ss, (gm, gs, sm, ss)


def test_tiny_bad_arguments(tiny):
    cfg, w = tiny
    proj = kva.Projector(cfg, w, max_tokens=64)
    x = torch.zeros((65, cfg["n_in"]), device="cuda")
    with pytest.raises(kva.KvaError):
        proj.project(x, outs=proj.alloc_outputs(65))
    with pytest.raises(kva.KvaError):
        kva.kva_project_ubatch(proj.ctx, x.data_ptr(), 0, [o.data_ptr() for o in proj.alloc_outputs(1)])
    with pytest.raises(kva.KvaError) as e:           # rows are read 16 bytes at a time
        kva.kva_project_ubatch(proj.ctx, x.data_ptr() + 4, 1, [o.data_ptr() for o in proj.alloc_outputs(1)])
    assert e.value.status == kva.KVA_ERR_ARG
    proj.close()


# ------------------------------------------------------------------ r2, one 1024-token ubatch

@pytest.fixture(scope="module")
def r2():
    cfg = synth.config("r2")
    w = synth.make_weights(cfg)
    prep = ref.prepare(cfg, w)
    return cfg, w, prep


@pytest.fixture(scope="module")
def r2_full(r2):
    """One r2 ubatch and the oracle's outputs for all 32 heads (computed once)."""
    cfg, w, prep = r2
    x = synth.make_input(cfg)
    return x, ref.project(cfg, prep, x)


@pytest.mark.parametrize("max_tokens", [1024, 1536])
def test_r2_full_ubatch_parity(r2, r2_full, max_tokens):
    """All 32 heads, all 1024 tokens, in a context of max_tokens = 1024 (the
    benchmark's: the N = d GEMMs split K three ways) and of 1536 (two ways)."""
    cfg, w, _ = r2
    x, want = r2_full
    proj = kva.Projector(cfg, w, max_tokens=max_tokens)
    got = _run(proj, x)
    _check(cfg, got, want, label=f"r2 1024, max_tokens {max_tokens}")
    # determinism: a second call is bitwise identical
    got2 = _run(proj, x)
    assert all(np.array_equal(a, b) for a, b in zip(got, got2))
    proj.close()


def test_r2_partial_last_ubatch(r2):
    cfg, w, prep = r2
    x = synth.make_input(cfg, n_tokens=1536, seed=21)
    proj = kva.Projector(cfg, w, max_tokens=1536)
    got = _run(proj, x)
    heads = [0, 3, 31]
    want = ref.project(cfg, prep, x[1024:], which=heads)
    _check(cfg, {i: got[i][1024:] for i in heads}, want, label="r2 tail 512")
    first = _run(proj, np.ascontiguousarray(x[:1024]))
    assert all(np.array_equal(got[i][:1024], first[i]) for i in range(len(got)))
    proj.close()


@pytest.mark.parametrize("m", [16, 128])
def test_r2_small_context_parity(r2, m):
    """Contexts of at most 128 tokens per call split the GEMMs whose N is the
    trunk width eight ways in K: all 32 heads against the oracle."""
    cfg, w, prep = r2
    x = synth.make_input(cfg, n_tokens=m, seed=23)
    proj = kva.Projector(cfg, w, max_tokens=m)
    got = _run(proj, x)
    want = ref.project(cfg, prep, x)
    _check(cfg, got, want, label=f"r2 context of {m} tokens")
    proj.close()


def test_r2_short_calls_bitwise_equal_to_full_ubatch(r2):
    """Calls of 64, 100 and 300 tokens run other GEMM tiles (64-, 128- and
    256-row head tiles, other trunk tiles) than a 1024-token call: the first
    tokens of a block must still come out bit for bit the same (causality
    makes them independent of the later tokens), and match the oracle."""
    cfg, w, prep = r2
    x = synth.make_input(cfg, n_tokens=1024, seed=22)
    proj = kva.Projector(cfg, w, max_tokens=1024)
    full = _run(proj, x)
    for n in (64, 100, 300):
        part = _run(proj, np.ascontiguousarray(x[:n]))
        for i in range(len(part)):
            assert np.array_equal(part[i], full[i][:n]), (n, i)
    want = ref.project(cfg, prep, x[:64], which=[0, 31])
    _check(cfg, {i: full[i][:64] for i in (0, 31)}, want, label="r2 first 64")
    proj.close()


# ------------------------------------------------------------------ r3: blocks, causality

@pytest.fixture(scope="module")
def r3():
    cfg = synth.config("r3")
    return cfg, synth.make_weights(cfg)


def test_r3_blocks_are_independent_and_causal(r3):
    cfg, w = r3
    x = synth.make_input(cfg, n_tokens=2048)
    proj = kva.Projector(cfg, w, max_tokens=2048)
    both = _run(proj, x)
    b0 = _run(proj, np.ascontiguousarray(x[:1024]))
    b1 = _run(proj, np.ascontiguousarray(x[1024:]))
    for i in range(len(both)):
        assert np.array_equal(both[i][:1024], b0[i]), i
        assert np.array_equal(both[i][1024:], b1[i]), i
    j = 1500
    x2 = x.copy()
    x2[j] *= np.float32(-1.5)
    pert = _run(proj, x2)
    for i in range(len(both)):
        assert np.array_equal(both[i][:j], pert[i][:j]), i
        assert not np.array_equal(both[i][j], pert[i][j]), i
    proj.close()


def test_r3_parity_all_heads(r3):
    """All 36 heads (24 DeltaNet, 8 attention, 4 drafters) of one ubatch."""
    cfg, w = r3
    x = synth.make_input(cfg, n_tokens=1024)
    proj = kva.Projector(cfg, w, max_tokens=1024)
    got = _run(proj, x)
    want = ref.project(cfg, ref.prepare(cfg, w), x)
    _check(cfg, got, want, label="r3 all heads")
    proj.close()


def test_r3_8192_tokens_in_one_call(r3):
    """The r3 workload as configured: an 8192-token prompt in one call of a
    max_tokens = 8192 context is 8 independent 1024-token blocks.  Each
    block's outputs equal, bit for bit, a 1024-token call of the same
    context on that block alone; blocks 0 and 7 match the oracle on all 36
    heads (the oracle's block independence is pinned on the CPU)."""
    cfg, w = r3
    x = synth.make_input(cfg, n_tokens=8192)
    proj = kva.Projector(cfg, w, max_tokens=8192)
    full = proj.project(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    for b in range(8):
        part = proj.project(torch.from_numpy(np.ascontiguousarray(x[b * 1024:(b + 1) * 1024])).cuda())
        torch.cuda.synchronize()
        for i in range(len(part)):
            assert torch.equal(full[i][b * 1024:(b + 1) * 1024], part[i]), (b, i)
        del part
    prep = ref.prepare(cfg, w)
    for b in (0, 7):
        want = ref.project(cfg, prep, x[b * 1024:(b + 1) * 1024])
        got = [o[b * 1024:(b + 1) * 1024].cpu().numpy() for o in full]
        _check(cfg, got, want, label=f"r3 8192-token call, block {b}")
    del full
    proj.close()


# ------------------------------------------------------------------ hooks and the KV-cache write

def test_dequant_q8_0_bit_exact():
    rng = np.random.default_rng(9)
    nb = 4096
    codes = rng.integers(-128, 128, size=(1, nb * 32), dtype=np.int8)
    sc_bits = rng.integers(0, 0x7C00, size=nb).astype(np.uint16)          # every finite magnitude
    sc_bits |= (rng.integers(0, 2, size=nb).astype(np.uint16) << 15)       # both signs
    sc_bits[:64] = np.arange(64, dtype=np.uint16)                           # subnormals and +0
    packed = synth.pack_q8_0(codes, sc_bits.view(np.float16).reshape(1, nb))
    want = ref.dequant_q8_0(packed, 1, nb * 32).astype(np.float32).reshape(-1)
    blocks = torch.from_numpy(packed.reshape(-1)).cuda()
    out = torch.empty(nb * 32, dtype=torch.float32, device="cuda")
    kva.kva_debug_dequant_q8_0(blocks.data_ptr(), nb, out.data_ptr(), kva.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_dequant_q8_0_f16_weights_bit_exact():
    """The fp16 weights the q8_0 GEMMs use (their own device routine) equal the
    exact d * q rounded once to nearest-even binary16, overflow included."""
    rng = np.random.default_rng(10)
    nb = 4096
    codes = rng.integers(-128, 128, size=(1, nb * 32), dtype=np.int8)
    sc_bits = rng.integers(0, 0x7C00, size=nb).astype(np.uint16)
    sc_bits |= (rng.integers(0, 2, size=nb).astype(np.uint16) << 15)
    sc_bits[:64] = np.arange(64, dtype=np.uint16)
    packed = synth.pack_q8_0(codes, sc_bits.view(np.float16).reshape(1, nb))
    want = ref.dequant_q8_0_f16_bits(packed, 1, nb * 32).reshape(-1)
    assert (want == 0x7C00).any() and (want == 0xFC00).any() and (want & 0x7C00 == 0).any()
    blocks = torch.from_numpy(packed.reshape(-1)).cuda()
    out = torch.empty(nb * 32, dtype=torch.int16, device="cuda")
    kva.kva_debug_dequant_q8_0_f16(blocks.data_ptr(), nb, out.data_ptr(), kva.current_stream())
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]


def _kv_cache(n_logical, n_pages):
    kp = torch.full((n_pages, 256, 4, 256), -1, dtype=torch.int16, device="cuda")
    vp = torch.full((n_pages, 256, 4, 256), -1, dtype=torch.int16, device="cuda")
    return kp, vp


def _check_kv_bf16(gk, gv, k, v, n_rot):
    """bf16 cache rows (bit patterns) against the oracle's float64 K and V."""
    assert np.array_equal(gv, ref.f64_to_bf16_bits(v))            # V: a single rounding of fp32 data
    # K: one bf16 ulp of the correctly rounded value, plus the fp32 rotation's
    # absolute error (angle, sin/cos and products, relative to the rotary pair's
    # norm): where a rotated value nearly cancels, that exceeds its own bf16 ulp.
    dk = np.abs(ref.bf16_bits_to_f64(gk) - ref.bf16_bits_to_f64(ref.f64_to_bf16_bits(k)))
    ulp = np.ldexp(1.0, np.frexp(np.abs(k))[1] - 8)
    pair = np.zeros_like(k)
    half = n_rot // 2
    pn = np.sqrt(k[..., :half] ** 2 + k[..., half:n_rot] ** 2)
    pair[..., :half], pair[..., half:n_rot] = pn, pn
    bound = ulp + 2.0 ** -20 * pair
    assert np.all(dk <= bound), float(np.max(dk / bound))
    assert np.mean(dk == 0) > (0.98 if k.shape[0] > 100 else 0.9)


@pytest.mark.parametrize("pos0,n,n_rot", [(0, 600, 64), (65536 - 700, 700, 64), (300, 5, 32), (1021, 3, 64),
                                          (4000, 1, 16)])
def test_kv_write_parity(pos0, n, n_rot):
    n_logical = (pos0 + n + 255) // 256
    gains, ptab, n_pages = synth.make_kv_write_inputs(pos0 + n, n_layers=1)
    kv = synth.make_kv_rows(n, scale=3.0)
    kp, vp = _kv_cache(n_logical, n_pages)
    ptab_d = torch.from_numpy(ptab).cuda()
    cache = kva.kva_paged_kv(kp.data_ptr(), vp.data_ptr(), ptab_d.data_ptr(), 256, n_pages, len(ptab),
                             4, 256, n_rot, 1.0e7, 1e-6)
    kv_d = torch.from_numpy(kv).cuda()
    g_d = torch.from_numpy(gains[0]).cuda()
    kva.kva_attn_kv_write(kv_d.data_ptr(), kv.shape[1], n, pos0, g_d.data_ptr(), cache, kva.current_stream())
    torch.cuda.synchronize()
    kpn = kp.cpu().numpy().view(np.uint16)
    vpn = vp.cpu().numpy().view(np.uint16)
    k, v = ref.kv_write_values(kv, gains[0], pos0, n_rot=n_rot)
    pos = pos0 + np.arange(n)
    _check_kv_bf16(kpn[ptab[pos // 256], pos % 256], vpn[ptab[pos // 256], pos % 256], k, v, n_rot)
    # slots outside the written range keep the poison
    used = np.zeros((n_pages, 256), dtype=bool)
    used[ptab[pos // 256], pos % 256] = True
    assert np.all(kpn[~used] == 0xFFFF) and np.all(vpn[~used] == 0xFFFF)


def test_kv_write_every_position_of_a_65536_token_prompt():
    """The bf16 paged KV write of a whole 65536-token prompt for 8 attention
    layers, in the launches the benchmark times (8192 tokens per call): every
    position of every layer against the oracle, at the bar above, and every
    slot of every page written."""
    n_tok, layers, chunk = 65536, 8, 8192
    gains, ptab, n_pages = synth.make_kv_write_inputs(n_tok, n_layers=layers)
    ptab_d = torch.from_numpy(ptab).cuda()
    st = kva.current_stream()
    for li in range(layers):
        kv = synth.make_kv_rows(n_tok, seed=40 + li, scale=3.0)
        kp, vp = _kv_cache((n_tok + 255) // 256, n_pages)
        cache = kva.kva_paged_kv(kp.data_ptr(), vp.data_ptr(), ptab_d.data_ptr(), 256, n_pages, len(ptab),
                                 4, 256, 64, 1.0e7, 1e-6)
        kv_d = torch.from_numpy(kv).cuda()
        g_d = torch.from_numpy(gains[li]).cuda()
        for c0 in range(0, n_tok, chunk):
            kva.kva_attn_kv_write(kv_d[c0].data_ptr(), kv.shape[1], chunk, c0, g_d.data_ptr(), cache, st)
        torch.cuda.synchronize()
        kpn = kp.cpu().numpy().view(np.uint16)
        vpn = vp.cpu().numpy().view(np.uint16)
        assert not (kpn == 0xFFFF).all(axis=-1).any() and not (vpn == 0xFFFF).all(axis=-1).any()
        def check(c0, li=li, kv=kv, kpn=kpn, vpn=vpn):
            k, v = ref.kv_write_values(kv[c0:c0 + chunk], gains[li], c0)
            pos = c0 + np.arange(chunk)
            _check_kv_bf16(kpn[ptab[pos // 256], pos % 256], vpn[ptab[pos // 256], pos % 256], k, v, 64)

        # the oracle's chunks in threads (NumPy releases the GIL in its loops)
        with concurrent.futures.ThreadPoolExecutor(max_workers=8) as pool:
            list(pool.map(check, range(0, n_tok, chunk)))
        print(f"kv write layer {li}: all {n_tok} positions match", flush=True)
        del kv_d, kp, vp


def _q8_rows_check(got_rows, want, where):
    """got_rows [..., 272] q8_0 bytes vs float64 rotated values [..., 256].
    Every dequantised value lies within the q8_0 bound of the float64 value
    (half a step, the fp16 storage of the scale, and the fp32 arithmetic before
    the decision); codes equal the oracle's except where the oracle's own
    y / d sits within that fp32 slack of a rounding tie."""
    gd = ref.q8_0_block_values(got_rows)
    d_bits, q = ref.q8_0_quantize(want)
    blk = want.reshape(want.shape[:-1] + (8, 32))
    amax = np.abs(blk).max(-1)
    d32 = amax / 127.0
    d16 = ref.f16_bits_to_f64(d_bits)
    slack = 2e-6 * amax                                 # fp32 Hadamard / norm / RoPE error, generous
    bound = 0.5 * d32 + np.abs(d16 - d32) * 127 + slack
    err = np.abs(gd.reshape(blk.shape) - blk)
    assert np.all(err <= bound[..., None] * (1 + 1e-9)), (where, float(np.max(err / bound[..., None])))
    gq = np.ascontiguousarray(got_rows.reshape(got_rows.shape[:-1] + (8, 34))[..., 2:]).view(np.int8)
    diff = gq != q
    t = blk / np.where(d32 == 0, 1, d32)[..., None]
    near_tie = np.abs(np.abs(t - np.trunc(t)) - 0.5) < (slack / np.where(d32 == 0, 1, d32))[..., None] + 1e-4
    assert np.all(~diff | near_tie), where
    assert np.all(np.abs(gq.astype(int) - q.astype(int)) <= 1), where
    return float(np.mean(diff))


def test_q8_scale_rule_is_correctly_rounded_division_for_every_binary32():
    """The KV write forms the q8_0 block scale d = amax / 127 and its
    reciprocal without the division sequence; the device routine it runs
    must give the correctly rounded quotients on every input it is used for
    (all 2^32 patterns; the guarded reciprocal everywhere)."""
    counts = torch.zeros(3, dtype=torch.int64, device="cuda")
    kva.kva_debug_check_q8_scale(counts.data_ptr(), kva.current_stream())
    torch.cuda.synchronize()
    assert counts.tolist() == [0, 0, 0]


@pytest.mark.parametrize("integer", [True, False])
def test_kv_write_q8_0_hadamard_parity(integer):
    """Hadamard-rotated q8_0 KV write.  Integer-valued inputs make V's rotation
    exact in fp32, so V's scales and codes must equal the oracle's bit for bit;
    K (k_norm, RoPE) and real-valued inputs are held to the q8_0 bound."""
    pos0, n = 1000, 701
    n_logical = (pos0 + n + 255) // 256
    gains, ptab, n_pages = synth.make_kv_write_inputs(pos0 + n, n_layers=1)
    if integer:
        rng = np.random.default_rng(21)
        kv = np.round(rng.standard_normal((n, 2048)) * 20).astype(np.float32)
        kv[7, 1024:1024 + 256] = 0.0                   # an all-zero V head: every block has d = 0, codes 0
    else:
        kv = synth.make_kv_rows(n, scale=3.0)
    kp = torch.full((n_pages, 256, 4, 272), 0xFF, dtype=torch.uint8, device="cuda")
    vp = torch.full((n_pages, 256, 4, 272), 0xFF, dtype=torch.uint8, device="cuda")
    ptab_d = torch.from_numpy(ptab).cuda()
    cache = kva.kva_paged_kv(kp.data_ptr(), vp.data_ptr(), ptab_d.data_ptr(), 256, n_pages, len(ptab),
                             4, 256, 64, 1.0e7, 1e-6, kva.KVA_KV_Q8_0_HADAMARD)
    kv_d = torch.from_numpy(kv).cuda()
    g_d = torch.from_numpy(gains[0]).cuda()
    print(f"q8_0 KV write: integer={integer} pos0={pos0} n={n}", flush=True)
    kva.kva_attn_kv_write(kv_d.data_ptr(), kv.shape[1], n, pos0, g_d.data_ptr(), cache, kva.current_stream())
    torch.cuda.synchronize()
    kpn, vpn = kp.cpu().numpy(), vp.cpu().numpy()
    k, v = ref.kv_write_q8_0_values(kv, gains[0], pos0)
    pos = pos0 + np.arange(n)
    gk = kpn[ptab[pos // 256], pos % 256]
    gv = vpn[ptab[pos // 256], pos % 256]
    if integer:
        want_v = ref.q8_0_block_bytes(*ref.q8_0_quantize(v))
        assert np.array_equal(gv, want_v)
        assert not gv[7, 0].any()
    fk = _q8_rows_check(gk, k, "k")
    fv = _q8_rows_check(gv, v, "v")
    print(f"  codes differing from the oracle's: k {fk:.2e}, v {fv:.2e}", flush=True)
    assert fk < 1e-3 and fv < 1e-3
    used = np.zeros((n_pages, 256), dtype=bool)
    used[ptab[pos // 256], pos % 256] = True
    assert np.all(kpn[~used] == 0xFF) and np.all(vpn[~used] == 0xFF)


def test_r2_projection_chained_into_deltanet_update(r2):
    """The r2 projector's 24 DeltaNet heads feed kva_deltanet_update straight
    from the head output buffers (rows of qkv | a | b); every layer is held to
    the oracle's update on the same fp32 rows (the DeltaNet bar of
    test_gpu_deltanet.py)."""
    cfg, w, _ = r2
    x = synth.make_input(cfg, n_tokens=1024, seed=23)
    proj = kva.Projector(cfg, w, max_tokens=1024)
    outs = proj.project(torch.from_numpy(x).cuda())
    dn = [i for i, h in enumerate(cfg["heads"]) if h["kind"] == "deltanet"]
    assert len(dn) == 24
    conv_w, a_log, dt_bias = synth.make_deltanet_params(len(dn))
    conv, S = synth.make_deltanet_state(len(dn))
    dev = [(torch.from_numpy(conv_w[l]).cuda(), torch.from_numpy(a_log[l]).cuda(),
            torch.from_numpy(dt_bias[l]).cuda(), torch.from_numpy(conv[l]).cuda(), torch.from_numpy(S[l]).cuda())
           for l in range(len(dn))]
    layers = [kva.kva_deltanet_layer(outs[hi].data_ptr(), cfg["heads"][hi]["out_dim"], *[t.data_ptr() for t in d])
              for hi, d in zip(dn, dev)]
    kva.kva_deltanet_update(layers, 1024, stream=kva.current_stream())
    torch.cuda.synchronize()
    # the oracle's 24 sequential scans run in worker processes (spawned: the
    # parent holds the GPU)
    import concurrent.futures
    import multiprocessing
    rows_all = [outs[dn[l]].cpu().numpy() for l in range(len(dn))]
    with concurrent.futures.ProcessPoolExecutor(max_workers=min(8, os.cpu_count() or 1),
                                                mp_context=multiprocessing.get_context("spawn")) as ex:
        refs = list(ex.map(ref.deltanet_update, rows_all, conv_w, a_log, dt_bias, conv, S))
    for l in range(len(dn)):
        S_ref, c_ref = refs[l]
        got = dev[l][4].cpu().numpy().astype(np.float64)
        rms = np.sqrt(np.mean(S_ref ** 2))
        mx = np.max(np.abs(got - S_ref)) / rms
        sd = np.sqrt(np.mean((got - S_ref) ** 2)) / rms
        print(f"r2 layer {cfg['heads'][dn[l]]['layer']}: state max|err|/rms {mx:.3e} rms {sd:.3e}", flush=True)
        assert mx <= 2e-2 and sd <= 4e-3
        assert np.array_equal(dev[l][3].cpu().numpy(), c_ref.astype(np.float32))
    proj.close()
