"""GPU parity for the q8_0 and q4_0 projectors and the chained
attention-layer KV-cache write at prompt scale (65536 tokens, processed in
8192-token calls as the benchmark does).  Oracle: float64 on the dequantised
weights (d * q, d * (n - 8)).  q4_0 is held to the q8_0 bar (the pages give
no bar of their own for it).

Bars: q8_0 outputs max|err| <= 5e-2 * RMS per head; KV cache after the
chained projection + k_norm + RoPE + bf16 store within the projector's bar
(2e-2 * RMS) plus one bf16 rounding of the largest value (2^-9 * max|v|).
"""
import numpy as np
import pytest
import torch

import learned_kv_approximation_amd as kva
import oracle
import synth
from oracle import ref

pytestmark = pytest.mark.gpu
TOL_Q8 = 5e-2
CHUNK = 8192
N_PROMPT = 65536


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _err(g, y):
    rms = np.sqrt(np.mean(y * y))
    return float(np.max(np.abs(g.astype(np.float64) - y)) / rms)


def _bf16_bar(y, tol=2e-2):
    return tol + 2.0 ** -9 * float(np.max(np.abs(y)) / np.sqrt(np.mean(y * y)))


def test_tiny_q8_0_parity():
    cfg = synth.config("tiny", weight_dtype="q8_0")
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=100)
    proj = kva.Projector(cfg, w, max_tokens=128)
    outs = proj.project(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    want = oracle.project(cfg, w, x)
    errs = [_err(o.cpu().numpy(), want[i]) for i, o in enumerate(outs)]
    print("tiny q8_0 max|err|/rms per head", errs)
    assert max(errs) <= TOL_Q8
    proj.close()


@pytest.mark.parametrize("dtype,d_bits,where", [("q8_0", 0x7BFF, "head"), ("q8_0", 0x7C00, "trunk"),
                                                  ("q8_0", 0x7E00, "head"), ("q4_0", 0x7BFF, "trunk"),
                                                  ("q4_0", 0xFC00, "head")])
def test_quantised_scale_out_of_fp16_range_is_rejected(dtype, d_bits, where):
    """A block whose fp16 weights d * code would overflow (65504 * 127 or
    * 8) or whose scale is an infinity or NaN is refused at create with
    KVA_ERR_RANGE, like an fp32 / bf16 weight outside fp16's range."""
    cfg = synth.config("tiny", weight_dtype=dtype)
    w = synth.make_weights(cfg)
    bpb = 34 if dtype == "q8_0" else 18
    if where == "head":
        t = w["heads"][1]["w"].copy()
        w = dict(w, heads=[dict(h) for h in w["heads"]])
        w["heads"][1]["w"] = t
    else:
        t = w["blocks"][2]["w_down"].copy()
        w = dict(w, blocks=[dict(b) for b in w["blocks"]])
        w["blocks"][2]["w_down"] = t
    flat = t.reshape(-1).view(np.uint8)
    flat[5 * bpb:5 * bpb + 2] = np.array([d_bits], dtype=np.uint16).view(np.uint8)
    if dtype == "q8_0":
        flat[5 * bpb + 2] = 127                 # a code of magnitude 127 in that block
    else:
        flat[5 * bpb + 2] = 0x00                # code 0: n - 8 = -8
    with pytest.raises(kva.KvaError) as e:
        kva.Projector(cfg, w, max_tokens=64)
    assert e.value.status == kva.KVA_ERR_RANGE, str(e.value)


@pytest.fixture(scope="module")
def r3q8():
    cfg = synth.config("r3_q8_0")
    w = synth.make_weights(cfg)
    return cfg, w, ref.prepare(cfg, w)


def test_r3_q8_0_prompt_in_chunks(r3q8):
    """65536 tokens in 8 calls of 8192: ubatches 0 and 63 against the oracle on
    all 36 heads, ubatch 31 on three, and ubatch 31 bitwise equal to a call
    on that ubatch alone."""
    cfg, w, prep = r3q8
    x = synth.make_input(cfg, n_tokens=N_PROMPT)
    proj = kva.Projector(cfg, w, max_tokens=CHUNK)
    outs = proj.alloc_outputs(CHUNK)
    xd = torch.from_numpy(x).cuda()
    heads = [0, 3, 35]
    keep = {}
    for c0 in range(0, N_PROMPT, CHUNK):
        proj.project(xd[c0:c0 + CHUNK], outs)
        for u in (0, 31, 63):
            s = u * 1024
            if c0 <= s < c0 + CHUNK:
                keep[u] = [outs[i][s - c0:s - c0 + 1024].cpu().numpy() for i in range(len(outs))]
    torch.cuda.synchronize()
    for u in (0, 31, 63):
        which = heads if u == 31 else list(range(len(cfg["heads"])))
        want = ref.project(cfg, prep, x[u * 1024:(u + 1) * 1024], which=which)
        errs = {cfg["heads"][i]["name"]: _err(keep[u][i], want[i]) for i in which}
        print(f"q8_0 ubatch {u}: {errs}", flush=True)
        assert max(errs.values()) <= TOL_Q8
    alone = proj.project(xd[31 * 1024:32 * 1024].contiguous())
    torch.cuda.synchronize()
    for i in range(len(alone)):
        assert np.array_equal(alone[i].cpu().numpy(), keep[31][i]), i
    proj.close()


def test_r3_q8_0_short_call_bitwise_equal(r3q8):
    """A 64-token call (one 64-row M-tile) and a 1024-token call give the same
    bits for the first 64 tokens, within the q8_0 bar of the oracle."""
    cfg, w, prep = r3q8
    x = synth.make_input(cfg, n_tokens=1024)
    proj = kva.Projector(cfg, w, max_tokens=1024)
    xd = torch.from_numpy(x).cuda()
    full = [o.cpu().numpy() for o in proj.project(xd)]
    short = [o.cpu().numpy() for o in proj.project(xd[:64].contiguous())]
    torch.cuda.synchronize()
    for i in range(len(full)):
        assert np.array_equal(short[i], full[i][:64]), i
    want = ref.project(cfg, prep, x[:64], which=[0, 35])
    errs = [_err(short[i], want[i]) for i in (0, 35)]
    print("q8_0 64-token call max|err|/rms", errs)
    assert max(errs) <= TOL_Q8
    proj.close()


def test_dequant_q4_0_f16_weights_bit_exact():
    """The fp16 weights the q4_0 GEMMs use equal d * (n - 8) rounded once to
    nearest-even binary16, over every scale magnitude and both signs."""
    rng = np.random.default_rng(13)
    nb = 4096
    codes = rng.integers(0, 16, size=(1, nb * 32), dtype=np.uint8)
    sc_bits = rng.integers(0, 0x7C00, size=nb).astype(np.uint16)
    sc_bits |= (rng.integers(0, 2, size=nb).astype(np.uint16) << 15)
    sc_bits[:64] = np.arange(64, dtype=np.uint16)
    packed = synth.pack_q4_0(codes, sc_bits.view(np.float16).reshape(1, nb))
    want = ref.dequant_q4_0_f16_bits(packed, 1, nb * 32).reshape(-1)
    blocks = torch.from_numpy(packed.reshape(-1)).cuda()
    out = torch.empty(nb * 32, dtype=torch.int16, device="cuda")
    kva.kva_debug_dequant_q4_0_f16(blocks.data_ptr(), nb, out.data_ptr(), kva.current_stream())
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]


@pytest.mark.parametrize("n", [40, 100, 300])
def test_tiny_q4_0_parity(n):
    cfg = synth.config("tiny", weight_dtype="q4_0")
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=n)
    proj = kva.Projector(cfg, w, max_tokens=n)
    outs = proj.project(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    want = oracle.project(cfg, w, x)
    errs = [_err(o.cpu().numpy(), want[i]) for i, o in enumerate(outs)]
    print(f"tiny q4_0 n={n} max|err|/rms per head", errs)
    assert max(errs) <= TOL_Q8
    proj.close()


def test_r3_q4_0_ubatch_parity():
    cfg = synth.config("r3_q4_0")
    w = synth.make_weights(cfg)
    prep = ref.prepare(cfg, w)
    x = synth.make_input(cfg, n_tokens=1024)
    proj = kva.Projector(cfg, w, max_tokens=1024)
    outs = proj.project(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    heads = list(range(len(cfg["heads"])))          # all 36
    want = ref.project(cfg, prep, x, which=heads)
    errs = {cfg["heads"][i]["name"]: _err(outs[i].cpu().numpy(), want[i]) for i in heads}
    print("r3 q4_0 max|err|/rms", max(errs.values()), flush=True)
    assert max(errs.values()) <= TOL_Q8
    proj.close()


@pytest.mark.parametrize("cfg_name", ["r3_q8_0", "r3_q4_0"])
def test_expanded_fp16_weights_give_the_in_register_bits(cfg_name):
    """A context of more than 256 tokens per call holds the q8_0 / q4_0
    weights expanded to fp16 at create (twice the weight bytes); one of at
    most 256 keeps the code and scale planes and dequantises in registers.
    Both multiply the same fp16 weights in the same K order (here both split
    the d-wide GEMMs two ways: max_tokens 2048 and 256), so a call's outputs
    must be bitwise equal."""
    cfg = synth.config(cfg_name)
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=200, seed=25)
    outs, wbytes = [], []
    for max_tokens in (2048, 256):
        proj = kva.Projector(cfg, w, max_tokens=max_tokens)
        outs.append([o.cpu() for o in proj.project(torch.from_numpy(x).cuda())])
        torch.cuda.synchronize()
        wbytes.append(kva.kva_get_stats(proj.ctx)["weight_bytes"])
        proj.close()
    print(f"{cfg_name}: weight bytes expanded {wbytes[0]}, planes {wbytes[1]}", flush=True)
    assert wbytes[0] > 1.8 * wbytes[1]
    for i, (a, b) in enumerate(zip(*outs)):
        assert torch.equal(a, b), (cfg_name, cfg["heads"][i]["name"])


@pytest.mark.parametrize("m", [16, 128])
def test_r3_q8_0_small_context_parity(m):
    """A context of at most 128 tokens per call splits the GEMMs whose N is
    the trunk width eight ways in K (the benchmark's per-M contexts)."""
    cfg = synth.config("r3_q8_0")
    w = synth.make_weights(cfg)
    prep = ref.prepare(cfg, w)
    x = synth.make_input(cfg, n_tokens=m, seed=24)
    proj = kva.Projector(cfg, w, max_tokens=m)
    outs = proj.project(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    heads = list(range(len(cfg["heads"])))
    want = ref.project(cfg, prep, x, which=heads)
    errs = {cfg["heads"][i]["name"]: _err(outs[i].cpu().numpy(), want[i]) for i in heads}
    print(f"r3 q8_0 context of {m} tokens: max|err|/rms {max(errs.values()):.4e}", flush=True)
    assert max(errs.values()) <= TOL_Q8
    proj.close()


@pytest.fixture(scope="module")
def r3bf16():
    cfg = synth.config("r3_kv")
    w = synth.make_weights(cfg)
    return cfg, w, ref.prepare(cfg, w)


def test_r3_projection_chained_into_paged_kv_cache(r3bf16):
    """The r3 bf16 projector over a 65536-token prompt, each attention head's
    k|v written through k_norm + RoPE into its layer's paged bf16 cache."""
    cfg, w, prep = r3bf16
    x = synth.make_input(cfg, n_tokens=N_PROMPT)
    attn = [i for i, h in enumerate(cfg["heads"]) if h["kind"] == "attn"]
    gains, ptab, n_pages = synth.make_kv_write_inputs(N_PROMPT, n_layers=len(attn), seed=cfg["seed"])
    proj = kva.Projector(cfg, w, max_tokens=CHUNK)
    outs = proj.alloc_outputs(CHUNK)
    xd = torch.from_numpy(x).cuda()
    ptab_d = torch.from_numpy(ptab).cuda()
    gains_d = torch.from_numpy(gains).cuda()
    pools = [(torch.full((n_pages, 256, 4, 256), -1, dtype=torch.int16, device="cuda"),
              torch.full((n_pages, 256, 4, 256), -1, dtype=torch.int16, device="cuda")) for _ in attn]
    caches = [kva.kva_paged_kv(kp.data_ptr(), vp.data_ptr(), ptab_d.data_ptr(), 256, n_pages, len(ptab),
                               4, 256, 64, 1.0e7, 1e-6) for kp, vp in pools]
    st = kva.current_stream()
    for c0 in range(0, N_PROMPT, CHUNK):
        proj.project(xd[c0:c0 + CHUNK], outs)
        for li, hi in enumerate(attn):
            kva.kva_attn_kv_write(outs[hi].data_ptr(), 2048, CHUNK, c0, gains_d[li].data_ptr(), caches[li], st)
    torch.cuda.synchronize()
    want = {u: ref.project(cfg, prep, x[u * 1024:(u + 1) * 1024], which=attn) for u in (0, 63)}
    for li, hi in enumerate(attn):
        kpn = pools[li][0].cpu().numpy().view(np.uint16)
        vpn = pools[li][1].cpu().numpy().view(np.uint16)
        for u in (0, 63):
            pos = u * 1024 + np.arange(1024)
            k, v = ref.kv_write_values(want[u][hi], gains[li], u * 1024)
            ek = _err(ref.bf16_bits_to_f64(kpn[ptab[pos // 256], pos % 256]), k)
            ev = _err(ref.bf16_bits_to_f64(vpn[ptab[pos // 256], pos % 256]), v)
            print(f"kv layer {cfg['heads'][hi]['layer']} ubatch {u}: k {ek:.3e} v {ev:.3e}", flush=True)
            assert ek <= _bf16_bar(k) and ev <= _bf16_bar(v), (u, li, ek, ev, _bf16_bar(k), _bf16_bar(v))
    # every slot of every page was written (no poison left anywhere)
    for kp, vp in pools:
        assert not bool((kp == -1).all(dim=-1).any()) and not bool((vp == -1).all(dim=-1).any())
    proj.close()


def _fused_r3(cfg, w, cases, kv_type=kva.KVA_KV_BF16):
    from test_gpu_fused_kv import fused_vs_chained
    attn = [i for i, h in enumerate(cfg["heads"]) if h["kind"] == "attn"]
    gains, ptab, n_pages = synth.make_kv_write_inputs(N_PROMPT, n_layers=len(attn), seed=cfg["seed"])
    n_max = max(n for n, _ in cases)
    x = synth.make_input(cfg, n_tokens=n_max)
    proj = kva.Projector(cfg, w, max_tokens=n_max)
    xd = torch.from_numpy(x).cuda()
    gains_d = torch.from_numpy(gains).cuda()
    for n, pos0 in cases:
        fused_vs_chained(proj, cfg, xd, n, pos0, ptab, n_pages, gains_d, kv_type)
    proj.close()


def test_r3_fused_kv_epilogue_equals_chained(r3bf16):
    """kva_project_ubatch_kv on the r3 bf16 projector: pools bitwise equal to
    the chained path (held to the oracle above), other heads bitwise equal."""
    cfg, w, _ = r3bf16
    _fused_r3(cfg, w, [(8192, 16384), (1000, 40007), (100, N_PROMPT - 100), (33, 5)])


def test_r3_q8_0_fused_kv_epilogue_equals_chained(r3q8):
    cfg, w, _ = r3q8
    _fused_r3(cfg, w, [(1024, 7 * 1024), (64, 300)])


def test_r3_fused_q8_0_kv_cache_equals_chained(r3bf16):
    """Hadamard-rotated q8_0 pools at r3 scale, fused vs chained."""
    cfg, w, _ = r3bf16
    _fused_r3(cfg, w, [(8192, 16384), (100, N_PROMPT - 100)], kv_type=kva.KVA_KV_Q8_0_HADAMARD)
