"""GPU tests of kva_project_ubatch_kv: the attention-layer state update (k_norm
+ RoPE + paged bf16 KV write) fused into the head GEMM's epilogue.

The fused path runs the same per-lane arithmetic as kva_attn_kv_write on the
same fp32 values (the head GEMM's accumulator plus bias), so the pools must
hold exactly the bits of kva_project_ubatch followed by kva_attn_kv_write,
and every other head's output must be bitwise that of kva_project_ubatch.
The chained path is itself held to the float64 oracle (here on a small
projector, and at r3 scale in test_gpu_q8_kv.py); the small case also
checks the fused pools against the oracle directly.

Shapes cover every head-GEMM tile the epilogue meets: calls of at most 64
rows (64x256 tiles), at most 128 rows (128x256), longer calls with ragged
256-row tiles, and a call where the KV tiles would otherwise fall into the
128-column remainder (the launch keeps them 256 wide).  Weight types: bf16,
q8_0, q4_0 (their staging buffers differ, so the epilogue stages 32 to 128
rows at a time).
"""
import numpy as np
import pytest
import torch

import learned_kv_approximation_amd as kva
import oracle
import synth
from oracle import ref

pytestmark = pytest.mark.gpu

KV_W = 2 * 4 * 256


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _small_cfg(weight_dtype):
    """A small trunk (d = 256) with two full-attention heads (k|v of 4 x 256)
    around DeltaNet-shaped heads (one full tile and a 16-column remainder)."""
    dn = {"kind": "deltanet", "out_dim": 256 + 16, "segments": [["qkv", 256], ["a", 8], ["b", 8]]}
    attn = {"kind": "attn", "out_dim": KV_W, "segments": [["k", 1024], ["v", 1024]]}
    heads = [dict(dn, name="kva.dn.a", layer=32), dict(attn, name="kva.attn.a", layer=35),
             dict(dn, name="kva.dn.b", layer=36), dict(attn, name="kva.attn.b", layer=39)]
    return synth.config("tiny", weight_dtype=weight_dtype, heads=heads, n_in=512)


def _pools(n, n_pages, kv_type=kva.KVA_KV_BF16):
    """Poisoned pools: bf16 rows of 0xFFFF, or q8_0 rows of 0xFF bytes."""
    if kv_type == kva.KVA_KV_BF16:
        shape, dt, poison = (n_pages, 256, 4, 256), torch.int16, -1
    else:
        shape, dt, poison = (n_pages, 256, 4, 272), torch.uint8, 0xFF
    return [(torch.full(shape, poison, dtype=dt, device="cuda"),
             torch.full(shape, poison, dtype=dt, device="cuda")) for _ in range(n)]


def _caches(pools, ptab_d, n_logical, n_pages, kv_type=kva.KVA_KV_BF16):
    return [kva.kva_paged_kv(kp.data_ptr(), vp.data_ptr(), ptab_d.data_ptr(), 256, n_pages, n_logical,
                             4, 256, 64, 1.0e7, 1e-6, kv_type) for kp, vp in pools]


def fused_vs_chained(proj, cfg, xd, n, pos0, ptab, n_pages, gains_d, kv_type=kva.KVA_KV_BF16):
    """Runs both paths on x[:n] at positions pos0.. and checks bitwise equality.
    Returns (fused pools, chained head outputs)."""
    attn = [i for i, h in enumerate(cfg["heads"]) if h["kind"] == "attn" and h["out_dim"] == KV_W]
    ptab_d = torch.from_numpy(ptab).cuda()
    pa, pb = _pools(len(attn), n_pages, kv_type), _pools(len(attn), n_pages, kv_type)
    ca = _caches(pa, ptab_d, len(ptab), n_pages, kv_type)
    cb = _caches(pb, ptab_d, len(ptab), n_pages, kv_type)
    st = kva.current_stream()
    print(f"fused vs chained: {cfg['name']} {cfg['weight_dtype']} n={n} pos0={pos0} kv_type={kv_type}", flush=True)
    outs_a = proj.alloc_outputs(n)
    proj.project(xd[:n], outs_a)
    for li, hi in enumerate(attn):
        kva.kva_attn_kv_write(outs_a[hi].data_ptr(), KV_W, n, pos0, gains_d[li].data_ptr(), ca[li], st)
    outs_b = [torch.full((n, h["out_dim"]), float("nan"), device="cuda") for h in cfg["heads"]]
    ptrs = [0 if i in attn else o.data_ptr() for i, o in enumerate(outs_b)]
    dests = [kva.kva_attn_dest(gains_d[li].data_ptr(), cb[li]) for li in range(len(attn))]
    kva.kva_project_ubatch_kv(proj.ctx, xd.data_ptr(), n, ptrs, pos0, dests, st)
    torch.cuda.synchronize()
    for li in range(len(attn)):
        for part in (0, 1):
            if not torch.equal(pa[li][part], pb[li][part]):
                a_, b_ = pa[li][part].cpu().numpy(), pb[li][part].cpu().numpy()
                bad = np.argwhere(a_ != b_)
                print(f"layer {li} {'kv'[part]}: {len(bad)} differing values, first {bad[:8].tolist()}, "
                      f"chained {a_[tuple(bad[:8].T)].tolist()} fused {b_[tuple(bad[:8].T)].tolist()}", flush=True)
            assert torch.equal(pa[li][part], pb[li][part]), ("kv"[part] + " pool", li)
    for i, h in enumerate(cfg["heads"]):
        if i not in attn:
            assert torch.equal(outs_a[i], outs_b[i]), ("head", i)
    # the fused call wrote exactly the tokens' slots
    pos = pos0 + np.arange(n)
    pages = ptab[pos // 256]
    ok = (pages >= 0) & (pages < n_pages)
    poison = -1 if kv_type == kva.KVA_KV_BF16 else 0xFF
    for kp, vp in pb:
        kn = kp.cpu().numpy()
        written = ~(kn == poison).all(axis=-1)      # [page][slot][kv head]
        want = np.zeros_like(written)
        want[pages[ok], pos[ok] % 256] = True
        assert np.array_equal(written, want)
    return pb, outs_a


@pytest.mark.parametrize("dtype", ["f32", "q8_0", "q4_0"])
def test_small_fused_kv_equals_chained_and_oracle(dtype):
    cfg = _small_cfg(dtype)
    w = synth.make_weights(cfg)
    n_max = 17 * 256
    x = synth.make_input(cfg, n_tokens=n_max)
    proj = kva.Projector(cfg, w, max_tokens=n_max)
    xd = torch.from_numpy(x).cuda()
    gains, ptab, n_pages = synth.make_kv_write_inputs(8192, n_layers=2, seed=7)
    gains_d = torch.from_numpy(gains).cuda()
    # a page entry outside [0, n_pages) on each side: those tokens are skipped
    bad = ptab.copy()
    bad[5], bad[9] = -1, n_pages
    for n, pos0, pt in [(40, 300, ptab), (100, 8192 - 100, ptab), (1200, 1234, bad),
                        (n_max, 3 * 256 + 17, ptab)]:
        pools, outs = fused_vs_chained(proj, cfg, xd, n, pos0, pt, n_pages, gains_d)
        if n > 1200:
            continue
        # oracle: projection in float64, then k_norm + RoPE; bf16 in the pools
        attn = [i for i, h in enumerate(cfg["heads"]) if h["kind"] == "attn"]
        want = oracle.project(cfg, w, x[:n], which=attn)
        pos = pos0 + np.arange(n)
        ok = (pt[pos // 256] >= 0) & (pt[pos // 256] < n_pages)
        for li, hi in enumerate(attn):
            k, v = ref.kv_write_values(want[hi], gains[li], pos0)
            kp, vp = (p.cpu().numpy().view(np.uint16) for p in pools[li])
            pg, sl = pt[pos[ok] // 256], pos[ok] % 256
            for name, got, ref_v in (("k", kp[pg, sl], k[ok]), ("v", vp[pg, sl], v[ok])):
                y = ref_v
                err = np.max(np.abs(ref.bf16_bits_to_f64(got) - y)) / np.sqrt(np.mean(y * y))
                tol = 5e-2 if dtype != "f32" else 2e-2
                bar = tol + 2.0 ** -9 * np.max(np.abs(y)) / np.sqrt(np.mean(y * y))
                print(f"  {dtype} n={n} head {hi} {name}: max|err|/rms {err:.3e} (bar {bar:.3e})", flush=True)
                assert err <= bar
    proj.close()


@pytest.mark.parametrize("dtype", ["f32", "q8_0"])
def test_small_fused_q8_0_kv_equals_chained_and_oracle(dtype):
    """The same with Hadamard-rotated q8_0 pools: fused bitwise equal to the
    chained write, and the dequantised rows within the q8_0 bound of the
    oracle (checked on the bf16-weight projector only, where the oracle's K
    and V are within 2e-2 of the GPU's)."""
    cfg = _small_cfg(dtype)
    w = synth.make_weights(cfg)
    n_max = 1200
    x = synth.make_input(cfg, n_tokens=n_max)
    proj = kva.Projector(cfg, w, max_tokens=n_max)
    xd = torch.from_numpy(x).cuda()
    gains, ptab, n_pages = synth.make_kv_write_inputs(8192, n_layers=2, seed=7)
    gains_d = torch.from_numpy(gains).cuda()
    for n, pos0 in [(40, 300), (100, 5000), (n_max, 1234)]:
        pools, _ = fused_vs_chained(proj, cfg, xd, n, pos0, ptab, n_pages, gains_d, kva.KVA_KV_Q8_0_HADAMARD)
        attn = [i for i, h in enumerate(cfg["heads"]) if h["kind"] == "attn"]
        want = oracle.project(cfg, w, x[:n], which=attn)
        pos = pos0 + np.arange(n)
        for li, hi in enumerate(attn):
            k, v = ref.kv_write_q8_0_values(want[hi], gains[li], pos0)
            for part, y in ((0, k), (1, v)):
                got = ref.q8_0_block_values(pools[li][part].cpu().numpy()[ptab[pos // 256], pos % 256])
                err = np.max(np.abs(got - y)) / np.sqrt(np.mean(y * y))
                tol = 5e-2 if dtype != "f32" else 2e-2
                # projector bar + q8_0 step (half of amax/127, amax <= ~4.5 RMS for these rows)
                bar = tol + 0.5 * np.max(np.abs(y)) / 127 / np.sqrt(np.mean(y * y)) * 1.1
                print(f"  {dtype} n={n} head {hi} {'kv'[part]}: max|err|/rms {err:.3e} (bar {bar:.3e})", flush=True)
                assert err <= bar
    proj.close()


def test_fused_kv_argument_errors():
    cfg = _small_cfg("f32")
    w = synth.make_weights(cfg)
    proj = kva.Projector(cfg, w, max_tokens=64)
    x = torch.from_numpy(synth.make_input(cfg, n_tokens=64)).cuda()
    gains, ptab, n_pages = synth.make_kv_write_inputs(512, n_layers=2, seed=7)
    gains_d, ptab_d = torch.from_numpy(gains).cuda(), torch.from_numpy(ptab).cuda()
    pools = _pools(2, n_pages)
    caches = _caches(pools, ptab_d, len(ptab), n_pages)
    outs = proj.alloc_outputs(64)
    ptrs = [o.data_ptr() for o in outs]
    dests = [kva.kva_attn_dest(gains_d[i].data_ptr(), caches[i]) for i in range(2)]
    st = kva.current_stream()
    with pytest.raises(kva.KvaError) as e:            # one destination missing
        kva.kva_project_ubatch_kv(proj.ctx, x.data_ptr(), 64, ptrs, 0, dests[:1], st)
    assert e.value.status == kva.KVA_ERR_SHAPE
    with pytest.raises(kva.KvaError) as e:            # positions past the page table
        kva.kva_project_ubatch_kv(proj.ctx, x.data_ptr(), 64, ptrs, 512 - 63, dests, st)
    assert e.value.status == kva.KVA_ERR_SHAPE
    odd = _caches(pools, ptab_d, len(ptab), n_pages)
    odd[1].n_rot = 32
    with pytest.raises(kva.KvaError) as e:            # differing rotary widths
        kva.kva_project_ubatch_kv(proj.ctx, x.data_ptr(), 64, ptrs, 0,
                                  [dests[0], kva.kva_attn_dest(gains_d[1].data_ptr(), odd[1])], st)
    assert e.value.status == kva.KVA_ERR_UNSUPPORTED
    bad_ptrs = list(ptrs)
    bad_ptrs[0] = 0                                   # a non-fused head needs its output
    with pytest.raises(kva.KvaError) as e:
        kva.kva_project_ubatch_kv(proj.ctx, x.data_ptr(), 64, bad_ptrs, 0, dests, st)
    assert e.value.status == kva.KVA_ERR_ARG
    torch.cuda.synchronize()
    # nothing was launched by the failed calls: the pools still hold only poison
    for kp, vp in pools:
        assert bool((kp == -1).all()) and bool((vp == -1).all())
    proj.close()
