"""GPU: invariants of the projection that hold whatever the values are.

- Scratch: a projection gives the same bits when every byte of the context's
  activation scratch was NaN beforehand (no kernel uses a scratch value that
  the same call did not write, except in results it discards: padding rows
  of the GEMM tiles, key columns past the block end).
- Guard bands: the head GEMM writes each head's [n_tokens][out_dim] output
  and nothing else: sentinel words right before and after every head's
  region (one shared allocation, heads back to back with gaps) survive, for
  full and ragged token counts, whole-head tiles and the tail tiles that
  gather the last out_dim % 256 columns of every head.
- Causality inside a block: a block's first n tokens come out bit for bit
  the same whatever the later tokens are (a call of n tokens against the
  full block), also with peaked scores, where the softmax reference points
  of the queries move between key tiles at different times.
- Reach of a NaN: a NaN in the input of token j makes every output of the
  tokens from j to the end of its block NaN and changes no bit of the other
  blocks or of the tokens before j's 64-token query tile.  The earlier
  tokens of that tile are not checked: the diagonal key tile multiplies
  their zero softmax weights with V rows that include token j's, and
  0 * NaN is NaN in the matrix cores.
"""
import numpy as np
import pytest
import torch

import learned_kv_approximation_amd as kva
import synth

pytestmark = pytest.mark.gpu
SENTINEL = 0x7FBADBAD          # a NaN bit pattern no projection produces


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(proj, x, outs=None):
    outs = proj.project(torch.from_numpy(x).cuda(), outs=outs)
    torch.cuda.synchronize()
    return outs


@pytest.mark.parametrize("dtype,n,block", [("f32", 1, 64), ("f32", 100, 64), ("f32", 256, 64), ("f32", 200, 1024),
                                           ("q8_0", 77, 64), ("q4_0", 130, 1024)])
def test_poisoned_scratch_gives_the_same_bits(dtype, n, block):
    cfg = synth.config("tiny", weight_dtype=dtype, attn_block=block)
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=n, seed=31)
    proj = kva.Projector(cfg, w, max_tokens=256)
    clean = [o.cpu() for o in _run(proj, x)]
    kva.kva_debug_poison_scratch(proj.ctx, kva.current_stream())
    dirty = [o.cpu() for o in _run(proj, x)]
    proj.close()
    for i, (a, b) in enumerate(zip(clean, dirty)):
        assert torch.isfinite(a).all(), i
        assert torch.equal(a, b), (dtype, n, i)


def test_poisoned_scratch_r2_ragged_call():
    cfg = synth.config("r2")
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=700, seed=32)
    proj = kva.Projector(cfg, w, max_tokens=1024)
    kva.kva_debug_poison_scratch(proj.ctx, kva.current_stream())
    first = _run(proj, x)                      # on poisoned scratch straight after create
    again = _run(proj, x)
    for i, (a, b) in enumerate(zip(first, again)):
        assert torch.isfinite(a).all(), i
        assert torch.equal(a, b), i
    proj.close()


def _guarded_outputs(cfg, n, guard=1024):
    """One int32 buffer: [guard][head 0][guard][head 1]...[guard], sentinel-filled."""
    sizes = [n * h["out_dim"] for h in cfg["heads"]]
    total = guard + sum(s + guard for s in sizes)
    buf = torch.full((total,), SENTINEL, dtype=torch.int32, device="cuda")
    outs, spans, off = [], [], guard
    for h, s in zip(cfg["heads"], sizes):
        outs.append(buf[off:off + s].view(torch.float32).view(n, h["out_dim"]))
        spans.append((off, off + s))
        off += s + guard
    return buf, outs, spans


@pytest.mark.parametrize("name,n", [("r2", 1024), ("r2", 700), ("r2", 37), ("tiny", 64), ("tiny", 45)])
def test_head_outputs_stay_inside_their_regions(name, n):
    cfg = synth.config(name)
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=n, seed=33)
    proj = kva.Projector(cfg, w, max_tokens=max(n, cfg["n_tokens"]))
    buf, outs, spans = _guarded_outputs(cfg, n)
    _run(proj, x, outs)
    proj.close()
    host = buf.cpu().numpy().view(np.uint32)
    inside = np.zeros(host.size, dtype=bool)
    for a, b in spans:
        inside[a:b] = True
    assert np.all(host[~inside] == SENTINEL), np.flatnonzero((host != SENTINEL) & ~inside)[:8]
    for i, (a, b) in enumerate(spans):
        assert not np.any(host[a:b] == SENTINEL), (i, int(np.sum(host[a:b] == SENTINEL)))


def _peaked(cfg, w, scale):
    return dict(w, blocks=[dict(b, wq=b["wq"] * np.float32(scale), wk=b["wk"] * np.float32(scale))
                           for b in w["blocks"]])


@pytest.mark.parametrize("scale", [1.0, 3.0])
def test_block_prefix_does_not_depend_on_later_tokens(scale):
    """One 1024-token attention block; with the Q and K weights scaled by 3
    a query's running maximum jumps between key tiles, at different tiles
    for different queries of one wave."""
    cfg = dict(synth.config("tiny"), attn_block=1024)
    w = _peaked(cfg, synth.make_weights(cfg), scale)
    x = synth.make_input(cfg, n_tokens=1024, seed=34)
    proj = kva.Projector(cfg, w, max_tokens=1024)
    full = [o.cpu() for o in _run(proj, x)]
    for n in (1, 5, 31, 32, 33, 47, 63, 64, 65, 100, 129, 511, 777, 1000, 1023):
        part = _run(proj, np.ascontiguousarray(x[:n]))
        for i, o in enumerate(part):
            assert torch.equal(o.cpu(), full[i][:n]), (scale, n, i)
    proj.close()


@pytest.mark.parametrize("j", [0, 100, 300, 340, 511])
def test_nan_reaches_only_later_tokens_of_its_block(j):
    block = 256
    cfg = dict(synth.config("tiny"), attn_block=block)
    w = synth.make_weights(cfg)
    x = synth.make_input(cfg, n_tokens=512, seed=35)
    proj = kva.Projector(cfg, w, max_tokens=512)
    clean = [o.cpu() for o in _run(proj, x)]
    xn = x.copy()
    xn[j, 7] = np.nan
    dirty = [o.cpu() for o in _run(proj, xn)]
    proj.close()
    bs, be, ts = (j // block) * block, (j // block + 1) * block, (j // 64) * 64
    for i, (a, b) in enumerate(zip(clean, dirty)):
        assert torch.isfinite(a).all(), i
        assert torch.isnan(b[j:be]).all(), (j, i)
        assert torch.equal(a[:ts], b[:ts]), (j, i)
        assert torch.equal(a[be:], b[be:]), (j, i)
        assert torch.isfinite(b[:ts]).all() and torch.isfinite(b[be:]).all(), (j, i)
    assert bs <= ts
