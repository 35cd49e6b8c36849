"""GPU: a seeded sweep over the call-level parameters of the tiny projector
(weight format, tokens per context, tokens per call, attention block size),
each case against the float64 oracle.  The combinations cross the kernel
choices a context makes (skinny trunk GEMM at <= 32 tokens per call, 64-row
tiles at <= 64, eight K ranges at <= 128, the tiled GEMM beyond) with ragged
token counts and blocks of 64..1024 tokens.

Bar: max|err| <= 2e-2 * RMS per head for f32 weights, 5e-2 for q8_0 / q4_0
(the projector's bars)."""
import numpy as np
import pytest
import torch

import learned_kv_approximation_amd as kva
import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cases(n=36, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = ("f32", "q8_0", "q4_0")[i % 3]
        max_tokens = int(rng.choice([16, 32, 48, 64, 100, 128, 200, 600]))
        n_tokens = int(rng.integers(1, max_tokens + 1))
        block = int(rng.choice([64, 128, 256, 1024]))
        out.append((dtype, max_tokens, n_tokens, block, int(rng.integers(0, 1 << 30))))
    return out


_WEIGHTS = {}


def _weights(dtype):
    if dtype not in _WEIGHTS:
        _WEIGHTS[dtype] = synth.make_weights(synth.config("tiny", weight_dtype=dtype))
    return _WEIGHTS[dtype]


@pytest.mark.parametrize("dtype,max_tokens,n_tokens,block,seed", _cases())
def test_tiny_sweep_against_oracle(dtype, max_tokens, n_tokens, block, seed):
    cfg = synth.config("tiny", weight_dtype=dtype, attn_block=block)
    w = _weights(dtype)
    x = synth.make_input(cfg, n_tokens=n_tokens, seed=seed)
    print(f"sweep: {dtype} max_tokens={max_tokens} n={n_tokens} block={block}", flush=True)
    proj = kva.Projector(cfg, w, max_tokens=max_tokens)
    outs = proj.project(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    got = [o.cpu().numpy().astype(np.float64) for o in outs]
    proj.close()
    want = oracle.project(cfg, w, x)
    tol = 2e-2 if dtype == "f32" else 5e-2
    for i, y in want.items():
        rms = np.sqrt(np.mean(y * y))
        err = float(np.max(np.abs(got[i] - y)) / rms)
        assert err <= tol, (cfg["heads"][i]["name"], err)
