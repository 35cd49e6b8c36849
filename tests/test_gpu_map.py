"""GPU parity for the single-map projector (kva_map_create / kva_map_project)
against the float64 oracle (oracle/ref.py: map_project).

Bars (the projector's): max|y_gpu - y_ref| <= 2e-2 * RMS(y_ref) per map for
fp32/bf16 maps (input and weights rounded to bf16), 5e-2 for q8_0 / q4_0
(input rounded to fp16, weights d*q rounded to fp16).  Row independence is
bitwise: a call's first rows equal a shorter call's.
"""
import numpy as np
import pytest
import torch

import learned_kv_approximation_amd as kva
import synth
from oracle import ref

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _err(g, y):
    return float(np.max(np.abs(g.astype(np.float64) - y)) / np.sqrt(np.mean(y * y)))


@pytest.mark.parametrize("dtype,n_in,n_maps", [("f32", 256, 3), ("bf16", 512, 2), ("q8_0", 512, 2),
                                               ("q4_0", 256, 3)])
def test_map_parity_small(dtype, n_in, n_maps):
    maps, biases = synth.make_map_weights(n_in, n_maps, dtype)
    x = synth.make_map_input(1000, n_in)
    mp = kva.MapProjector(maps, biases, dtype=dtype, n_in=n_in, max_tokens=1000)
    xd = torch.from_numpy(x).cuda()
    tol = 5e-2 if dtype in ("q8_0", "q4_0") else 2e-2
    want_all = ref.map_project(x, maps, biases, dtype)
    for n in (40, 100, 1000):                      # 64-, 128- and 256-row tiles, ragged
        print(f"map {dtype} n_in={n_in} maps={n_maps} n={n}", flush=True)
        outs = mp.project(xd[:n])
        torch.cuda.synchronize()
        errs = [_err(o.cpu().numpy(), w[:n]) for o, w in zip(outs, want_all)]
        print("  max|err|/rms per map", [f"{e:.3e}" for e in errs], flush=True)
        assert max(errs) <= tol
        if n == 1000:
            full = [o.cpu().numpy() for o in outs]
    short = mp.project(xd[:100])
    torch.cuda.synchronize()
    assert all(np.array_equal(s.cpu().numpy(), f[:100]) for s, f in zip(short, full))
    mp.close()


def test_map_parity_full_width():
    """The benchmark's map shape (5120 wide) on two maps, one 1024-token call."""
    maps, biases = synth.make_map_weights(5120, 2, "bf16")
    x = synth.make_map_input(1024, 5120)
    mp = kva.MapProjector(maps, biases, dtype="bf16", max_tokens=1024)
    outs = mp.project(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    want = ref.map_project(x, maps, biases, "bf16")
    errs = [_err(o.cpu().numpy(), w) for o, w in zip(outs, want)]
    print("5120-wide maps: max|err|/rms", errs, flush=True)
    assert max(errs) <= 2e-2
    mp.close()


def test_map_argument_errors():
    maps, biases = synth.make_map_weights(256, 2, "bf16")
    with pytest.raises(kva.KvaError) as e:
        kva.kva_map_create(100, 2, kva.DTYPES["bf16"], [m.ctypes.data for m in maps], None, 64)
    assert e.value.status == kva.KVA_ERR_SHAPE
    with pytest.raises(kva.KvaError) as e:
        kva.kva_map_create(256, 2, 9, [m.ctypes.data for m in maps], None, 64)
    assert e.value.status == kva.KVA_ERR_DTYPE
    mp = kva.MapProjector(maps, None, dtype="bf16", max_tokens=64)
    x = torch.zeros((65, 256), device="cuda")
    with pytest.raises(kva.KvaError) as e:
        mp.project(x)
    assert e.value.status == kva.KVA_ERR_SHAPE
    # a map context is not a projector context, and the other way round
    with pytest.raises(kva.KvaError) as e:
        kva.kva_project_ubatch(mp.ctx, x.data_ptr(), 1, [x.data_ptr()])
    assert e.value.status == kva.KVA_ERR_UNSUPPORTED
    # no bias: zero input gives zero output
    out = mp.project(torch.zeros((3, 256), device="cuda"))
    torch.cuda.synchronize()
    assert all(not o.any() for o in out)
    mp.close()
