"""GPU: kva_map_project_noalloc (the single-map projection whose residual
copy lives in the library's static device array) against kva_map_project on
the same context, bit for bit: two calls in a row, the second smaller, so
the second runs on what the first left in the shared array; then the size
limit."""
import numpy as np
import pytest
import torch

import learned_kv_approximation_amd as kva
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dtype,n_in,n_maps,sizes", [("bf16", 5120, 3, (1024, 300)), ("q8_0", 512, 2, (700, 65)),
                                                     ("f32", 256, 3, (200, 1))])
def test_noalloc_equals_map_project(dtype, n_in, n_maps, sizes):
    maps, biases = synth.make_map_weights(n_in, n_maps, dtype)
    mp = kva.MapProjector(maps, biases, dtype=dtype, n_in=n_in, max_tokens=1536)
    s = kva.current_stream()
    for k, n in enumerate(sizes):
        x = torch.from_numpy(synth.make_map_input(n, n_in, seed=40 + k)).cuda()
        ref_out = [torch.empty((n, n_in), dtype=torch.float32, device="cuda") for _ in range(n_maps)]
        got = [torch.full((n, n_in), float("nan"), dtype=torch.float32, device="cuda") for _ in range(n_maps)]
        kva.kva_map_project(mp.ctx, x.data_ptr(), n, [o.data_ptr() for o in ref_out], s)
        kva.kva_map_project_noalloc(mp.ctx, x.data_ptr(), n, [o.data_ptr() for o in got], s)
        torch.cuda.synchronize()
        for i in range(n_maps):
            assert torch.isfinite(ref_out[i]).all(), (n, i)
            assert torch.equal(got[i], ref_out[i]), (dtype, n, i)
    mp.close()


def test_noalloc_rejects_sizes_past_its_array():
    maps, biases = synth.make_map_weights(5120, 1, "bf16")
    mp = kva.MapProjector(maps, biases, dtype="bf16", n_in=5120, max_tokens=2048)
    x = torch.zeros((1537, 5120), dtype=torch.float32, device="cuda")
    out = torch.empty((1537, 5120), dtype=torch.float32, device="cuda")
    with pytest.raises(kva.KvaError) as e:
        kva.kva_map_project_noalloc(mp.ctx, x.data_ptr(), 1537, [out.data_ptr()], kva.current_stream())
    assert e.value.status == kva.KVA_ERR_SHAPE
    kva.kva_map_project_noalloc(mp.ctx, x.data_ptr(), 1536, [out.data_ptr()], kva.current_stream())
    torch.cuda.synchronize()
    mp.close()
