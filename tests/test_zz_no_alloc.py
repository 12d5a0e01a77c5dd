"""spax_layer_step_static (the layer step that allocates nothing: its
scratch is the library's static device array) against spax_layer_step with
a caller workspace: bitwise equal outputs and tier lists, on two calls in a
row, the second with a smaller layer (the array keeps the first call's
contents)."""
import numpy as np
import pytest

import workloads as WL
from tests.spax_testlib import log, to_dev, to_host
from tests.test_gpu_layer import LayerWeights, _build_layer, _io, _ks

pytestmark = pytest.mark.gpu


def _outputs(L, out):
    res = {k: to_host(out[k]) for k in ("qkv", "o", "g", "u", "a", "down")}
    res["lists"] = [(to_host(out["F"][g])[:L.k_full[g]], to_host(out["A"][g])[:L.k_approx[g]])
                    for g in range(4)]
    return res


def _run(L, h, z, x, static):
    import torch

    import activation_sparse_decode_token_amd as spax
    io, out = _io(L, h, z, x)
    if static:
        spax.layer_step_static(L, io)
    else:
        ws = torch.zeros(spax.layer_workspace_bytes(L), dtype=torch.uint8, device="cuda:0")
        spax.layer_step(L, io, ws)
    torch.cuda.synchronize()
    return _outputs(L, out)


@pytest.mark.parametrize("kernel", [0, 2])
def test_static_layer_step_equals_workspace_call(kernel):
    # 7B-shaped layer, then a smaller one with ragged tiles
    for hidden, inter, cfg in ((4096, 11008, 4), (512, 1408, 810)):
        w = LayerWeights(cfg, 1, hidden, inter, 0.02)
        ks = _ks(hidden, inter, WL.TierSplit(50, 25, 25))
        L = _build_layer(w, "fp16", "int4", 0, ks, kernel)
        h = WL.laplace_fp16(cfg, 1, "h", 0, hidden)
        z = WL.laplace_fp16(cfg, 1, "z", 0, hidden)
        x = WL.laplace_fp16(cfg, 1, "x", 0, hidden)
        got = _run(L, h, z, x, static=True)
        want = _run(L, h, z, x, static=False)
        for k in ("qkv", "o", "g", "u", "a", "down"):
            assert np.array_equal(got[k].view(np.uint16), want[k].view(np.uint16)), \
                f"{hidden}: {k} differs from the workspace call"
        for g in range(4):
            for t in range(2):
                assert np.array_equal(got["lists"][g][t], want["lists"][g][t]), \
                    f"{hidden}: group {g} lists differ"
        log(f"static layer step, hidden {hidden}, kernel {kernel}: bitwise equal")
