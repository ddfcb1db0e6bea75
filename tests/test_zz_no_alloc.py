"""The allocation-free decode entry point (moe_forward_decode_noalloc)
against moe_forward_decode with its own workspace, through the C ABI.

Both run the same kernels on the same inputs, so results must agree bit for
bit: ids, weights and outputs.  Two calls in a row on one GPU share the
library's scratch; the second has a smaller input, so stale contents of the
first call are present while it runs.
"""

import numpy as np
import pytest

import synth
from layers import make_layer

torch = pytest.importorskip("torch")
M = pytest.importorskip("quantized_expert_ffn_route_amd")

pytestmark = pytest.mark.gpu

MID = synth.LayerSpec(hidden=512, inter=256, n_experts=32, top_k=4, has_shared=True, act="bf16",
                      n_slots=(8, 16, 8))


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _both(tl, x, y_dt):
    d, L = tl.dl.d, tl.dl.c_struct()
    T, H, K = x.shape[0], tl.spec.hidden, tl.spec.top_k
    ydt = torch.float32 if y_dt == M.MOE_F32 else torch.bfloat16
    out = []
    for fn in ("ws", "noalloc"):
        y = torch.full((T, H), float("nan"), dtype=ydt, device="cuda")
        ids = torch.full((T, K), -7, dtype=torch.int32, device="cuda")
        w = torch.full((T, K), float("nan"), dtype=torch.float32, device="cuda")
        xd = _dev(x)
        if fn == "ws":
            M.forward_decode(d, L, xd, y, y_dt, ids, w)
        else:
            M.forward_decode_noalloc(d, L, xd, y, y_dt, ids, w)
        torch.cuda.synchronize()
        out.append((y, ids, w))
    return out


@pytest.mark.parametrize("y_dt", ["f32", "bf16"])
def test_noalloc_matches_workspace_entry(y_dt):
    ydt = M.MOE_F32 if y_dt == "f32" else M.MOE_BF16
    tl = make_layer(MID, seed=30)
    full = make_layer(synth.FULL, seed=3, source="codes", n_calib=1024)
    # larger first, then smaller inputs: the scratch keeps the earlier contents
    for layer, T, seed in ((tl, 21, 300), (tl, 5, 301), (full, 3, 302), (full, 1, 303)):
        x = synth.tokens(layer.spec, T, seed)
        print(f"  noalloc vs ws: H={layer.spec.hidden} T={T} y={y_dt}", flush=True)
        (ya, ia, wa), (yb, ib, wb) = _both(layer, x, ydt)
        assert torch.equal(ia, ib)
        assert torch.equal(wa.view(torch.int32), wb.view(torch.int32))
        assert torch.equal(ya.view(torch.int16) if ya.dtype == torch.bfloat16 else ya.view(torch.int32),
                           yb.view(torch.int16) if yb.dtype == torch.bfloat16 else yb.view(torch.int32))
