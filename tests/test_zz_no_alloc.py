"""moe_fused_noalloc (the entry point for callers that cannot allocate) against
moe_fused through the C ABI: two calls in a row on the library's static
scratch, the second with a smaller batch, each bit-identical to moe_fused
with a workspace of its own; a problem too large for the scratch is
rejected."""
import numpy as np
import pytest
import torch

from block_scaled_precision_amd import inputs as gen
from tests.conftest import has_gpu
from tests.helpers import gpu_weights, print_flush

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

# decode-shaped (small-M kernel), a few tokens (routing inside FC1; on request
# the fused small-batch path), and MXFP8 with a shared expert (tiled kernel)
CASES = {
    "decode": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=64, H=1024, I=512, E=32, k=8),
    "decode_few": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=8, H=1024, I=512, E=32, k=8),
    "w6a8_shared": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=96, H=512, I=512, E=8, k=4, I_shared=512),
}


@pytest.mark.parametrize("name,fused", [("decode", False), ("decode_few", False), ("decode_few", True),
                                        ("w6a8_shared", False)])
def test_noalloc_matches_workspace_entry_point(name, fused):
    from block_scaled_precision_amd import moe_mx as m
    w = CASES[name]
    gw = gpu_weights(w)
    x = gen.hidden_states(w).cuda()
    logits = gen.router_logits(w).cuda()
    for T in (w.T, w.T // 3):  # second call smaller
        prob = m.make_problem(T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared, fused_small_batch=fused)
        assert m.moe_fused_workspace_bytes(prob) <= m.NOALLOC_SCRATCH_BYTES
        print_flush(f"moe_fused_noalloc {name} T={T} fused={fused}")
        y_ref = m.moe_fused(prob, x[:T], gw, router_logits=logits[:T])
        y = torch.full((T, w.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        ids = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
        before = torch.cuda.memory_allocated()
        m.moe_fused_noalloc(prob, x[:T], gw, y, router_logits=logits[:T], topk_ids_out=ids)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"{name} T={T} fused={fused}"
        r_ids, _, _, _ = m.moe_route(logits[:T], w.k)
        assert torch.equal(ids, r_ids)


def test_noalloc_rejects_problems_beyond_the_scratch():
    from block_scaled_precision_amd import moe_mx as m
    w = gen.WORKLOADS["prefill_w4a8"]
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act)
    assert m.moe_fused_workspace_bytes(prob) > m.NOALLOC_SCRATCH_BYTES
    small = gen.scaled(w, E=8, H=1024, I=512, k=2)
    gw = gpu_weights(small)
    prob = m.make_problem(w.T, small.H, small.I, small.E, small.k, small.wfmt, small.act)
    x = torch.zeros((w.T, small.H), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((w.T, small.E), dtype=torch.float32, device="cuda")
    y = torch.empty((w.T, small.H), dtype=torch.bfloat16, device="cuda")
    need = m.moe_fused_workspace_bytes(prob)
    print_flush(f"moe_fused_noalloc over the scratch: needs {need} bytes")
    assert need > m.NOALLOC_SCRATCH_BYTES
    with pytest.raises(m.MoeError, match="workspace too small"):
        m.moe_fused_noalloc(prob, x, gw, y, router_logits=lg)
