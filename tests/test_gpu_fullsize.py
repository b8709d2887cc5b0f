"""Full-size parity: each large workload at its benchmark shape, through the
same entry point and launch configuration that bench.py times.

* routing ids of every token are bit-exact against the oracle, and weights
  agree to 1e-6;
* the permutation (moe_route at the same size) is bit-exact;
* the layer output is checked on sampled tokens: each token's output depends
  only on its own row and the experts it routes to, so the oracle computes
  those rows alone, decoding only the experts they use.

Weights are drawn in fp32 on the GPU by the seeded generator; the library
quantizes them on the GPU and the oracle quantizes the same fp32 values on the
CPU (neither side sees the other's codes).
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_amd import inputs as gen
from oracle import moe as om
from oracle.routing import permute, topk_route
from tests.conftest import has_gpu
from tests.helpers import ExpertArrays, assert_y_close, gpu_weights, oracle_weights, print_flush

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

# sampled tokens per workload (first, last, and one in between)
SAMPLES = {
    "decode_w4a16": [0, 41],
    "prefill_w4a8": [0, 5000, 8191],
    "skew_w4a16": [0, 4095],
    "w6a8_shared": [0, 2047],
}


@pytest.mark.parametrize("name", list(SAMPLES))
def test_full_size_layer(name):
    from block_scaled_precision_amd import moe_mx as m

    w = gen.WORKLOADS[name]
    print_flush(f"full-size {name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} {w.wfmt}/{w.act} Is={w.I_shared}")
    gw = gpu_weights(w, device="cuda", fp32_on="cuda")
    logits = gen.router_logits(w, device="cuda")
    x = gen.hidden_states(w, device="cuda")
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    y = m.moe_fused(prob, x, gw, router_logits=logits, topk_ids_out=ids, topk_w_out=wts)
    r_ids, r_w, r_off, r_sa = m.moe_route(logits, w.k)
    torch.cuda.synchronize()

    # routing of every token, and the permutation, bit-exact
    lg = logits.cpu().numpy()
    o_ids, o_w = topk_route(lg, w.k)
    assert np.array_equal(ids.cpu().numpy(), o_ids)
    assert np.max(np.abs(wts.cpu().numpy().astype(np.float64) - o_w)) <= 1e-6
    _, o_off, o_sa = permute(o_ids, w.E)
    assert np.array_equal(r_ids.cpu().numpy(), o_ids)
    assert np.array_equal(r_off.cpu().numpy(), o_off)
    assert np.array_equal(r_sa.cpu().numpy(), o_sa)

    # layer output on sampled tokens
    toks = SAMPLES[name]
    experts = sorted(set(int(e) for e in o_ids[toks].ravel()))
    ow = oracle_weights(w, experts=experts, fp32_on="cuda")
    arrs = tuple(ExpertArrays({e: ow[e][i] for e in experts}, w.E) for i in range(4))
    ref = om.moe_forward(x.to(torch.float64).cpu().numpy(), lg, *arrs, k=w.k, wfmt=w.wfmt, act=w.act,
                         shared=ow.get("shared"), tokens=toks)
    got = y[toks].float().cpu().numpy()
    mr, rr = assert_y_close(got, ref["y"], f"{name} tokens {toks}")
    print_flush(f"  tokens {toks}: {len(experts)} experts, max_rel={mr:.3e} rms_rel={rr:.3e}")
    del gw, y
    torch.cuda.empty_cache()
