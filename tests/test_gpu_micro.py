"""The fused small-batch path (MOE_FLAG_FUSED_SMALL_BATCH: at most 8 tokens,
bf16 activations, MXFP4 weights; routing and FC1 in one kernel, FC2 with the
weighted combine and the shared expert in another) against the oracle: routing bit-exact, the layer within
the output bar, at every batch size it takes, with a shared expert, expert
shards, precomputed top-k, the gated activation variants, E = 1024, bit-exact
repeats, graph replay and the allocation-free entry point."""
import numpy as np
import pytest
import torch

from block_scaled_precision_amd import inputs as gen
from oracle import moe as om
from tests.conftest import has_gpu
from tests.helpers import assert_y_close, gpu_weights, oracle_weights, print_flush

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

BASE = gen.scaled(gen.WORKLOADS["decode_w4a16"], T=8, H=1024, I=512, E=64, k=8)
SHARED = gen.scaled(BASE, I_shared=768, wfmt="e2m1", act="bf16")
WIDE_E = gen.scaled(BASE, T=2, E=1024, k=6, H=1024, I=256)
_cache = {}


def _prep(w):
    key = (w.H, w.I, w.E, w.I_shared)
    if key not in _cache:
        gw = gpu_weights(w)
        ow = oracle_weights(w)
        arrs = [np.stack([ow[e][i] for e in range(w.E)]) for i in range(4)]
        _cache[key] = (gw, arrs, ow.get("shared"))
    return _cache[key]


def _run(w, T, **kw):
    from block_scaled_precision_amd import moe_mx as m
    gw, arrs, shared = _prep(w)
    x = gen.hidden_states(w, T=T)
    logits = gen.router_logits(w, T=T)
    act_fn = kw.pop("act_fn", "silu")
    prob = m.make_problem(T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared, act_fn=act_fn,
                          shared_weight=kw.pop("shared_weight", 1.0), fused_small_batch=True)
    ids = torch.empty((T, w.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, w.k), dtype=torch.float32, device="cuda")
    y = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda(), topk_ids_out=ids, topk_w_out=wts)
    torch.cuda.synchronize()
    return m, gw, arrs, shared, x, logits, prob, ids, wts, y, act_fn


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 7, 8])
def test_small_batch_parity(T):
    m, gw, arrs, shared, x, logits, prob, ids, wts, y, _ = _run(BASE, T)
    print_flush(f"small batch T={T}")
    ref = om.moe_forward(x.double().numpy(), logits.numpy(), *arrs, k=BASE.k, wfmt=BASE.wfmt, act=BASE.act)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert np.max(np.abs(wts.cpu().numpy() - ref["w"])) <= 1e-6
    mr, rr = assert_y_close(y.float().cpu().numpy(), ref["y"], f"T={T}")
    print_flush(f"  max_rel={mr:.2e} rms_rel={rr:.2e}")


@pytest.mark.parametrize("T,sw,act_fn", [(1, 1.0, "silu"), (4, 0.375, "silu"), (8, -2.0, "relu2"),
                                         (3, 1.0, "swiglu_oai")])
def test_small_batch_shared_expert(T, sw, act_fn):
    m, gw, arrs, shared, x, logits, prob, ids, wts, y, _ = _run(SHARED, T, shared_weight=sw, act_fn=act_fn)
    print_flush(f"small batch T={T} shared_weight={sw} {act_fn}")
    ref = om.moe_forward(x.double().numpy(), logits.numpy(), *arrs, k=SHARED.k, wfmt=SHARED.wfmt, act=SHARED.act,
                         shared=shared, shared_weight=sw, act_fn=act_fn)
    assert_y_close(y.float().cpu().numpy(), ref["y"], f"T={T} shared")


@pytest.mark.parametrize("act_fn", ["relu2", "swiglu_oai"])
def test_small_batch_activations(act_fn):
    m, gw, arrs, shared, x, logits, prob, ids, wts, y, _ = _run(BASE, 6, act_fn=act_fn)
    ref = om.moe_forward(x.double().numpy(), logits.numpy(), *arrs, k=BASE.k, wfmt=BASE.wfmt, act=BASE.act,
                         act_fn=act_fn)
    assert_y_close(y.float().cpu().numpy(), ref["y"], f"T=6 {act_fn}")


def test_small_batch_many_experts():
    """E = 1024 (16 key slots per lane in the in-kernel top-k)."""
    m, gw, arrs, shared, x, logits, prob, ids, wts, y, _ = _run(WIDE_E, 2)
    ref = om.moe_forward(x.double().numpy(), logits.numpy(), *arrs, k=WIDE_E.k, wfmt=WIDE_E.wfmt, act=WIDE_E.act)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_y_close(y.float().cpu().numpy(), ref["y"], "E=1024")


@pytest.mark.parametrize("T,L", [(5, 16), (8, 8)])
def test_small_batch_expert_shards(T, L):
    from block_scaled_precision_amd import moe_mx as m
    gw, arrs, shared = _prep(BASE)
    x = gen.hidden_states(BASE, T=T)
    logits = gen.router_logits(BASE, T=T)
    parts = []
    for r in range(BASE.E // L):
        sl = slice(r * L, (r + 1) * L)
        shard = m.MoeWeights(gw.w1[sl], gw.w1_scale[sl], gw.w2[sl], gw.w2_scale[sl], BASE.wfmt)
        prob = m.make_problem(T, BASE.H, BASE.I, BASE.E, BASE.k, BASE.wfmt, BASE.act, local_offset=r * L,
                              local_count=L, fused_small_batch=True)
        yp = m.moe_fused(prob, x.cuda(), shard, router_logits=logits.cuda()).float().cpu().numpy()
        refp = om.moe_forward(x.double().numpy(), logits.numpy(), *arrs, k=BASE.k, wfmt=BASE.wfmt, act=BASE.act,
                              local_offset=r * L, local_count=L)["y"]
        if np.abs(refp).max() == 0:
            assert np.abs(yp).max() == 0
        else:
            assert_y_close(yp, refp, f"T={T} shard {r}")
        parts.append(yp.astype(np.float64))
    full = om.moe_forward(x.double().numpy(), logits.numpy(), *arrs, k=BASE.k, wfmt=BASE.wfmt, act=BASE.act)["y"]
    assert_y_close(sum(parts), full, f"T={T} shard sum")


def test_small_batch_precomputed_topk_and_repeat():
    from block_scaled_precision_amd import moe_mx as m
    T = 7
    gw, arrs, shared = _prep(BASE)
    x = gen.hidden_states(BASE, T=T).cuda()
    logits = gen.router_logits(BASE, T=T).cuda()
    prob = m.make_problem(T, BASE.H, BASE.I, BASE.E, BASE.k, BASE.wfmt, BASE.act, fused_small_batch=True)
    y1 = m.moe_fused(prob, x, gw, router_logits=logits)
    ids, wts, _, _ = m.moe_route(logits, BASE.k)
    y2 = m.moe_fused(prob, x, gw, topk_ids_in=ids, topk_w_in=wts)
    y3 = m.moe_fused(prob, x, gw, router_logits=logits)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_small_batch_graph_replay_and_noalloc():
    from block_scaled_precision_amd import moe_mx as m
    T = 4
    gw, arrs, shared = _prep(BASE)
    xs = [gen.hidden_states(BASE, T=T).cuda(), gen.hidden_states(BASE, seed=1, T=T).cuda()]
    ls = [gen.router_logits(BASE, T=T).cuda(), gen.router_logits(BASE, seed=1, T=T).cuda()]
    prob = m.make_problem(T, BASE.H, BASE.I, BASE.E, BASE.k, BASE.wfmt, BASE.act, fused_small_batch=True)
    xb, lb = xs[0].clone(), ls[0].clone()
    y = torch.empty((T, BASE.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((m.moe_fused_workspace_bytes(prob),), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        m.moe_fused(prob, xb, gw, router_logits=lb, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        m.moe_fused(prob, xb, gw, router_logits=lb, y=y, workspace=ws)
    for rep in range(4):
        i = rep % 2
        xb.copy_(xs[i])
        lb.copy_(ls[i])
        g.replay()
        got = y.clone()
        eager = m.moe_fused(prob, xs[i], gw, router_logits=ls[i])
        yn = torch.empty_like(eager)
        m.moe_fused_noalloc(prob, xs[i], gw, yn, router_logits=ls[i])
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        assert torch.equal(yn.view(torch.int16), eager.view(torch.int16)), f"noalloc {rep}"
    ref = om.moe_forward(xs[1].cpu().double().numpy(), ls[1].cpu().numpy(), *arrs, k=BASE.k, wfmt=BASE.wfmt,
                         act=BASE.act)
    assert_y_close(got.float().cpu().numpy(), ref["y"], "graph replay")


def test_default_path_small_batches():
    """Without the flag, batches of at most 16 tokens take the general path
    with top-k and the permutation in one workgroup: routing bit-exact and y
    within the bar, with precomputed top-k equal to the router's."""
    from block_scaled_precision_amd import moe_mx as m
    gw, arrs, shared = _prep(BASE)
    for T in (1, 5, 8):
        x = gen.hidden_states(BASE, T=T)
        logits = gen.router_logits(BASE, T=T)
        prob = m.make_problem(T, BASE.H, BASE.I, BASE.E, BASE.k, BASE.wfmt, BASE.act)
        ids = torch.empty((T, BASE.k), dtype=torch.int32, device="cuda")
        wts = torch.empty((T, BASE.k), dtype=torch.float32, device="cuda")
        y = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda(), topk_ids_out=ids, topk_w_out=wts)
        r_ids, r_w, r_off, r_sa = m.moe_route(logits.cuda(), BASE.k)
        torch.cuda.synchronize()
        ref = om.moe_forward(x.double().numpy(), logits.numpy(), *arrs, k=BASE.k, wfmt=BASE.wfmt, act=BASE.act)
        assert np.array_equal(ids.cpu().numpy(), ref["ids"]) and np.array_equal(r_ids.cpu().numpy(), ref["ids"])
        assert np.max(np.abs(wts.cpu().numpy() - ref["w"])) <= 1e-6
        assert np.array_equal(r_off.cpu().numpy(), ref["offsets"]) and np.array_equal(r_sa.cpu().numpy(),
                                                                                          ref["sorted_assign"])
        assert_y_close(y.float().cpu().numpy(), ref["y"], f"default path T={T}")


def test_fused_small_batch_rejects_what_it_cannot_take():
    from block_scaled_precision_amd import moe_mx as m
    gw, arrs, shared = _prep(BASE)
    x = gen.hidden_states(BASE, T=9).cuda()
    logits = gen.router_logits(BASE, T=9).cuda()
    prob = m.make_problem(9, BASE.H, BASE.I, BASE.E, BASE.k, BASE.wfmt, BASE.act, fused_small_batch=True)
    with pytest.raises(m.MoeError, match="unsupported"):
        m.moe_fused(prob, x, gw, router_logits=logits)


def _draw(n, seed=20261207):
    """Seeded random problems inside the path's limits: 1-8 tokens with at
    most 64 assignments, H a multiple of 512, I and I_shared of 256, every
    gated activation, a shared expert in half of them."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        T = int(rng.integers(1, 9))
        E = int(rng.choice([1, 5, 16, 64, 200]))
        k = int(rng.integers(1, min(E, 64 // T, 8) + 1))
        H = 512 * int(rng.integers(1, 5))
        I = 256 * int(rng.integers(1, 5))
        Is = int(rng.choice([0, 256 * int(rng.integers(1, 4))]))
        act_fn = str(rng.choice(["silu", "relu2", "swiglu_oai"]))
        w = gen.Workload(f"micro_random{i}", T, H, I, E, k, "e2m1", "bf16", I_shared=Is)
        cases.append(pytest.param(w, act_fn, id=f"{i}_T{T}_H{H}_I{I}_E{E}_k{k}_Is{Is}_{act_fn}"))
    return cases


@pytest.mark.parametrize("w,act_fn", _draw(16))
def test_random_problem(w, act_fn):
    from block_scaled_precision_amd import moe_mx as m
    gw = gpu_weights(w)
    ow = oracle_weights(w)
    arrs = [np.stack([ow[e][i] for e in range(w.E)]) for i in range(4)]
    x = gen.hidden_states(w)
    logits = gen.router_logits(w)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared, act_fn=act_fn,
                          fused_small_batch=True)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    print_flush(f"small batch random {w.name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} Is={w.I_shared} {act_fn}")
    y = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda(), topk_ids_out=ids)
    torch.cuda.synchronize()
    ref = om.moe_forward(x.double().numpy(), logits.numpy(), *arrs, k=w.k, wfmt=w.wfmt, act=w.act,
                         shared=ow.get("shared"), act_fn=act_fn)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert_y_close(y.float().cpu().numpy(), ref["y"], w.name)
