"""moe_fused on the GPU against the oracle at sizes the oracle finishes in
seconds: every workload family, scaled down so that experts span several
16-row tiles and ragged tails; plus precomputed routing, expert shards and
degenerate batches."""
import numpy as np
import pytest
import torch

from block_scaled_precision_amd import inputs as gen
from oracle import moe as om
from tests.conftest import has_gpu
from tests.helpers import assert_y_close, gpu_weights, oracle_weights, print_flush

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

CASES = {
    "tiny_w4a16": gen.WORKLOADS["tiny_w4a16"],
    "decode_w4a16_small": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=64, H=512, I=256, E=48),
    "prefill_w4a8_small": gen.scaled(gen.WORKLOADS["prefill_w4a8"], T=300, H=512, I=512, E=16, k=4),
    "skew_w4a16_small": gen.scaled(gen.WORKLOADS["skew_w4a16"], T=256, H=256, I=256, E=32, k=4),
    "w6a8_shared_small": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=100, H=512, I=512, E=24, k=6,
                                    I_shared=512),
    "w6a8_no_shared": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=33, H=256, I=128, E=8, k=3, I_shared=0),
    "w4a8_single_token": gen.scaled(gen.WORKLOADS["prefill_w4a8"], T=1, H=256, I=128, E=8, k=2),
    # several 192-row M-tiles per expert with a ragged last tile (the tiled
    # kernel: K a multiple of 512 but below the wide kernel's 1024)
    "w4a8_multi_tile": gen.scaled(gen.WORKLOADS["prefill_w4a8"], T=700, H=512, I=512, E=4, k=2),
    "w6a8_multi_tile_shared": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=300, H=512, I=512, E=2, k=2,
                                         I_shared=512),
    # enough (M-tile, N-block) items that every persistent workgroup of the
    # tiled GEMMs streams several of them back to back
    "w4a8_stream_items": gen.scaled(gen.WORKLOADS["prefill_w4a8"], T=512, H=2048, I=1024, E=32, k=4),
    "w6a8_stream_items": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=512, H=2048, I=1024, E=32, k=4,
                                    I_shared=1024),
    # the wide E2M1 kernel (K multiples of 512, at least 1024) with two M-tiles
    # per expert, the second ragged
    "w4a8_wide_multi_tile": gen.scaled(gen.WORKLOADS["prefill_w4a8"], T=600, H=1024, I=1024, E=4, k=2),
    # the wide kernel in dense mode: an E2M1 shared expert next to routed experts
    "w4a8_wide_shared": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=256, H=1024, I=1024, E=8, k=2,
                                   I_shared=1024, wfmt="e2m1"),
    # the wide kernel with one expert per token (token index = assignment id)
    "w4a8_wide_k1": gen.scaled(gen.WORKLOADS["prefill_w4a8"], T=400, H=1024, I=1024, E=4, k=1),
    # a dense shared expert with more FC1 items than workgroups: on 256 CUs its
    # FC1 takes 128-row tiles with 256-row N-blocks and its FC2 192-row tiles
    # with 128-row N-blocks (smaller inputs take 192-row tiles for both)
    "w6a8_shared_fc1_items": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=1024, H=512, I=512, E=8, k=2,
                                        I_shared=4096),
    # the tiled kernel with 128-row M-tiles (experts average at most 96 rows)
    # under skewed routing: some experts span several tiles, two get none
    "w6a8_low_rows_skew": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=256, H=512, I=512, E=16, k=4,
                                     I_shared=0, skew=True),
    # MXFP8 activations with H not a multiple of 512: the 16-row stream kernels
    # instead of the tiled or wide ones
    "w4a8_h384": gen.scaled(gen.WORKLOADS["prefill_w4a8"], T=200, H=384, I=256, E=4, k=2),
    # bf16 activations, experts averaging at least 32 rows: the 64-row mid-M
    # kernel; skewed routing gives experts of several M-tiles, ragged tails and
    # two experts with no rows
    "skew_w4a16_mid": gen.scaled(gen.WORKLOADS["skew_w4a16"], T=512, H=1024, I=512, E=16, k=4),
    # the mid-M kernel over many items per workgroup
    "w4a16_mid_items": gen.scaled(gen.WORKLOADS["skew_w4a16"], T=1024, H=2048, I=1024, E=8, k=4),
    # the mid-M kernel in dense mode (bf16 shared expert, last M-tile of 8 rows)
    "w4a16_mid_shared": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=200, H=512, I=512, E=4, k=2,
                                   I_shared=1024, wfmt="e2m1", act="bf16"),
    # 64-row mid-M tiles (experts averaging 32 to 96 rows) under skewed routing,
    # and in dense mode for a shared expert over fewer than 96 tokens
    "skew_w4a16_mid64": gen.scaled(gen.WORKLOADS["skew_w4a16"], T=256, H=1024, I=512, E=16, k=4),
    "w4a16_mid64_shared": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=80, H=512, I=512, E=2, k=1,
                                     I_shared=512, wfmt="e2m1", act="bf16"),
    # the mid-M kernel with one expert per token (token index = assignment id)
    "w4a16_mid_k1": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=300, H=512, I=1024, E=4, k=1),
    # bf16 activations with I not a multiple of 256: the 16-row stream kernels
    "w4a16_k384": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=40, H=384, I=384, E=8, k=2),
}

_cache = {}


def _prepare(name):
    if name in _cache:
        return _cache[name]
    w = CASES[name]
    from block_scaled_precision_amd import moe_mx as m
    gw = gpu_weights(w)
    ow = oracle_weights(w)
    # the two quantizers must agree bit for bit on every weight
    for e in range(w.E):
        for i, gt in enumerate((gw.w1, gw.w1_scale, gw.w2, gw.w2_scale)):
            assert np.array_equal(gt[e].cpu().numpy(), ow[e][i]), (name, e, i)
    if w.I_shared:
        for i, gt in enumerate((gw.ws1, gw.ws1_scale, gw.ws2, gw.ws2_scale)):
            assert np.array_equal(gt.cpu().numpy(), ow["shared"][i])
    x = gen.hidden_states(w)
    logits = gen.router_logits(w)
    arrs = [np.stack([ow[e][i] for e in range(w.E)]) for i in range(4)]
    shared = ow.get("shared")
    _cache[name] = (w, gw, arrs, shared, x, logits, m)
    return _cache[name]


def _oracle_y(w, arrs, shared, x, logits, **kw):
    return om.moe_forward(x.to(torch.float64).numpy(), None if logits is None else logits.numpy(),
                          *arrs, k=w.k, wfmt=w.wfmt, act=w.act, shared=shared, **kw)


@pytest.mark.parametrize("name", list(CASES))
def test_layer_parity(name):
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    print_flush(f"moe_fused {name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} {w.wfmt}/{w.act} Is={w.I_shared}")
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    wts = torch.empty((w.T, w.k), dtype=torch.float32, device="cuda")
    y = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda(), topk_ids_out=ids, topk_w_out=wts)
    torch.cuda.synchronize()
    ref = _oracle_y(w, arrs, shared, x, logits)
    assert np.array_equal(ids.cpu().numpy(), ref["ids"])
    assert np.max(np.abs(wts.cpu().numpy() - ref["w"])) <= 1e-6
    mr, rr = assert_y_close(y.float().cpu().numpy(), ref["y"], name)
    print_flush(f"  max_rel={mr:.2e} rms_rel={rr:.2e}")


def test_repeat_is_stable():
    """Same call twice: ids identical, y equal up to the fp32 accumulation order."""
    w, gw, arrs, shared, x, logits, m = _prepare("prefill_w4a8_small")
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act)
    y1 = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda()).float().cpu().numpy()
    y2 = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda()).float().cpu().numpy()
    d = np.abs(y1 - y2).max() / np.abs(y1).max()
    assert d < 1e-2


@pytest.mark.parametrize("name", ["decode_w4a16_small", "prefill_w4a8_small", "w6a8_shared_small"])
def test_precomputed_topk_matches_router(name):
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared)
    ids, wts, _, _ = m.moe_route(logits.cuda(), w.k)
    print_flush(f"moe_fused {name} with precomputed top-k")
    y = m.moe_fused(prob, x.cuda(), gw, topk_ids_in=ids, topk_w_in=wts).float().cpu().numpy()
    torch.cuda.synchronize()
    ref = _oracle_y(w, arrs, shared, x, None, topk_ids=ids.cpu().numpy(), topk_w=wts.cpu().numpy())
    assert_y_close(y, ref["y"], f"precomputed {name}")


# (case, experts per shard) over the small-M, tiled (with a shared expert)
# and wide kernels; the shared expert, when there is one, is added by shard 0
@pytest.mark.parametrize("name,L", [("decode_w4a16_small", 12), ("prefill_w4a8_small", 4),
                                    ("w6a8_shared_small", 8), ("w4a8_wide_multi_tile", 2)])
def test_expert_shards_sum_to_full_layer(name, L):
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    parts = []
    for r in range(w.E // L):
        sl = slice(r * L, (r + 1) * L)
        own_shared = r == 0 and w.I_shared > 0
        extra = (gw.ws1, gw.ws1_scale, gw.ws2, gw.ws2_scale) if own_shared else ()
        shard = m.MoeWeights(gw.w1[sl], gw.w1_scale[sl], gw.w2[sl], gw.w2_scale[sl], w.wfmt, *extra)
        prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared if own_shared else 0,
                              local_offset=r * L, local_count=L)
        print_flush(f"moe_fused {name} shard {r}")
        yp = m.moe_fused(prob, x.cuda(), shard, router_logits=logits.cuda()).float().cpu().numpy()
        refp = _oracle_y(w, arrs, shared if own_shared else None, x, logits, local_offset=r * L,
                         local_count=L)["y"]
        assert_y_close(yp, refp, f"{name} shard {r}")
        parts.append(yp.astype(np.float64))
    full = _oracle_y(w, arrs, shared, x, logits)["y"]
    assert_y_close(sum(parts), full, f"{name} shard sum")


def test_shard_without_assignments_is_zero():
    """A shard whose experts no token selects (the skewed router's two -inf
    experts): empty tile lists for the tiled GEMMs, and y exactly zero."""
    w, gw, arrs, shared, x, logits, m = _prepare("w6a8_low_rows_skew")
    off, L = w.E - 2, 2
    shard = m.MoeWeights(gw.w1[off:], gw.w1_scale[off:], gw.w2[off:], gw.w2_scale[off:], w.wfmt)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, local_offset=off, local_count=L)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    print_flush("moe_fused shard of unselected experts")
    y = m.moe_fused(prob, x.cuda(), shard, router_logits=logits.cuda(), topk_ids_out=ids)
    torch.cuda.synchronize()
    assert not np.isin(ids.cpu().numpy(), [off, off + 1]).any()
    assert torch.count_nonzero(y).item() == 0


def test_zero_tokens_is_noop():
    w, gw, arrs, shared, x, logits, m = _prepare("tiny_w4a16")
    prob = m.make_problem(0, w.H, w.I, w.E, w.k, w.wfmt, w.act)
    y = m.moe_fused(prob, x.cuda()[:0], gw, router_logits=logits.cuda()[:0])
    torch.cuda.synchronize()
    assert y.shape == (0, w.H)


def test_output_guard_bytes_untouched():
    """y is written exactly: canary values around it survive."""
    w, gw, arrs, shared, x, logits, m = _prepare("tiny_w4a16")
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act)
    buf = torch.full((w.T * w.H + 2 * 64,), 12345.0, dtype=torch.bfloat16, device="cuda")
    y = buf[64:64 + w.T * w.H].view(w.T, w.H)
    m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda(), y=y)
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:64] == 12345.0) and torch.all(b[-64:] == 12345.0)
    ref = _oracle_y(w, arrs, shared, x, logits)
    assert_y_close(y.float().cpu().numpy(), ref["y"], "guarded")
