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
    # more than one token block and more than 32 experts: the multi-block scan's totals
    "decode_w4a16_e96": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=200, H=512, I=256, E=96),
    "prefill_w4a8_e40": gen.scaled(gen.WORKLOADS["prefill_w4a8"], T=500, H=1024, I=512, E=40, k=4),
    # a few tokens: routing inside FC1 (and the fused small-batch path on request)
    "decode_w4a16_t4": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=4, H=512, I=256, E=48),
    # the small-M FC1 routing the batch itself: one token over 384 experts (six
    # top-k key slots per lane, scale groups of 4 stages), and 16 tokens with
    # 128 assignments (its limits)
    "decode_w4a16_t1_e384": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=1, H=1024, I=256, E=384),
    "decode_w4a16_t16": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=16, H=512, I=512, E=64),
    # FC1 routing with one expert per token, and with E not a multiple of 64
    # (four key slots per lane, the last partly past E)
    "decode_w4a16_t16_k1": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=16, H=512, I=256, E=8, k=1),
    "decode_w4a16_t3_e200": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=3, H=512, I=256, E=200, k=6),
    # one token routed to 100 of 100 experts: more slots than one 64-lane
    # selection round, so the routing kernels route it
    "decode_w4a16_t1_k100": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=1, H=512, I=256, E=100, k=100),
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
    # the small-M kernel with K a multiple of 1024 (scale groups of 4 stages in
    # FC1 and FC2, the instantiation the decode workload runs)
    "w4a16_small_gs4": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=32, H=1024, I=1024, E=8, k=4),
    # the small-M kernel in dense mode (a bf16 shared expert over fewer than 32 tokens)
    "w4a16_small_shared": gen.scaled(gen.WORKLOADS["decode_w4a16"], T=24, H=512, I=256, E=8, k=2,
                                     I_shared=512),
    # the wide kernel with whole M-tiles per XCD and the N-block split of the
    # last ntiles % 8 tiles in one launch, where a persistent workgroup streams
    # an item of each part (FC1: 32 N-blocks; FC2: 24 N-blocks)
    "w4a8_wide_full_tail_fc1": gen.scaled(gen.WORKLOADS["prefill_w4a8"], T=800, H=1024, I=4096, E=6, k=2),
    "w4a8_wide_full_tail_fc2": gen.scaled(gen.WORKLOADS["prefill_w4a8"], T=800, H=6144, I=1024, E=6, k=2),
    # E3M2 weights with bf16 activations (the stream kernels), with a shared expert
    "w6a16_shared": gen.scaled(gen.WORKLOADS["w6a8_shared"], T=50, H=512, I=256, E=8, k=2, I_shared=256,
                               act="bf16"),
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


# one case per kernel family: small-M, mid-M, tiled (+ shared), wide, stream
@pytest.mark.parametrize("name", ["w4a16_small_gs4", "skew_w4a16_mid", "w6a8_shared_small",
                                  "w4a8_wide_multi_tile", "w4a8_h384", "decode_w4a16_t4"])
def test_repeat_is_bit_identical(name):
    """The same call twice gives the same bits: every output row has one
    writer and the combine adds the slots in a fixed order."""
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared)
    print_flush(f"moe_fused {name} twice")
    y1 = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda())
    y2 = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda())
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# the shared expert's weight through each kernel family's dense FC2 epilogue:
# tiled, wide, mid-M, small-M, stream
@pytest.mark.parametrize("name,sw", [("w6a8_shared_small", 0.375), ("w4a8_wide_shared", -2.0),
                                     ("w4a16_mid_shared", 0.375), ("w4a16_small_shared", -2.0),
                                     ("w6a16_shared", 0.375)])
def test_shared_weight(name, sw):
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared, shared_weight=sw)
    print_flush(f"moe_fused {name} shared_weight={sw}")
    y = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda())
    torch.cuda.synchronize()
    ref = _oracle_y(w, arrs, shared, x, logits, shared_weight=sw)
    assert_y_close(y.float().cpu().numpy(), ref["y"], f"{name} shared_weight={sw}")


# the gated activations (b12x page, "What's in here", MoE) through each kernel
# family's FC1 epilogue: small-M, mid-M, tiled (+ shared), wide, stream
@pytest.mark.parametrize("act_fn", ["relu2", "swiglu_oai"])
@pytest.mark.parametrize("name", ["w4a16_small_gs4", "skew_w4a16_mid", "w6a8_shared_small",
                                  "w4a8_wide_multi_tile", "w4a8_h384", "w6a16_shared"])
def test_activation_variants(name, act_fn):
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared, act_fn=act_fn)
    print_flush(f"moe_fused {name} act_fn={act_fn}")
    y = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda())
    torch.cuda.synchronize()
    ref = _oracle_y(w, arrs, shared, x, logits, act_fn=act_fn)
    mr, rr = assert_y_close(y.float().cpu().numpy(), ref["y"], f"{name} {act_fn}")
    print_flush(f"  max_rel={mr:.2e} rms_rel={rr:.2e}")


def _wide_schedule_parts(counts, nb, grid=256):
    """For the wide kernel's persistent schedule on `grid` workgroups: number of
    tiles, whole tiles per XCD, and whether some workgroup streams an item of
    the whole-tile part and then an item of the tail part."""
    ntiles = int(sum((c + 191) // 192 for c in counts))
    full, Q = ntiles // 8, grid // 8
    tail_items = (ntiles % 8) * nb
    mixed = False
    for x in range(8):
        t0 = tail_items * x // 8
        n = full * nb + tail_items * (x + 1) // 8 - t0
        for q in range(Q):
            js = range(q, n, Q)
            mixed |= any(j < full * nb for j in js) and any(j >= full * nb for j in js)
    return ntiles, full, mixed


@pytest.mark.parametrize("name,fc1", [("w4a8_wide_full_tail_fc1", True), ("w4a8_wide_full_tail_fc2", False)])
def test_wide_schedule_case_covers_both_parts(name, fc1):
    """The wide cases above exercise the transition from whole tiles to the
    tail split inside one workgroup's item stream (on 256 CUs)."""
    w = CASES[name]
    from oracle.routing import permute, topk_route
    ids, _ = topk_route(gen.router_logits(w).numpy(), w.k)
    counts, _, _ = permute(ids, w.E)
    nb = w.I // 128 if fc1 else w.H // 256
    ntiles, full, mixed = _wide_schedule_parts(counts, nb)
    assert full >= 1 and ntiles % 8 != 0 and mixed, (ntiles, full, mixed)
    if torch.cuda.is_available():
        assert torch.cuda.get_device_properties(0).multi_processor_count == 256


@pytest.mark.parametrize("name", ["prefill_w4a8_small", "w4a8_wide_multi_tile", "w6a8_shared_small", "w4a8_h384",
                                  "decode_w4a16_small", "skew_w4a16_mid", "w6a16_shared"])
def test_intermediate_flip_rate(name):
    """The FC2 input the device leaves in its workspace against the oracle's:
    routing, offsets and the permutation are bit-exact; the intermediate codes
    come from fp32 h on the device and fp64 h in the oracle, so a few may land
    on the other side of a rounding or scale boundary.  Reports the rate of
    such flips and bounds it."""
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared)
    ws = torch.empty((m.moe_fused_workspace_bytes(prob),), dtype=torch.uint8, device="cuda")
    print_flush(f"moe_fused {name}: intermediates")
    m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda(), workspace=ws)
    torch.cuda.synchronize()
    ref = _oracle_y(w, arrs, shared, x, logits, intermediates=True)
    A, L = w.T * w.k, w.E

    def part(name_, nbytes):
        o = m.moe_fused_workspace_offset(prob, name_)
        return ws[o:o + nbytes].cpu().numpy()

    off = part("expert_offsets", 4 * (L + 1)).view(np.int32)
    sa = part("sorted_assign", 4 * A).view(np.int32)
    assert np.array_equal(off, ref["offsets"]) and np.array_equal(sa, ref["sorted_assign"])
    inter = ref["intermediates"]
    if w.act == "mxfp8":
        codes = part("h", A * w.I).reshape(A, w.I)
        scales = part("h_scale", A * w.I // 32).reshape(A, w.I // 32)
        oc = np.stack([inter[int(a)][0] for a in sa])
        osc = np.stack([inter[int(a)][1] for a in sa])
        code_flips = float(np.mean(codes != oc))
        scale_flips = float(np.mean(scales != osc))
        print_flush(f"  {name}: E4M3 code flips {code_flips:.2e}, E8M0 scale flips {scale_flips:.2e}")
        # a flip is a value on the other side of one rounding boundary: the
        # block scales differ by at most one step, and each decoded value by
        # one E4M3 step (1/8 of the larger magnitude) plus what fp32
        # accumulation error can reach near zero (2**-12 of the block's
        # largest value); a misplaced or wrong value would be off by O(1)
        # of the block maximum
        from oracle.mx import dequantize
        assert np.abs(scales.astype(int) - osc.astype(int)).max() <= 1
        gv, ov = dequantize(codes, scales, "e4m3"), dequantize(oc, osc, "e4m3")
        bmax = np.repeat(np.abs(ov).reshape(A, -1, 32).max(axis=2), 32, axis=1)
        tol = np.maximum(np.abs(gv), np.abs(ov)) / 8 + bmax * 2.0 ** -12
        worst = float(np.max(np.abs(gv - ov) / np.where(tol > 0, tol, 1.0)))
        print_flush(f"  largest difference / (one step + 2**-12 block max): {worst:.3f}")
        assert worst <= 1.0
        assert code_flips <= 5e-3 and scale_flips <= 5e-3
    else:
        h = part("h", A * w.I * 2).view(np.uint16).reshape(A, w.I)
        from oracle.mx import bf16_bits_to_f64
        got = bf16_bits_to_f64(h)
        want = np.stack([inter[int(a)] for a in sa])
        flips = float(np.mean(got != want))
        print_flush(f"  {name}: bf16 intermediate flips {flips:.2e}")
        # each flip is one bf16 step (8 significant bits) plus what fp32
        # accumulation error can reach near zero (2**-14 of the row maximum)
        rmax = np.abs(want).max(axis=1, keepdims=True)
        tol = np.maximum(np.abs(got), np.abs(want)) * 2.0 ** -7 + rmax * 2.0 ** -14
        worst = float(np.max(np.abs(got - want) / np.where(tol > 0, tol, 1.0)))
        print_flush(f"  largest difference / (one step + 2**-14 row max): {worst:.3f}")
        assert worst <= 1.0
        assert flips <= 5e-3


def _tp_slice(t, r, n, fmt, what):
    """Shard r of n of one expert-stacked weight (torch or numpy) along I:
    W1 keeps gate rows and up rows [r I/n, (r+1) I/n); W2 keeps those columns
    of its packed codes / scales (I/n is a multiple of 32, so MX blocks stay
    whole)."""
    lib = torch if isinstance(t, torch.Tensor) else np
    if what in ("w1", "s1"):
        I = t.shape[-2] // 2
        c = I // n
        out = lib.cat([t[..., r * c:(r + 1) * c, :], t[..., I + r * c:I + (r + 1) * c, :]], -2) if lib is torch \
            else np.concatenate([t[..., r * c:(r + 1) * c, :], t[..., I + r * c:I + (r + 1) * c, :]], -2)
    else:
        c = t.shape[-1] // n
        out = t[..., r * c:(r + 1) * c]
    return out.contiguous() if lib is torch else np.ascontiguousarray(out)


# TokenSpeed SiTU page, "Supported contract": a tensor-parallel rank holds a
# slice of the intermediate size of every expert and returns a partial output
# that the caller all-reduces
@pytest.mark.parametrize("name,n", [("decode_w4a16_small", 2), ("decode_w4a16_t4", 2), ("prefill_w4a8_small", 4),
                                    ("w6a8_shared_small", 2), ("w4a8_wide_full_tail_fc1", 2)])
def test_tensor_parallel_shards_sum_to_full_layer(name, n):
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    parts = []
    for r in range(n):
        Ir, Isr = w.I // n, w.I_shared // n
        names = ("w1", "s1", "w2", "s2")
        g = [_tp_slice(t, r, n, w.wfmt, k) for t, k in zip((gw.w1, gw.w1_scale, gw.w2, gw.w2_scale), names)]
        sw = m.MoeWeights(*g, w.wfmt)
        o_arrs = [_tp_slice(a, r, n, w.wfmt, k) for a, k in zip(arrs, names)]
        o_shared = None
        if w.I_shared:
            sw.ws1, sw.ws1_scale, sw.ws2, sw.ws2_scale = [
                _tp_slice(t, r, n, w.wfmt, k) for t, k in zip((gw.ws1, gw.ws1_scale, gw.ws2, gw.ws2_scale), names)]
            o_shared = tuple(_tp_slice(a, r, n, w.wfmt, k) for a, k in zip(shared, names))
        prob = m.make_problem(w.T, w.H, Ir, w.E, w.k, w.wfmt, w.act, I_shared=Isr)
        print_flush(f"moe_fused {name} TP rank {r}/{n}: I={Ir} I_shared={Isr}")
        yp = m.moe_fused(prob, x.cuda(), sw, router_logits=logits.cuda()).float().cpu().numpy()
        wr = gen.scaled(w, I=Ir, I_shared=Isr)
        refp = _oracle_y(wr, o_arrs, o_shared, x, logits)["y"]
        assert_y_close(yp, refp, f"{name} TP rank {r}")
        parts.append(yp.astype(np.float64))
    full = _oracle_y(w, arrs, shared, x, logits)["y"]
    assert_y_close(sum(parts), full, f"{name} TP shard sum")


@pytest.mark.parametrize("name,fused", [("decode_w4a16_small", False), ("decode_w4a16_t4", False),
                                        ("decode_w4a16_t4", True), ("w6a8_shared_small", False),
                                        ("w4a8_wide_multi_tile", False)])
def test_graph_capture_and_replay(name, fused):
    """moe_fused captured in a HIP graph (torch.cuda.graph) and replayed: every
    replay, with new inputs copied in and eager work between replays, matches
    the eager call on the same inputs bit for bit, and the oracle."""
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared, fused_small_batch=fused)
    xs = [x.cuda(), (x.float() * -0.5).to(torch.bfloat16).cuda()]
    ls = [logits.cuda(), logits.flip(0).contiguous().cuda()]
    xb, lb = xs[0].clone(), ls[0].clone()
    y = torch.empty((w.T, w.H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((m.moe_fused_workspace_bytes(prob),), dtype=torch.uint8, device="cuda")
    print_flush(f"moe_fused {name}: graph capture")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm up outside the capture
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
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        if rep < 2:
            ref = _oracle_y(w, arrs, shared, xs[i].cpu(), ls[i].cpu())
            assert_y_close(got.float().cpu().numpy(), ref["y"], f"{name} graph replay {rep}")


@pytest.mark.parametrize("name", ["decode_w4a16_small", "decode_w4a16_t4", "prefill_w4a8_small",
                                  "w6a8_shared_small"])
def test_precomputed_topk_matches_router(name):
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared)
    ids, wts, _, _ = m.moe_route(logits.cuda(), w.k)
    print_flush(f"moe_fused {name} with precomputed top-k")
    y = m.moe_fused(prob, x.cuda(), gw, topk_ids_in=ids, topk_w_in=wts).float().cpu().numpy()
    torch.cuda.synchronize()
    ref = _oracle_y(w, arrs, shared, x, None, topk_ids=ids.cpu().numpy(), topk_w=wts.cpu().numpy())
    assert_y_close(y, ref["y"], f"precomputed {name}")


# few tokens on the small-M kernel: FC1 routes the batch in its prologue
@pytest.mark.parametrize("name,shard", [("decode_w4a16_t4", None), ("decode_w4a16_t1_e384", None),
                                        ("decode_w4a16_t16", None), ("decode_w4a16_t4", (12, 12)),
                                        ("decode_w4a16_t1_e384", (100, 200)), ("decode_w4a16_t16_k1", None),
                                        ("decode_w4a16_t3_e200", None), ("decode_w4a16_t3_e200", (50, 120))])
def test_routing_in_fc1_matches_routing_kernels(name, shard):
    """The routing that the few-token FC1 computes itself (top-k outputs,
    the expert offsets and permuted assignments it leaves in the workspace)
    and the layer output equal, bit for bit, those of the path that takes the
    routing kernels' top-k as input; and y is within the bar of the oracle."""
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    off, L = shard if shard else (0, 0)
    if shard:
        sl = slice(off, off + L)
        gw = m.MoeWeights(gw.w1[sl], gw.w1_scale[sl], gw.w2[sl], gw.w2_scale[sl], w.wfmt)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=0, local_offset=off, local_count=L)
    ids, wts, _, _ = m.moe_route(logits.cuda(), w.k)
    need = m.moe_fused_workspace_bytes(prob)
    runs = {}
    for how in ("logits", "topk_in"):
        ws = torch.full((need,), 0xAB, dtype=torch.uint8, device="cuda")
        ids_o = torch.full((w.T, w.k), -1, dtype=torch.int32, device="cuda")
        w_o = torch.full((w.T, w.k), -1.0, dtype=torch.float32, device="cuda")
        print_flush(f"moe_fused {name} shard {shard}: routing from {how}")
        if how == "logits":
            y = m.moe_fused(prob, x.cuda(), gw, router_logits=logits.cuda(), workspace=ws, topk_ids_out=ids_o,
                            topk_w_out=w_o)
        else:
            y = m.moe_fused(prob, x.cuda(), gw, topk_ids_in=ids, topk_w_in=wts, workspace=ws, topk_ids_out=ids_o,
                            topk_w_out=w_o)
        torch.cuda.synchronize()
        nl = L if shard else w.E
        o = m.moe_fused_workspace_offset(prob, "expert_offsets")
        offs = ws[o:o + 4 * (nl + 1)].cpu().numpy().view(np.int32)
        o = m.moe_fused_workspace_offset(prob, "sorted_assign")
        sa = ws[o:o + 4 * int(offs[-1])].cpu().numpy().view(np.int32)
        runs[how] = (y.cpu(), ids_o.cpu(), w_o.cpu(), offs, sa)
    (y1, i1, w1, o1, s1), (y2, i2, w2, o2, s2) = runs["logits"], runs["topk_in"]
    assert torch.equal(i1, ids.cpu()) and torch.equal(w1, wts.cpu())
    assert torch.equal(i2, ids.cpu()) and torch.equal(w2, wts.cpu())
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    assert torch.equal(y1, y2)
    ref = _oracle_y(w, arrs, None, x, logits, local_offset=off, local_count=L if shard else None)
    assert_y_close(y1.float().numpy(), ref["y"], f"routed FC1 {name}")


# (case, experts per shard) over the small-M, tiled (with a shared expert)
# and wide kernels; the shared expert, when there is one, is added by shard 0
@pytest.mark.parametrize("name,L", [("decode_w4a16_small", 12), ("decode_w4a16_t4", 12), ("prefill_w4a8_small", 4),
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


def test_few_token_shard_without_assignments_is_zero():
    """The same for a few tokens, whose FC1 routes the batch itself: a shard
    of experts with -inf logits (never selected) gets no tile, FC1 and FC2
    run no item, and y is exactly zero."""
    w, gw, arrs, shared, x, logits, m = _prepare("decode_w4a16_t4")
    off, L = w.E - 8, 8
    logits = logits.clone()
    logits[:, off:] = float("-inf")
    shard = m.MoeWeights(gw.w1[off:], gw.w1_scale[off:], gw.w2[off:], gw.w2_scale[off:], w.wfmt)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, local_offset=off, local_count=L)
    ids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
    y = torch.full((w.T, w.H), 7.0, dtype=torch.bfloat16, device="cuda")
    print_flush("moe_fused few-token shard of unselected experts")
    m.moe_fused(prob, x.cuda(), shard, router_logits=logits.cuda(), topk_ids_out=ids, y=y)
    torch.cuda.synchronize()
    assert not ((ids.cpu().numpy() >= off).any())
    assert torch.count_nonzero(y).item() == 0


@pytest.mark.parametrize("name", ["decode_w4a16_t4", "w6a8_shared_small"])
def test_prepared_call_matches_moe_fused(name):
    """FusedCall (arguments checked and marshalled once) gives the bits of
    moe_fused, also after new contents are written into the same buffers."""
    w, gw, arrs, shared, x, logits, m = _prepare(name)
    prob = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, I_shared=w.I_shared)
    xg, lg = x.cuda(), logits.cuda()
    call = m.FusedCall(prob, xg, gw, router_logits=lg)
    print_flush(f"FusedCall {name}")
    for _ in range(2):
        y = call().clone()
        y_ref = m.moe_fused(prob, xg, gw, router_logits=lg)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
        xg.copy_(torch.flip(xg, [0]))
        lg.copy_(torch.flip(lg, [1]))


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
