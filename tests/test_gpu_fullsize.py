"""Full-size parity: each large workload at its benchmark shape, through the
same entry point and launch configuration that bench.py times.

* routing ids of every token are bit-exact against the oracle, and weights
  agree to 1e-6;
* the permutation (moe_route at the same size) is bit-exact;
* the layer output: the whole decode batch (every token, every active
  expert); for the larger batches, tokens chosen to reach the parts of the
  launch that small cases do not: each expert's ragged second M-tile, the
  M-tiles whose N-blocks the wide kernel splits across XCDs, the hot expert
  of the skewed router, plus the first and last token.  Each token's output
  depends only on its own row and its experts, so the oracle computes those
  rows alone, one job per expert.

Weights are drawn in fp32 on the GPU by the seeded generator; the library
quantizes them on the GPU and the oracle quantizes the same fp32 values on the
CPU (neither side sees the other's codes).  The decode and prefill workloads
share one weight set, so both sides quantize it once.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_amd import inputs as gen
from oracle.routing import permute, topk_route
from tests.conftest import has_gpu
from tests.helpers import assert_y_close, gpu_weights, oracle_rows, print_flush

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

NAMES = ["decode_w4a16", "decode_t1", "decode_t2", "decode_t4", "decode_t8", "prefill_w4a8", "skew_w4a16",
         "w6a8_shared"]
# the decode shapes at batches of 1 to 8 tokens (the small-batch path)
SMALL = {f"decode_t{T}": gen.scaled(gen.WORKLOADS["decode_w4a16"], name=f"decode_t{T}", T=T) for T in (1, 2, 4, 8)}
_oracle_cache = {}
_gpu = {}


def _gpu_weights(w):
    key = (w.H, w.I, w.E, w.wfmt, w.I_shared)
    if key not in _gpu:
        _gpu.clear()
        torch.cuda.empty_cache()
        _gpu[key] = gpu_weights(w, device="cuda", fp32_on="cuda")
    return _gpu[key]


def _tile_tokens(ids, E, k, bm):
    """Tokens in (a) the last M-tile of every expert with more than one tile of
    `bm` rows, (b) every tile of the last ntiles % 8 of the tile list (tiles
    ordered by expert, then row): the rows of the token of a tile's last row."""
    counts, offsets, sa = permute(ids, E)
    tiles = []  # (first permuted row, rows)
    for e in range(E):
        for p0 in range(int(offsets[e]), int(offsets[e + 1]), bm):
            tiles.append((p0, min(bm, int(offsets[e + 1]) - p0), e))
    pick = set()
    for e in range(E):
        et = [t for t in tiles if t[2] == e]
        if len(et) > 1:
            p0, r, _ = et[-1]
            pick.add(int(sa[p0 + r - 1]) // k)
    for p0, r, _ in tiles[len(tiles) - len(tiles) % 8:]:
        pick.add(int(sa[p0 + r - 1]) // k)
    return sorted(pick), len(tiles)


def _sample(name, w, o_ids):
    T = w.T
    if name == "decode_w4a16" or name in SMALL:
        return list(range(T))
    if name == "prefill_w4a8":
        toks, ntiles = _tile_tokens(o_ids, w.E, w.k, 192)
        print_flush(f"  {ntiles} M-tiles of 192 rows; {len(toks)} tokens in ragged second tiles or XCD-split tiles")
        return sorted(set(toks) | {0, T // 2, T - 1})
    if name == "skew_w4a16":
        # the hot expert's last (ragged) 128-row tile and a token of a cold expert
        counts, offsets, sa = permute(o_ids, w.E)
        hot = int(np.argmax(counts))
        cold = int(np.argmin(np.where(counts > 0, counts, 1 << 30)))
        last = int(sa[offsets[hot + 1] - 1]) // w.k
        first_cold = int(sa[offsets[cold]]) // w.k
        return sorted({0, last, first_cold, T - 1})
    return [0, 1000, T - 1]


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("name", NAMES)
def test_full_size_layer(name):
    from block_scaled_precision_amd import moe_mx as m

    w = SMALL[name] if name in SMALL else gen.WORKLOADS[name]
    print_flush(f"full-size {name}: T={w.T} H={w.H} I={w.I} E={w.E} k={w.k} {w.wfmt}/{w.act} Is={w.I_shared}")
    gw = _gpu_weights(w)
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
    if name == "skew_w4a16":
        counts = np.diff(o_off)
        top = np.sort(counts)[::-1]
        print_flush(f"  expert histogram: top-10 take {top[:10].sum() / counts.sum():.1%} of assignments; "
                    f"largest {top[:5].tolist()}; experts with none: {np.flatnonzero(counts == 0).tolist()}")

    # layer output on the sampled tokens
    toks = _sample(name, w, o_ids)
    n_exp = len(set(o_ids[toks].ravel().tolist()))
    print_flush(f"  oracle on {len(toks)} tokens ({n_exp} experts)")
    ref = oracle_rows(w, x[toks].cpu(), o_ids[toks], o_w[toks], fp32_on="cuda", cache=_oracle_cache)
    got = y[toks].float().cpu().numpy()
    mr, rr = assert_y_close(got, ref, f"{name} tokens {toks[:8]}...")
    print_flush(f"  {len(toks)} tokens, {n_exp} experts: max_rel={mr:.3e} rms_rel={rr:.3e}")
    if name in SMALL:
        # the fused small-batch path on the same batch
        pf = m.make_problem(w.T, w.H, w.I, w.E, w.k, w.wfmt, w.act, fused_small_batch=True)
        fids = torch.empty((w.T, w.k), dtype=torch.int32, device="cuda")
        yf = m.moe_fused(pf, x, gw, router_logits=logits, topk_ids_out=fids)
        torch.cuda.synchronize()
        assert np.array_equal(fids.cpu().numpy(), o_ids)
        mr, rr = assert_y_close(yf.float().cpu().numpy(), ref, f"{name} fused small batch")
        print_flush(f"  fused small-batch path: max_rel={mr:.3e} rms_rel={rr:.3e}")
    del y
    if name == NAMES[-1]:
        _gpu.clear()
        _oracle_cache.clear()
        torch.cuda.empty_cache()
