"""moe_route on the GPU against the oracle: ids, offsets and permutation bit-exact,
weights within 1e-6."""
import numpy as np
import pytest
import torch

from block_scaled_precision_amd import inputs as gen
from oracle.routing import permute, topk_route
from tests.conftest import has_gpu
from tests.helpers import print_flush

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]


def _run(logits_cpu: torch.Tensor, k: int):
    from block_scaled_precision_amd import moe_mx as m
    ids, w, off, sa = m.moe_route(logits_cpu.cuda(), k)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy(), off.cpu().numpy(), sa.cpu().numpy()


def _check(logits_cpu, k):
    E = logits_cpu.shape[1]
    gi, gw, go, gs = _run(logits_cpu, k)
    oi, ow = topk_route(logits_cpu.numpy(), k)
    _, oo, osa = permute(oi, E)
    assert np.array_equal(gi, oi)
    assert np.max(np.abs(gw - ow), initial=0.0) <= 1e-6
    assert np.array_equal(go, oo)
    assert np.array_equal(gs, osa)


@pytest.mark.parametrize("name", list(gen.WORKLOADS))
def test_workload_logits(name):
    w = gen.WORKLOADS[name]
    print_flush(f"moe_route {name} T={w.T} E={w.E} k={w.k}")
    _check(gen.router_logits(w), w.k)


@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (63, 384, 8), (65, 384, 8), (130, 17, 17), (7, 1024, 9),
                                   (200, 1024, 1), (300, 64, 64), (9, 200, 100), (5, 1024, 130),
                                   (64, 1024, 64), (64, 64, 1),
                                   # top-k and permutation in one launch: up to 16 tokens, k up to 64
                                   (16, 384, 8), (12, 1024, 64), (3, 1024, 1), (16, 64, 64), (17, 384, 8)])
def test_ties_and_shapes(T, E, k):
    g = torch.Generator().manual_seed(T * 131 + E)
    logits = (torch.randint(-4, 5, (T, E), generator=g) * 0.5).float()   # many exact ties
    print_flush(f"moe_route ties T={T} E={E} k={k}")
    _check(logits, k)


def _draw(n, seed=20261205):
    """Seeded random routing problems: T, E and k anywhere in the supported
    range, half of them with logits on a coarse grid (many exact ties)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        T = int(rng.choice([1, 2, 3, 8, 15, 16, 17, 31, 64, 65, 127, 500, 1000, 2049]))
        E = int(rng.integers(1, 1025))
        k = int(rng.integers(1, min(E, 160) + 1))
        ties = bool(rng.random() < 0.5)
        cases.append(pytest.param(T, E, k, ties, i, id=f"{i}_T{T}_E{E}_k{k}" + ("_ties" if ties else "")))
    return cases


@pytest.mark.parametrize("T,E,k,ties,i", _draw(32))
def test_random_shapes(T, E, k, ties, i):
    g = torch.Generator().manual_seed(1000 + i)
    logits = (torch.randint(-4, 5, (T, E), generator=g) * 0.5).float() if ties else torch.randn((T, E), generator=g)
    print_flush(f"moe_route random T={T} E={E} k={k} ties={ties}")
    _check(logits, k)


def test_minus_inf_and_empty():
    g = torch.Generator().manual_seed(3)
    logits = torch.randn((100, 40), generator=g)
    logits[:, 30:] = float("-inf")
    logits[::3, 5] = float("-inf")
    print_flush("moe_route -inf")
    _check(logits, 8)
    from block_scaled_precision_amd import moe_mx as m
    ids, w, off, sa = m.moe_route(torch.empty((0, 16), device="cuda"), 4)
    torch.cuda.synchronize()
    assert off.cpu().numpy().tolist() == [0] * 17 and sa.numel() == 0


def test_deterministic_repeat():
    g = torch.Generator().manual_seed(4)
    logits = torch.randn((4096, 128), generator=g)
    a = _run(logits, 8)
    b = _run(logits, 8)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
