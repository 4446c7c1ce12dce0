"""GPU routing with planted exact ties, bit-exact against the oracle's routing.

The routing contract: top-k of the fp32 logits ordered by (logit descending, expert index
ascending), so equal logits go to the lower expert index and -0.0 equals +0.0; pairs sorted by
(local expert, t*k + j). Expert indices, counts, offsets, the permutation and its inverse must
match oracle.route bit for bit; the routing weights within 1e-6 (equal logits: 1/k within 1e-7).
Top-8 of 128 experts is the pages' routing ("Os Números que Impressionam" on "IA: MoE Kernel 3x
Mais Rápido Chegou!"); ties are where a selection kernel most easily departs from the definition.

Both selection kernels are covered: k <= 8 (per-lane sorted lists merged across 8 lanes) and
k > 8 (one wavefront per token, k rounds of a wave-wide argmax), with E at, below and above 64
experts per lane.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_32_amd.layer import MoELayer

pytestmark = pytest.mark.gpu

ROW_KINDS = ("integers", "all_equal", "signed_zeros", "boundary_tie", "coarse_grid")


def tie_logits(T, E, k, seed):
    """[T, E] fp32 logits whose rows cycle through five kinds of exact ties (see ROW_KINDS)."""
    rng = np.random.default_rng(seed)
    lg = np.empty((T, E), np.float32)
    kinds = []
    for t in range(T):
        kind = ROW_KINDS[t % len(ROW_KINDS)]
        kinds.append(kind)
        if kind == "integers":                       # few distinct values: ties everywhere
            row = rng.integers(-3, 4, E).astype(np.float32)
        elif kind == "all_equal":                    # every expert ties; weights 1/k
            row = np.full(E, rng.choice([0.0, -0.0, 1.5, -2.25]), np.float32)
        elif kind == "signed_zeros":                 # fewer than k positives, then +0.0 and -0.0 mixed
            row = np.where(rng.random(E) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
            npos = int(rng.integers(0, max(1, k)))
            row[rng.choice(E, npos, replace=False)] = rng.integers(1, 3, npos).astype(np.float32)
            nneg = min(E - npos, int(rng.integers(0, E // 4 + 1)))
            free = np.nonzero(row <= 0)[0]
            row[rng.choice(free, nneg, replace=False)] = np.float32(-1.0)
        elif kind == "boundary_tie":                 # k-1 distinct leaders, then a tie group across slot k
            row = np.minimum(rng.standard_normal(E), 3.5).astype(np.float32)
            pos = rng.permutation(E)
            lead = min(k - 1, E)
            row[pos[:lead]] = 10.0 + np.arange(lead, dtype=np.float32)
            grp = pos[lead:lead + min(4, E - lead)]
            row[grp] = np.float32(5.0)
        else:                                        # normal values on a 1/4 grid
            row = (np.round(rng.standard_normal(E) * 4.0) / 4.0).astype(np.float32)
        lg[t] = row
    return lg, kinds


CASES = [
    # T, E, k, E_local, e0
    pytest.param(1000, 128, 8, 128, 0, id="E128_k8"),
    pytest.param(777, 8, 2, 8, 0, id="E8_k2"),
    pytest.param(300, 5, 5, 5, 0, id="E5_k5_all_chosen"),
    pytest.param(450, 33, 7, 33, 0, id="E33_k7"),
    pytest.param(600, 128, 8, 40, 50, id="E128_k8_share"),
    pytest.param(500, 512, 32, 512, 0, id="E512_k32_wave"),
    pytest.param(333, 64, 16, 64, 0, id="E64_k16_wave"),
    pytest.param(400, 200, 10, 200, 0, id="E200_k10_wave"),
    pytest.param(256, 96, 9, 96, 0, id="E96_k9_wave"),
    pytest.param(300, 512, 32, 100, 400, id="E512_k32_wave_share"),
]


@pytest.mark.parametrize("T,E,k,el,e0", CASES)
def test_routing_ties_bit_exact(T, E, k, el, e0):
    print(f"case route_ties T={T} E={E} k={k} E_local={el} e0={e0}", flush=True)
    lg, kinds = tie_logits(T, E, k, seed=1000 + E + k + e0)
    assert np.any(np.signbit(lg) & (lg == 0)), "the input must hold negative zeros"
    layer = MoELayer(T, 256, 128, E, k, "bf16", el, e0)
    layer.route(torch.from_numpy(lg).to("cuda"))
    torch.cuda.synchronize()
    got = {n: t.numpy() for n, t in layer.routing().items()}
    ref = oracle.route(lg, k, e0, el)
    assert np.array_equal(got["idx"], ref["idx"]), "expert indices differ"
    assert np.array_equal(got["counts"], ref["counts"]), "counts differ"
    assert np.array_equal(got["offsets"], ref["offsets"]), "offsets differ"
    assert np.array_equal(got["perm"], ref["perm"]), "permutation differs"
    assert np.array_equal(got["pair_pos"], ref["pair_pos"]), "inverse permutation differs"
    assert np.max(np.abs(got["weight"] - ref["w"])) <= 1e-6
    eq = np.array([kd == "all_equal" for kd in kinds])
    assert np.max(np.abs(got["weight"][eq] - 1.0 / k)) <= 1e-7
    # on all-equal rows the chosen experts are 0..k-1 in order
    assert np.array_equal(got["idx"][eq], np.broadcast_to(np.arange(k), (int(eq.sum()), k)))
