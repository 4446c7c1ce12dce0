"""GPU: moe_route_static, the routing entry point that allocates nothing (its scratch is a static
device array inside the library), against moe_route with a caller workspace.

Both write the routing results into a `saved` buffer filled with the same NaN bit pattern
beforehand; the two buffers must then be byte-identical (untouched regions stay the pattern). Calls
run back to back with shrinking inputs, so each later call finds the previous call's contents in
the shared scratch; the routing results are also checked against the oracle's.
"""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_32_amd import binding

pytestmark = pytest.mark.gpu


def route_both(T, E, k, el, e0, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[:, :3] = np.round(lg[:, :3])                      # some exact ties
    d = binding.Desc.make(T, 256, 128, E, k, "bf16", el, e0)
    fwd, _, saved = binding.query_sizes(d)
    lgd = torch.from_numpy(lg).to("cuda")
    sa = torch.full((saved,), 0xFF, dtype=torch.uint8, device="cuda")
    sb = torch.full((saved,), 0xFF, dtype=torch.uint8, device="cuda")
    ws = torch.full((fwd,), 0xFF, dtype=torch.uint8, device="cuda")
    binding.moe_route(d, lgd, sa, ws, fwd)
    binding.moe_route_static(d, lgd, sb)
    torch.cuda.synchronize()
    a, b = sa.cpu().numpy(), sb.cpu().numpy()
    assert np.array_equal(a, b), f"saved differs at {np.nonzero(a != b)[0][:8]}"
    off = binding.saved_layout(d)
    r = oracle.route(lg, k, e0, el)
    rows = T * k
    idx = b[off["idx"]:off["idx"] + 4 * rows].view(np.int32).reshape(T, k)
    perm = b[off["perm"]:off["perm"] + 4 * rows].view(np.int32)
    counts = b[off["counts"]:off["counts"] + 4 * el].view(np.int32)
    assert np.array_equal(idx, r["idx"])
    assert np.array_equal(counts, r["counts"])
    assert np.array_equal(perm[:r["perm"].size], r["perm"])


@pytest.mark.parametrize("calls", [
    # (T, E, k, E_local, e0, seed), in call order: each later input is smaller
    [(16384, 128, 8, 128, 0, 1), (4000, 64, 16, 40, 10, 2), (333, 16, 4, 16, 0, 3)],
])
def test_route_static_matches_route_on_successive_calls(calls):
    for T, E, k, el, e0, seed in calls:
        print(f"case moe_route_static T={T} E={E} k={k} E_local={el} e0={e0}", flush=True)
        route_both(T, E, k, el, e0, seed)


def test_route_static_rejects_oversized_scratch():
    # 4096 blocks of 64 tokens at 128 local experts need 8,389,120 bytes: more than the 8 MiB array
    d = binding.Desc.make(4096 * 64, 256, 128, 128, 8, "bf16")
    with pytest.raises(binding.MoEError, match="MOE_ERR_UNSUPPORTED_SHAPE"):
        binding.moe_route_static(d, 1 << 20, 1 << 20, stream=0)
    d = binding.Desc.make(4095 * 64, 256, 128, 128, 8, "bf16")    # the largest that fits: accepted
    lg = torch.zeros(4095 * 64, 128, dtype=torch.float32, device="cuda")
    _, _, saved = binding.query_sizes(d)
    sv = torch.empty(saved, dtype=torch.uint8, device="cuda")
    binding.moe_route_static(d, lg, sv)
    torch.cuda.synchronize()
