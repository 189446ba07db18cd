"""GPU: the routing step without a workspace (rm_moe_route_noalloc, the
library's fixed scratch array) against rm_moe_route with a caller workspace,
through the C ABI, on two calls in a row -- the second smaller, so it runs
over scratch the first call left behind.  Gates, list offsets and row lists
must agree bit for bit (the same kernels; integer work is exact)."""
import numpy as np
import pytest
import torch

import synthetic_inputs as si
from tests.gpu_util import ensure_lib, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_lib()


def _route_inputs(B, T, D, E, seed):
    from rankmixer_token_mixing_amd import binding as bd
    rng = np.random.default_rng(seed)
    s = bd.to_device(si.to_bf16_bits(rng.standard_normal((B, T, D)).astype(np.float32)))
    wr = bd.to_device(si.to_bf16_bits((rng.standard_normal((T, E, D)) / np.sqrt(D)).astype(np.float32)))
    br = bd.to_device((0.1 * rng.standard_normal((T, E))).astype(np.float32))
    return s, wr, br


def test_noalloc_route_matches_the_workspace_route_twice():
    from rankmixer_token_mixing_amd import binding as bd
    lib = bd.load()
    assert lib.rm_moe_route_noalloc_max_scratch_bytes() == 16 << 20
    for i, (B, T, D, E) in enumerate([(2048, 16, 768, 8), (333, 4, 64, 5)]):
        note(f"[gpu] rm_moe_route_noalloc call {i + 1}: B={B} T={T} D={D} E={E}")
        assert lib.rm_moe_route_noalloc_scratch_bytes(B, T, E) <= lib.rm_moe_route_noalloc_max_scratch_bytes()
        s, wr, br = _route_inputs(B, T, D, E, seed=10 + i)
        g_ref, o_ref, r_ref = bd.rm_moe_route(s, wr, br)
        gates = torch.full((B, T, E), float("nan"), dtype=torch.float32, device="cuda")
        offsets = torch.full((T * E + 1,), -7, dtype=torch.int32, device="cuda")
        rows = torch.full((B * T * E,), -7, dtype=torch.int32, device="cuda")
        bd.rm_moe_route_noalloc(s, wr, br, gates, offsets, rows)
        torch.cuda.synchronize()
        assert torch.equal(gates.view(torch.int32), g_ref.view(torch.int32))
        assert torch.equal(offsets, o_ref)
        n = int(o_ref[-1])
        assert 0 < n < B * T * E
        assert torch.equal(rows[:n], r_ref[:n])

