"""The measurement probes on the GPU: each runs, fills its output, and the
MFMA and k-step loops scale with their iteration count (the flop counts the
ceilings are computed from assume a fixed time per round)."""
import pytest
import torch

from rankmixer_token_mixing_amd import binding as bd

pytestmark = pytest.mark.gpu


def _timed(fn):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    e1.synchronize()
    return e0.elapsed_time(e1)


def test_mfma_and_kstep_probes_run_and_scale():
    lib = bd.load()
    frags = torch.randn(lib.rm_probe_mfma_frag_bytes() // 2, device="cuda").to(torch.bfloat16)
    out = torch.full((lib.rm_probe_mfma_out_floats(),), float("nan"), device="cuda")
    slab = torch.randn(lib.rm_probe_kstep_slab_bytes() // 2, device="cuda").to(torch.bfloat16)
    kout = torch.full((lib.rm_probe_kstep_out_floats(),), float("nan"), device="cuda")
    bd.probe_mfma_bf16(frags, out, 4)
    bd.probe_kstep_bf16(slab, kout, 4)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and torch.isfinite(kout).all()
    assert (out != 0).any() and (kout != 0).any()
    for run in (lambda n: bd.probe_mfma_bf16(frags, out, n), lambda n: bd.probe_kstep_bf16(slab, kout, n)):
        run(50)
        short = min(_timed(lambda: run(100)) for _ in range(3))
        long = min(_timed(lambda: run(400)) for _ in range(3))
        assert 2.5 < long / short < 5.0, (short, long)


def test_copy_probe_copies():
    n = (8 << 20) + 48
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    bd.probe_copy(src, dst, n)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
