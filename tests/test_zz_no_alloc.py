"""Allocation-free triangle attention (pairattn_tri_fwd_noalloc) on the GPU.

Its workspace is the library's static per-device scratch instead of a
caller buffer; the same kernels run, so its output must equal that of
pairattn_tri_fwd bit for bit.  Two calls in a row, the second smaller (so
the scratch still holds the first call's larger problem), then an fp32 call:
each against pairattn_tri_fwd on the same inputs.
"""
import numpy as np
import pytest

from pair_representation_attention_amd import device, inputs, lib

CASES = [
    # I, dtype, mask, orientation, seed
    (384, "bf16", "pad", lib.PAIRATTN_START, 2),     # the padded workload's shape
    (100, "bf16", "random", lib.PAIRATTN_END, 5),       # smaller, ragged, other orientation
    (64, "f32", "none", lib.PAIRATTN_START, 1),         # the fp32 workload's shape
]


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_on_consecutive_calls():
    torch = pytest.importorskip("torch")
    assert torch.cuda.is_available()
    for I, dt, mask, ori, seed in CASES:
        print(f"[noalloc] I={I} dtype={dt} mask={mask} orientation={ori} seed={seed}", flush=True)
        case = inputs.make_tri_case(I=I, c=128, H=4, d=32, dtype=dt, mask=mask, seed=seed, affine=True, biases=True)
        p = case.params_start if ori == lib.PAIRATTN_START else case.params_end
        run = device.TriRunner(case.z, case.mask, p, 4, dt)
        ref = run(ori).clone()
        out = torch.full_like(run.out, float("nan"))
        prm = device.make_params(p, dt)          # weights only: no workspace
        assert prm.workspace is None
        lib.pairattn_tri_fwd_noalloc(run.z, run.mask, prm, out, I, 128, 4, 32, ori)
        torch.cuda.synchronize()
        same = torch.equal(out.view(torch.int16) if dt == "bf16" else out.view(torch.int32),
                           ref.view(torch.int16) if dt == "bf16" else ref.view(torch.int32))
        diff = (out.float() - ref.float()).abs().max().item()
        print(f"[noalloc]   bitwise equal: {same}, max |diff| {diff:.3e}", flush=True)
        assert same, f"I={I} {dt}: allocation-free output differs from pairattn_tri_fwd (max {diff})"
        assert np.isfinite(out.float().cpu().numpy()).all()
        del run, prm, out, ref


@pytest.mark.gpu
def test_noalloc_rejects_oversized_before_device_work():
    torch = pytest.importorskip("torch")
    case = inputs.make_tri_case(I=8, c=128, H=4, d=32, dtype="bf16", mask="none", seed=3)
    prm = device.make_params(case.params_start, "bf16")
    z = torch.zeros((1,), device="cuda")
    st = lib.pairattn_tri_fwd_noalloc(z, None, prm, z.data_ptr() + (1 << 30), 600, 128, 4, 32, 0, check=False)
    assert st == lib.PAIRATTN_ERR_UNSUPPORTED and "scratch" in lib.last_error()
