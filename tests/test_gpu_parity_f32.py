"""GPU parity of the fp32 path (fp16-pair operands on the matrix cores)
against the fp64 oracle, through the C ABI.  Bar: max abs error <= 1e-4.

Run on an MI355X:  python -m pytest tests -m gpu
"""
import numpy as np
import pytest

import oracle
from pair_representation_attention_amd import inputs
from parity_common import check, gpu_to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from pair_representation_attention_amd import lib
    lib.load()   # raises if the HIP library is missing: no fallback
    yield


def _dev():
    from pair_representation_attention_amd import device
    return device


@pytest.mark.parametrize("c,H", [(64, 4), (64, 8), (128, 8), (256, 4), (256, 8)])
def test_f32_other_widths(c, H):
    case = inputs.make_tri_case(I=45, c=c, H=H, d=32, dtype="f32", mask="random", seed=40 + c + H,
                                affine=True, biases=True)
    dev = _dev()
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        got = gpu_to_f64(dev.TriRunner(case.z, case.mask, p, H, "f32")(ori))
        ref = oracle.tri_fwd(case.z, case.mask, p.as_dict(), H, ori)
        check(got, ref, "f32", f"f32 tri c={c} H={H} ori={ori}")


def test_f32_fully_masked_rows_give_b_o():
    """A row (START) or column (END) with every key masked: o = 0, out = b_o."""
    case = inputs.make_tri_case(I=70, c=128, H=4, d=32, dtype="f32", mask="random", seed=41, affine=True,
                                biases=True)
    mask = case.mask.copy()
    mask[5, :] = 0
    mask[:, 9] = 0
    dev = _dev()
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        got = gpu_to_f64(dev.TriRunner(case.z, mask, p, 4, "f32")(ori))
        ref = oracle.tri_fwd(case.z, mask, p.as_dict(), 4, ori)
        check(got, ref, "f32", f"f32 masked rows ori={ori}")
        b_o = p.b_o.astype(np.float64)
        dead = got[5] if ori == 0 else got[:, 9]
        assert np.array_equal(dead, np.broadcast_to(b_o, dead.shape))


# ----------------------------------------------------------------------------
# the running maximum: logits spread over a wide range (the maximum is raised
# many times along the keys) and logits offset far from zero.  The kernel
# sweeps with shift 0 first and sweeps again with the running maximum where a
# query's l is not in [1, 65504): offsets of -60 (l < 1), +45 and +200 (a
# weight past 65504) and -200 (every weight 0 in fp32, l = 0 for rows that
# keep keys) take the second sweep; fully masked rows (l = 0 exactly) do not.
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("scale", [4.0, 8.0])
def test_f32_wide_logits_rescale(scale):
    case = inputs.make_tri_case(I=100, c=128, H=4, d=32, dtype="f32", mask="random", seed=42, affine=True,
                                biases=True)
    p = case.params_start
    p.w_q = (p.w_q * scale).astype(np.float32)
    p.w_k = (p.w_k * scale).astype(np.float32)
    got = gpu_to_f64(_dev().TriRunner(case.z, case.mask, p, 4, "f32")(0))
    ref = oracle.tri_fwd(case.z, case.mask, p.as_dict(), 4, 0)
    check(got, ref, "f32", f"f32 wide logits x{scale}")


@pytest.mark.parametrize("t,keep", [(-60.0, 0), (45.0, 3), (200.0, 0), (-200.0, 0), (-200.0, 3)])
def test_f32_offset_logits(t, keep):
    """The pair bias offset by t for every head, through LayerNorm's beta:
    beta = t * w_b (w_b^T w_b)^-1 1 gives beta . w_b[:, h] = t.  The offset
    also grows v and the gate (beta enters every projection), so W_o is
    scaled down by the same factor to keep the outputs at unit scale, where
    the 1e-4 bar applies (fp32 holds a logit near 300 only to ~3e-5)."""
    case = inputs.make_tri_case(I=64, c=128, H=4, d=32, dtype="f32", mask="none", seed=43, affine=True,
                                biases=True)
    p = case.params_start
    wb = p.w_b.astype(np.float64)
    p.ln_beta = (wb @ np.linalg.solve(wb.T @ wb, np.full(4, t))).astype(np.float32)
    p.ln_gamma = (0.25 * p.ln_gamma).astype(np.float32)
    p.w_o = (p.w_o / max(1.0, abs(t) / 8.0)).astype(np.float32)
    mask = None
    if keep:
        rng = np.random.default_rng(43)
        mask = np.zeros((64, 64), np.uint8)
        for i in range(64):
            mask[i, rng.choice(64, size=keep, replace=False)] = 1
    got = gpu_to_f64(_dev().TriRunner(case.z, mask, p, 4, "f32")(0))
    ref = oracle.tri_fwd(case.z, mask, p.as_dict(), 4, 0)
    b = oracle.attention_bias(case.z, p.as_dict(), 4, oracle.START)
    assert np.abs(b.mean() - t) < 1.0
    check(got, ref, "f32", f"f32 offset logits t={t} keep={keep}")


# ----------------------------------------------------------------------------
# the row-block form, the bias entry point and properties
# ----------------------------------------------------------------------------
def test_f32_bias_entry_point_matches_oracle():
    case = inputs.make_tri_case(I=50, c=128, H=4, d=32, dtype="f32", mask="none", seed=44, affine=True)
    dev = _dev()
    zf = dev.to_device(case.z, "f32")
    from pair_representation_attention_amd import lib
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        b = torch.empty((4, 50, 50), dtype=torch.float32, device="cuda")
        pp = dev.make_params(p, "f32")
        lib.pairattn_tri_bias(zf, pp, b, 50, 128, 4, ori)
        torch.cuda.synchronize()
        ref = oracle.attention_bias(case.z, p.as_dict(), 4, ori)
        err = np.max(np.abs(b.cpu().numpy() - ref))
        print(f"[parity] f32 bias ori={ori} max_abs={err:.3e}", flush=True)
        assert err < 1e-5


def test_f32_rows_block_equals_full_start():
    case = inputs.make_tri_case(I=96, c=128, H=4, d=32, dtype="f32", mask="random", seed=45, affine=True,
                                biases=True)
    dev = _dev()
    p = case.params_start
    full = dev.TriRunner(case.z, case.mask, p, 4, "f32")(0).clone()
    zf = dev.to_device(case.z, "f32")
    r0, r1 = 33, 70
    rr = dev.RowsRunner(zf, zf[r0:r1].contiguous(), dev.mask_to_device(case.mask[r0:r1]), p, 4, "f32")
    got = rr()
    ref = oracle.tri_start(case.z, case.mask, p.as_dict(), 4, rows=np.arange(r0, r1))
    check(gpu_to_f64(got), ref, "f32", "f32 rows block I=96")
    # the bias goes through natural-log fp32 and back, so allow rounding
    assert torch.max(torch.abs(got - full[r0:r1])).item() < 1e-5


def test_f32_end_equals_start_on_transpose_bitwise():
    case = inputs.make_tri_case(I=77, c=64, H=8, d=32, dtype="f32", mask="random", seed=46, affine=True,
                                biases=True)
    dev = _dev()
    p = case.params_start
    end = dev.TriRunner(case.z, case.mask, p, 8, "f32")(1).clone()
    zt = np.ascontiguousarray(case.z.transpose(1, 0, 2))
    st = dev.TriRunner(zt, np.ascontiguousarray(case.mask.T), p, 8, "f32")(0)
    assert torch.equal(end, st.transpose(0, 1))


def test_f32_deterministic_bitwise():
    case = inputs.make_tri_case(I=130, c=128, H=4, d=32, dtype="f32", mask="random", seed=47)
    run = _dev().TriRunner(case.z, case.mask, case.params_start, 4, "f32")
    a = run(0).clone()
    for _ in range(2):
        assert torch.equal(run(0), a)


@pytest.mark.parametrize("mask", ["bernoulli", "columns", "none"])
def test_f32_msa_small(mask):
    case = inputs.make_msa_case(S=6, I=41, c_m=64, c_z=128, H=8, d=32, dtype="f32", mask=mask, seed=48,
                                affine=True, biases=True)
    if case.mask is not None:
        case.mask[3, :] = 0
    got = gpu_to_f64(_dev().MsaRunner(case.m, case.z, case.mask, case.params, 8, "f32")())
    ref = oracle.msa_row(case.m, case.z, case.mask, case.params.as_dict(), 8)
    check(got, ref, "f32", f"f32 msa small mask={mask}")


def test_cfg_msa_fp32_s5120_i384():
    """Extra-MSA row attention at full size (5120 sequences): sampled
    sequences against the oracle."""
    cfg = inputs.CONFIGS["msa_fp32_s5120_i384"]
    case = inputs.make_msa_case(S=cfg["S"], I=cfg["I"], c_m=cfg["c_m"], c_z=cfg["c_z"], H=cfg["H"], d=cfg["d"],
                                dtype=cfg["dtype"], mask=cfg["mask"], seed=cfg["seed"])
    got = _dev().MsaRunner(case.m, case.z, case.mask, case.params, cfg["H"], "f32")()
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    seqs = np.array(sorted(set([0, cfg["S"] - 1, 2561]) | set(rng.choice(cfg["S"], 6, replace=False).tolist())))
    g = gpu_to_f64(got[torch.as_tensor(seqs, device="cuda")])
    ref = oracle.msa_row(case.m, case.z, case.mask, case.params.as_dict(), cfg["H"], seqs=seqs)
    check(g, ref, "f32", f"cfg msa_fp32_s5120_i384 seqs={seqs.tolist()}")
