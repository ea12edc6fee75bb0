"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle.

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


# ----------------------------------------------------------------------------
# small shapes: full output against the oracle, tails and masks
# ----------------------------------------------------------------------------
# I a multiple of 32 without a mask takes the software-pipelined sweep of the
# bf16 kernel: 32, 64, 96 and 160 give 1, 2, 3 and 5 key blocks (a single
# final block, one pipelined block, an odd count, several), the others the
# generic sweep with its tail block.
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("I", [1, 7, 32, 33, 64, 96, 100, 160])
@pytest.mark.parametrize("mask", ["none", "random"])
def test_tri_small_shapes(dtype, I, mask):
    case = inputs.make_tri_case(I=I, c=128, H=4, d=32, dtype=dtype, mask=mask, seed=100 + I,
                                affine=True, biases=True)
    dev = _dev()
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        run = dev.TriRunner(case.z, case.mask, p, 4, dtype)
        got = gpu_to_f64(run(ori))
        torch.cuda.synchronize()
        ref = oracle.tri_fwd(case.z, case.mask, p.as_dict(), 4, ori)
        check(got, ref, dtype, f"tri I={I} ori={ori} mask={mask}")


@pytest.mark.parametrize("c,H", [(64, 4), (256, 8), (128, 8)])
def test_tri_other_widths(c, H):
    case = inputs.make_tri_case(I=45, c=c, H=H, d=32, dtype="bf16", mask="random", seed=7 + c + H,
                                affine=True, biases=True)
    dev = _dev()
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        got = gpu_to_f64(dev.TriRunner(case.z, case.mask, p, H, "bf16")(ori))
        ref = oracle.tri_fwd(case.z, case.mask, p.as_dict(), H, ori)
        check(got, ref, "bf16", f"tri c={c} H={H} ori={ori}")


# ----------------------------------------------------------------------------
# logits far from zero: the kernel's zero-shift sweep cannot represent the
# softmax weights there (fp16 overflow above 2^16, too little mass below), so
# the workgroup sweeps again with per-query shifts.  The pair-bias offset is
# set through the LayerNorm beta: beta = t * w_b (w_b^T w_b)^-1 1 gives
# beta . w_b[:, h] = t for every head h.
# ----------------------------------------------------------------------------
def _offset_case(t: float, keep_per_row: int, seed: int):
    case = inputs.make_tri_case(I=64, c=128, H=4, d=32, dtype="bf16", mask="none", seed=seed, affine=True,
                                biases=True)
    p = case.params_start
    wb = p.w_b.astype(np.float64)
    beta = wb @ np.linalg.solve(wb.T @ wb, np.full(4, t))
    p.ln_beta = inputs.round_to_bf16(beta.astype(np.float32))
    p.ln_gamma = inputs.round_to_bf16((0.25 * p.ln_gamma).astype(np.float32))
    mask = None
    if keep_per_row:
        rng = np.random.default_rng(seed)
        mask = np.zeros((64, 64), np.uint8)
        for i in range(64):
            mask[i, rng.choice(64, size=keep_per_row, replace=False)] = 1
    return case.z, mask, p


@pytest.mark.parametrize("t,keep", [(-4.0, 3), (12.0, 0), (-8.0, 0)])
def test_far_logits_take_the_shifted_sweep(t, keep):
    z, mask, p = _offset_case(t, keep, seed=31)
    got = gpu_to_f64(_dev().TriRunner(z, mask, p, 4, "bf16")(0))
    ref = oracle.tri_fwd(z, mask, p.as_dict(), 4, 0)
    b = oracle.attention_bias(z, p.as_dict(), 4, oracle.START)
    assert np.abs(b.mean() - t) < 1.0    # the offset is in place
    check(got, ref, "bf16", f"far logits t={t} keep={keep}")


# ----------------------------------------------------------------------------
# workload configurations
# ----------------------------------------------------------------------------
def test_cfg_tri_fp32_i64():
    cfg = inputs.CONFIGS["tri_fp32_i64"]
    case = inputs.make_tri_case(I=cfg["I"], c=cfg["c"], H=cfg["H"], d=cfg["d"], dtype=cfg["dtype"],
                                mask=cfg["mask"], seed=cfg["seed"])
    dev = _dev()
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        got = gpu_to_f64(dev.TriRunner(case.z, case.mask, p, 4, "f32")(ori))
        ref = oracle.tri_fwd(case.z, case.mask, p.as_dict(), 4, ori)
        check(got, ref, "f32", f"cfg tri_fp32_i64 ori={ori}")


def _sample(I, n, rng):
    s = set([0, I - 1, I // 2]) | set(rng.choice(I, size=min(n, I), replace=False).tolist())
    return np.array(sorted(s))


def test_cfg_tri_bf16_i384_padded():
    cfg = inputs.CONFIGS["tri_bf16_i384_pad"]
    case = inputs.make_tri_case(I=cfg["I"], c=cfg["c"], H=cfg["H"], d=cfg["d"], dtype=cfg["dtype"],
                                mask=cfg["mask"], seed=cfg["seed"])
    dev = _dev()
    rng = np.random.default_rng(0)
    rows = np.concatenate([_sample(case.I, 10, rng), [350, 383]])   # includes padded residues
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        got = gpu_to_f64(dev.TriRunner(case.z, case.mask, p, 4, "bf16")(ori))
        if ori == 0:
            ref = oracle.tri_start(case.z, case.mask, p.as_dict(), 4, rows=rows)
            g = got[rows]
        else:
            ref = oracle.tri_end(case.z, case.mask, p.as_dict(), 4, cols=rows)
            g = got[:, rows]
        check(g, ref, "bf16", f"cfg tri_bf16_i384_pad ori={ori}")
        # padded residues: every key masked -> out = b_o (= 0 here)
        pad = case.mask.sum(1) == 0
        assert np.all(got[pad] == 0.0) if ori == 0 else np.all(got[:, pad] == 0.0)


def test_cfg_msa_bf16():
    cfg = inputs.CONFIGS["msa_bf16_s512_i384"]
    case = inputs.make_msa_case(S=cfg["S"], I=cfg["I"], c_m=cfg["c_m"], c_z=cfg["c_z"], H=cfg["H"], d=cfg["d"],
                                dtype=cfg["dtype"], mask=cfg["mask"], seed=cfg["seed"])
    dev = _dev()
    got = gpu_to_f64(dev.MsaRunner(case.m, case.z, case.mask, case.params, 8, "bf16")())
    rng = np.random.default_rng(1)
    seqs = _sample(case.S, 8, rng)
    ref = oracle.msa_row(case.m, case.z, case.mask, case.params.as_dict(), 8, seqs=seqs)
    check(got[seqs], ref, "bf16", "cfg msa_bf16_s512_i384")


@pytest.mark.parametrize("mask", ["bernoulli", "columns", "none"])
def test_msa_small(mask):
    case = inputs.make_msa_case(S=5, I=37, c_m=256, c_z=128, H=8, d=32, dtype="bf16", mask=mask, seed=17,
                                affine=True, biases=True)
    if case.mask is not None:
        case.mask[2, :] = 0
    got = gpu_to_f64(_dev().MsaRunner(case.m, case.z, case.mask, case.params, 8, "bf16")())
    ref = oracle.msa_row(case.m, case.z, case.mask, case.params.as_dict(), 8)
    check(got, ref, "bf16", f"msa small mask={mask}")


def test_msa_small_fp32():
    case = inputs.make_msa_case(S=4, I=21, c_m=64, c_z=64, H=4, d=32, dtype="f32", mask="bernoulli", seed=19,
                                affine=True, biases=True)
    got = gpu_to_f64(_dev().MsaRunner(case.m, case.z, case.mask, case.params, 4, "f32")())
    ref = oracle.msa_row(case.m, case.z, case.mask, case.params.as_dict(), 4)
    check(got, ref, "f32", "msa small fp32")


def test_cfg_tri_bf16_i1536_sampled():
    cfg = inputs.CONFIGS["tri_bf16_i1536"]
    case = inputs.make_tri_case(I=cfg["I"], c=cfg["c"], H=cfg["H"], d=cfg["d"], dtype=cfg["dtype"],
                                mask=cfg["mask"], seed=cfg["seed"])
    dev = _dev()
    rng = np.random.default_rng(2)
    rows = np.array([0, 777, 1535])
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        out = dev.TriRunner(case.z, case.mask, p, 4, "bf16")(ori)
        if ori == 0:
            got = gpu_to_f64(out[torch.as_tensor(rows, device=out.device)])
            ref = oracle.tri_start(case.z, None, p.as_dict(), 4, rows=rows)
        else:
            got = gpu_to_f64(out[:, torch.as_tensor(rows, device=out.device)])
            ref = oracle.tri_end(case.z, None, p.as_dict(), 4, cols=rows)
        check(got, ref, "bf16", f"cfg tri_bf16_i1536 ori={ori} rows={rows.tolist()}")
        del out


def test_cfg_rows_bf16_i4096_r512():
    """A block of 512 starting-node rows of Z[4096, 4096, 128] (repeated
    171-residue blocks plus noise): the bias comes from the whole Z through
    pairattn_tri_bias, the rows through pairattn_tri_rows_fwd.  The oracle
    evaluates sampled (row, query) outputs from the rows of Z they need."""
    cfg = inputs.CONFIGS["rows_bf16_i4096_r512"]
    I, R, c, H, d = cfg["I"], cfg["R"], cfg["c"], cfg["H"], cfg["d"]
    print(f"[cfg rows] generating Z[{I},{I},{c}]", flush=True)
    case = inputs.make_rows_case(I=I, R=R, c=c, H=H, d=d, asu=cfg["asu"], noise=cfg["noise"], seed=cfg["seed"])
    dev = _dev()
    zf = torch.from_numpy(case.zbits.view(np.int16)).to("cuda").view(torch.bfloat16)
    r0 = case.r0
    rr = dev.RowsRunner(zf, zf[r0:r0 + R], None, case.params, H, "bf16")
    got = rr()
    torch.cuda.synchronize()
    p = case.params.as_dict()
    rows = np.array([0, 217, R - 1])
    queries = np.array([0, 5, 170, 171, 2047, r0 + 217, I - 1])
    zq = inputs.bf16_bits_to_f32(case.zbits[queries])
    bias_q = oracle.attention_bias(zq, p, H, oracle.START)            # [H, Q, I] for these query rows
    got_bias = rr.bias[:, torch.as_tensor(queries, device="cuda")].cpu().numpy()
    assert np.max(np.abs(got_bias - bias_q)) < 3e-2
    zr = inputs.bf16_bits_to_f32(case.zbits[r0 + rows])
    ref = oracle.tri_rows(zr, bias_q, None, p, H, queries=queries, bias_restricted=True)
    g = gpu_to_f64(got[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(queries, device="cuda")])
    check(g, ref, "bf16", f"cfg rows_bf16_i4096_r512 rows={(r0 + rows).tolist()} queries={queries.tolist()}")
    del rr, zf
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# properties of the GPU path
# ----------------------------------------------------------------------------
def test_end_equals_start_on_transpose_bitwise():
    case = inputs.make_tri_case(I=77, c=128, H=4, d=32, dtype="bf16", mask="random", seed=5, affine=True,
                                biases=True)
    dev = _dev()
    p = case.params_start
    end = dev.TriRunner(case.z, case.mask, p, 4, "bf16")(1).clone()
    zt = np.ascontiguousarray(case.z.transpose(1, 0, 2))
    st = dev.TriRunner(zt, np.ascontiguousarray(case.mask.T), p, 4, "bf16")(0)
    assert torch.equal(end, st.transpose(0, 1))


def test_rows_block_equals_full_start():
    case = inputs.make_tri_case(I=96, c=128, H=4, d=32, dtype="bf16", mask="random", seed=6, affine=True,
                                biases=True)
    dev = _dev()
    p = case.params_start
    full = dev.TriRunner(case.z, case.mask, p, 4, "bf16")(0).clone()
    zf = dev.to_device(case.z, "bf16")
    r0, r1 = 33, 70
    rr = dev.RowsRunner(zf, zf[r0:r1].contiguous(), dev.mask_to_device(case.mask[r0:r1]), p, 4, "bf16")
    got = rr()
    assert torch.equal(got, full[r0:r1])
    ref = oracle.tri_start(case.z, case.mask, p.as_dict(), 4, rows=np.arange(r0, r1))
    check(gpu_to_f64(got), ref, "bf16", "rows block I=96")


def test_bias_entry_point_matches_oracle():
    case = inputs.make_tri_case(I=50, c=128, H=4, d=32, dtype="bf16", mask="none", seed=8, affine=True)
    dev = _dev()
    zf = dev.to_device(case.z, "bf16")
    rr = dev.RowsRunner(zf, zf[:2].contiguous(), None, case.params_start, 4, "bf16")
    b = rr.compute_bias().cpu().numpy()
    ref = oracle.attention_bias(case.z, case.params_start.as_dict(), 4, oracle.START)
    # bias = bf16(LN(z)) . w_b with fp32 accumulation
    assert np.max(np.abs(b - ref)) < 3e-2


def test_deterministic_bitwise():
    case = inputs.make_tri_case(I=130, c=128, H=4, d=32, dtype="bf16", mask="random", seed=9)
    dev = _dev()
    run = dev.TriRunner(case.z, case.mask, case.params_start, 4, "bf16")
    a = run(0).clone()
    for _ in range(2):
        assert torch.equal(run(0), a)
