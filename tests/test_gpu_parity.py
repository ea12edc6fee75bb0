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
# masks whose 32-key blocks are all kept, all masked or mixed, row by row.
# The bf16 kernel sweeps only the blocks between the first and the last one
# with a kept key in either row of a workgroup (rows 2r and 2r+1), runs every
# block there through its masked units, and skips the select where all 32
# keys are kept; rows without a kept key skip the sweep.  The patterns below
# put leading and trailing empty blocks, empty blocks in the middle, full
# blocks, single kept keys, fully masked rows and rows whose partner row
# differs into one mask (START reads its rows, END its columns).
# ----------------------------------------------------------------------------
def _block_mix_mask(I: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    nb = (I + 31) // 32
    m = np.zeros((I, I), np.uint8)
    for i in range(I):
        kind = i % 8
        if kind == 0:                       # every key
            m[i, :] = 1
        elif kind == 1:                     # a prefix ending inside a block (the padding pattern)
            m[i, : rng.integers(1, I)] = 1
        elif kind == 2:                     # nothing: out = b_o
            pass
        elif kind == 3:                     # a suffix starting inside a block (leading empty blocks)
            m[i, rng.integers(0, I):] = 1
        elif kind == 4:                     # random blocks fully kept, fully masked or Bernoulli
            for b in range(nb):
                r = rng.integers(0, 3)
                sl = slice(b * 32, min(I, b * 32 + 32))
                m[i, sl] = 1 if r == 0 else (0 if r == 1 else (rng.random(sl.stop - sl.start) < 0.5))
        elif kind == 5:                     # one kept key
            m[i, rng.integers(0, I)] = 1
        elif kind == 6:                     # two kept runs with empty blocks between them
            a = rng.integers(0, max(1, I // 4))
            b = rng.integers(I // 2, I)
            m[i, a: a + 40] = 1
            m[i, b:] = 1
        else:                               # Bernoulli(0.95)
            m[i, :] = rng.random(I) < 0.95
    return m


@pytest.mark.parametrize("I", [160, 200, 384])
def test_block_mixed_masks(I):
    case = inputs.make_tri_case(I=I, c=128, H=4, d=32, dtype="bf16", mask="none", seed=300 + I, affine=True,
                                biases=True)
    rows = _block_mix_mask(I, seed=I)      # line i: the keys of attention row i
    dev = _dev()
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        # START keeps key k of row i iff mask[i, k]; END keeps key k of column j iff mask[k, j]
        mask = rows if ori == 0 else np.ascontiguousarray(rows.T)
        got = gpu_to_f64(dev.TriRunner(case.z, mask, p, 4, "bf16")(ori))
        ref = oracle.tri_fwd(case.z, mask, p.as_dict(), 4, ori)
        check(got, ref, "bf16", f"block-mixed mask I={I} ori={ori}")
        # rows (START) or columns (END) without a kept key give out = b_o exactly
        none = np.where(~rows.any(axis=1))[0]
        assert len(none) > 0
        bo = inputs.round_to_bf16(p.b_o.astype(np.float32)).astype(np.float64)
        sel = got[none, :, :] if ori == 0 else got[:, none, :]
        assert np.array_equal(sel, np.broadcast_to(bo, sel.shape))


# The same patterns at H = 8, where a workgroup is one row and three query
# blocks, each wave copies and reads only its own tiles, and a block's keep
# bits enter the logits through the operand that widens the bias (-inf for
# masked keys) instead of a select per unit.
@pytest.mark.parametrize("I", [160, 200])
def test_block_mixed_masks_h8(I):
    case = inputs.make_tri_case(I=I, c=128, H=8, d=32, dtype="bf16", mask="none", seed=400 + I, affine=True,
                                biases=True)
    rows = _block_mix_mask(I, seed=I + 1)
    dev = _dev()
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        mask = rows if ori == 0 else np.ascontiguousarray(rows.T)
        got = gpu_to_f64(dev.TriRunner(case.z, mask, p, 8, "bf16")(ori))
        ref = oracle.tri_fwd(case.z, mask, p.as_dict(), 8, ori)
        check(got, ref, "bf16", f"block-mixed mask H=8 I={I} ori={ori}")
        none = np.where(~rows.any(axis=1))[0]
        assert len(none) > 0
        bo = inputs.round_to_bf16(p.b_o.astype(np.float32)).astype(np.float64)
        sel = got[none, :, :] if ori == 0 else got[:, none, :]
        assert np.array_equal(sel, np.broadcast_to(bo, sel.shape))


# MSA row attention at H = 8 over several key blocks: without a mask and I a
# multiple of 32 (no select at all; with 5 blocks the copies of block kb+2
# go out while blocks kb and kb+1 are in flight), and with the block
# patterns above as the sequences' masks (a sequence without a kept key
# gives out = b_o).
@pytest.mark.parametrize("S,I,mask", [(6, 96, "none"), (4, 160, "none"), (16, 200, "blocks")])
def test_msa_h8_sweep_shapes(S, I, mask):
    case = inputs.make_msa_case(S=S, I=I, c_m=256, c_z=128, H=8, d=32, dtype="bf16", mask="none", seed=500 + I,
                                affine=True, biases=True)
    m = None if mask == "none" else np.ascontiguousarray(_block_mix_mask(I, seed=I + 2)[:S])
    got = gpu_to_f64(_dev().MsaRunner(case.m, case.z, m, case.params, 8, "bf16")())
    ref = oracle.msa_row(case.m, case.z, m, case.params.as_dict(), 8)
    check(got, ref, "bf16", f"msa H=8 S={S} I={I} mask={mask}")
    if m is not None:
        none = np.where(~m.any(axis=1))[0]
        assert len(none) > 0
        bo = inputs.round_to_bf16(case.params.b_o.astype(np.float32)).astype(np.float64)
        assert np.array_equal(got[none], np.broadcast_to(bo, got[none].shape))


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


@pytest.mark.parametrize("c_m,H", [(256, 4), (128, 8)])
@pytest.mark.parametrize("S,I", [(5, 37), (200, 384)])
def test_msa_other_widths(c_m, H, S, I):
    """Widths whose q|k|v|g operands exceed the LDS (4*H*32 columns of c_m
    channels over 128 KB) take the streamed projection: one LayerNorm per
    position tile, the operand in slices through LDS.  S = 5, I = 37 leaves
    waves without a tile in the last batch; S = 200, I = 384 (2400 tiles)
    gives workgroups more than one batch."""
    case = inputs.make_msa_case(S=S, I=I, c_m=c_m, c_z=128, H=H, d=32, dtype="bf16", mask="bernoulli",
                                seed=23 + c_m + H + I, affine=True, biases=True)
    got = gpu_to_f64(_dev().MsaRunner(case.m, case.z, case.mask, case.params, H, "bf16")())
    if S <= 8:
        ref = oracle.msa_row(case.m, case.z, case.mask, case.params.as_dict(), H)
        check(got, ref, "bf16", f"msa c_m={c_m} H={H} S={S} I={I}")
    else:
        seqs = _sample(S, 6, np.random.default_rng(2))
        ref = oracle.msa_row(case.m, case.z, case.mask, case.params.as_dict(), H, seqs=seqs)
        check(got[seqs], ref, "bf16", f"msa c_m={c_m} H={H} S={S} I={I}")


def test_msa_small_fp32():
    case = inputs.make_msa_case(S=4, I=21, c_m=64, c_z=64, H=4, d=32, dtype="f32", mask="bernoulli", seed=19,
                                affine=True, biases=True)
    got = gpu_to_f64(_dev().MsaRunner(case.m, case.z, case.mask, case.params, 4, "f32")())
    ref = oracle.msa_row(case.m, case.z, case.mask, case.params.as_dict(), 4)
    check(got, ref, "f32", "msa small fp32")


def _super_column_width(n_qg, n_rg):
    """Query groups per super-column at H = 4, as the launch chooses them: the
    first width in 4..8 that divides the query groups and whose super-columns
    are whole multiples or whole fractions of an XCD's range of tiles, else 4."""
    per = n_qg * n_rg // 8
    for w in range(4, 9):
        if n_qg % w == 0 and per > 0 and ((n_rg * w) % per == 0 or per % (n_rg * w) == 0):
            return w
    return 4


def _attn_tiles_hit(rows, I, H=4):
    """(XCD, super-column) pairs of the bf16 attention's tile order that the
    sampled rows reach, every query of each row being checked.  Mirrors the
    launch: workgroups of 2 rows x 4 query blocks (H = 4), logical tile
    L' = (L % 8) * (n / 8) + L / 8 for L < 8 * (n / 8) (each XCD takes a
    contiguous range), tiles walked in super-columns of w query groups."""
    n_qg = ((I + 31) // 32 + 3) // 4
    n_rg = (I + 1) // 2
    w = _super_column_width(n_qg, n_rg)
    n = n_qg * n_rg
    per = n // 8
    hit = set()
    for L in range(n):
        Lp = (L % 8) * per + L // 8 if L < per * 8 else L
        sc = Lp // (n_rg * w)
        sc_w = min(w, n_qg - sc * w)
        rgi = (Lp - sc * n_rg * w) // sc_w
        if 2 * rgi in rows or 2 * rgi + 1 in rows:
            hit.add((L % 8, sc))
    return hit, -(-n_qg // w)


def test_cfg_tri_bf16_i1536_sampled():
    """16 starting-node rows and 16 ending-node columns of Z[1536,1536,128]:
    both rows of 8 workgroup pairs spread over the range, so that every XCD's
    contiguous range of tiles and every query super-column is checked."""
    cfg = inputs.CONFIGS["tri_bf16_i1536"]
    case = inputs.make_tri_case(I=cfg["I"], c=cfg["c"], H=cfg["H"], d=cfg["d"], dtype=cfg["dtype"],
                                mask=cfg["mask"], seed=cfg["seed"])
    dev = _dev()
    I = case.I
    rows = np.array([0, 1, 200, 201, 574, 575, 576, 577, 800, 801, 1150, 1151, 1152, 1153, 1534, 1535])
    hit, n_sc = _attn_tiles_hit(set(rows.tolist()), I)
    assert {x for x, _ in hit} == set(range(8)), hit          # all 8 XCD tile ranges
    assert {sc for _, sc in hit} == set(range(n_sc)), hit     # all super-columns
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


def _rows_covering_tiles(I):
    """One row of a row group in each (XCD, super-column) pair of the bf16
    attention's tile order, plus the last row."""
    n_qg = ((I + 31) // 32 + 3) // 4
    n_rg = (I + 1) // 2
    rows = {I - 1}
    seen = set()
    for rg in range(n_rg):
        hit, _ = _attn_tiles_hit({2 * rg}, I)
        if hit - seen:
            rows.add(2 * rg)
            seen |= hit
    return np.array(sorted(rows)), seen


@pytest.mark.parametrize("I,width", [(1280, 5), (1792, 7)])
def test_super_column_widths_write_every_tile(I, width):
    """Query-group counts whose super-column width is neither 4 nor 6 (10
    groups: 5; 14 groups: 7).  The output starts as NaN: every element must be
    written, in both orientations, and sampled rows and columns that reach
    every XCD range and super-column match the oracle."""
    n_qg = ((I + 31) // 32 + 3) // 4
    assert _super_column_width(n_qg, (I + 1) // 2) == width
    case = inputs.make_tri_case(I=I, c=128, H=4, d=32, dtype="bf16", mask="none", seed=31)
    rows, seen = _rows_covering_tiles(I)
    hit, n_sc = _attn_tiles_hit(set(rows.tolist()), I)
    assert {x for x, _ in hit} == set(range(8)) and {sc for _, sc in hit} == set(range(n_sc)), hit
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        run = _dev().TriRunner(case.z, None, p, 4, "bf16")
        run.out.fill_(float("nan"))
        out = run(ori)
        assert bool(torch.isfinite(out).all()), f"I={I} ori={ori}: output elements left unwritten"
        if ori == 0:
            got = gpu_to_f64(out[torch.as_tensor(rows, device=out.device)])
            ref = oracle.tri_start(case.z, None, p.as_dict(), 4, rows=rows)
        else:
            got = gpu_to_f64(out[:, torch.as_tensor(rows, device=out.device)])
            ref = oracle.tri_end(case.z, None, p.as_dict(), 4, cols=rows)
        check(got, ref, "bf16", f"I={I} width={width} ori={ori} rows={rows.tolist()}")
        del out, run


def test_cfg_tri_bf16_i1536_end_is_start_on_transpose_bitwise():
    """The whole ending-node output of Z[1536,1536,128] against the starting-
    node output of Z^T with the same weights, bit for bit: every tile of both
    launches, at no cost on the host."""
    cfg = inputs.CONFIGS["tri_bf16_i1536"]
    case = inputs.make_tri_case(I=cfg["I"], c=cfg["c"], H=cfg["H"], d=cfg["d"], dtype=cfg["dtype"],
                                mask=cfg["mask"], seed=cfg["seed"])
    from pair_representation_attention_amd import lib
    dev = _dev()
    p = case.params_end
    end = dev.TriRunner(case.z, None, p, 4, "bf16")
    e = end(1)
    zt = end.z.transpose(0, 1).contiguous()
    prm = dev.make_params(p, "bf16", lib.pairattn_tri_workspace_bytes(case.I, 128, 4, 32, lib.PAIRATTN_BF16))
    s = torch.empty_like(zt)
    lib.pairattn_tri_fwd(zt, None, prm, s, case.I, 128, 4, 32, lib.PAIRATTN_START)
    torch.cuda.synchronize()
    assert torch.equal(e, s.transpose(0, 1)), "END(Z) differs from START(Z^T)^T"
    del end, prm, zt, s


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
    """pairattn_tri_bias: B[h, j, k] = fp16(LN(z[j, k])) . fp16(gamma o w_b[:, h]) accumulated in fp32,
    + beta . w_b[:, h] in fp32.  Each of the c products carries the relative
    errors of two fp16 roundings (2^-11 each), so
      |B - B_exact| <= (2^-10 + 2^-20) sum_c |x^_c gamma_c w_b[c, h]| + 1e-6
    per element (x^ the exact normalised activation; fp32 LayerNorm and
    accumulation errors are below 2^-20 of the same sum)."""
    case = inputs.make_tri_case(I=50, c=128, H=4, d=32, dtype="bf16", mask="none", seed=8, affine=True)
    dev = _dev()
    zf = dev.to_device(case.z, "bf16")
    rr = dev.RowsRunner(zf, zf[:2].contiguous(), None, case.params_start, 4, "bf16")
    b = rr.compute_bias().cpu().numpy().astype(np.float64)
    pd = case.params_start.as_dict()
    ref = oracle.attention_bias(case.z, pd, 4, oracle.START)
    xh = oracle.layer_norm(case.z.astype(np.float64), np.ones(128), np.zeros(128), 1e-5)   # [I, I, c]
    gw = np.abs(np.asarray(pd["ln_gamma"], np.float64)[:, None] * np.asarray(pd["w_b"], np.float64))   # [c, H]
    bound = (2.0 ** -10 + 2.0 ** -20) * np.einsum("jkc,ch->hjk", np.abs(xh), gw) + 1e-6
    err = np.abs(b - ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3f}"
    print(f"[bias] max err {err.max():.3e}, max err/bound {np.max(err / bound):.3f}", flush=True)


@pytest.mark.parametrize("gamma", [2.0 ** 12, 2.0 ** 20])
def test_fp16_range_edge_saturates_finite_and_deterministic(gamma):
    """The bf16 path's intermediates at and beyond the fp16 range (documented
    in pairattn.h).  gamma = 2^12 puts q, k and v near the edge (|k| ~ 4e3 x
    N(0,1), logits ~ 1e7, far past where the zero-shift sweep holds: the
    shifted rerun);
    gamma = 2^20 puts gamma o W and every q, k, v past 65504, so they
    saturate.  Either way the output must be finite, equal on every call,
    and within the largest magnitude the saturated operands allow."""
    case = inputs.make_tri_case(I=64, c=128, H=4, d=32, dtype="bf16", mask="random", seed=41, affine=True,
                                biases=True)
    p = case.params_start
    p.ln_gamma = np.full(128, gamma, np.float32)          # a power of two: bf16-exact
    dev = _dev()
    for ori in (0, 1):
        run = dev.TriRunner(case.z, case.mask, p, 4, "bf16")
        a = run(ori).clone()
        b = run(ori).clone()
        torch.cuda.synchronize()
        g = gpu_to_f64(a)
        assert np.all(np.isfinite(g)), f"gamma={gamma} ori={ori}: non-finite output"
        assert torch.equal(a, b), f"gamma={gamma} ori={ori}: not deterministic"
        # o is a convex combination of v (|v| <= 65504), the gate is at most 1:
        # |out| <= 65504 * sum_c |W_o| + |b_o| per channel
        lim = 65504.0 * np.abs(p.w_o.astype(np.float64)).sum(0) + np.abs(p.b_o.astype(np.float64))
        assert np.all(np.abs(g) <= lim * (1 + 2 ** -7))
        print(f"[range] gamma={gamma:g} ori={ori}: max |out| {np.abs(g).max():.3e}", flush=True)


def test_deterministic_bitwise():
    case = inputs.make_tri_case(I=130, c=128, H=4, d=32, dtype="bf16", mask="random", seed=9)
    dev = _dev()
    run = dev.TriRunner(case.z, case.mask, case.params_start, 4, "bf16")
    a = run(0).clone()
    for _ in range(2):
        assert torch.equal(run(0), a)
