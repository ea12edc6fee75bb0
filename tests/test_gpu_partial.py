"""GPU parity of partial attention (one key shard with its log-sum-exp) and
its finish, the local step of ring attention over a 2D device grid, against
the fp64 oracle through the C ABI.  fp32 path: max abs error <= 1e-4 on o,
lse and the finished output.  bf16 path: the bf16 bar on o and the output,
max abs error <= 2e-2 on lse.

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


def _lib():
    from pair_representation_attention_amd import lib
    return lib


def _dev():
    from pair_representation_attention_amd import device
    return device


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


LSE_TOL = {"f32": 1e-4, "bf16": 2e-2}


def _check_lse(got, ref, what, dtype="f32"):
    got = got.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isinf(got), np.isinf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    print(f"[parity] {what} lse max_abs={err:.3e}", flush=True)
    assert err <= LSE_TOL[dtype]


class _Partial:
    """Device buffers for one (rows, queries) block across key shards."""

    def __init__(self, q_pairs, params, H, kn_max, dtype="f32"):
        lib, dev = _lib(), _dev()
        self.R, self.Jq, self.c = q_pairs.shape
        self.H, self.dtype = H, dtype
        self.q = dev.to_device(q_pairs, dtype)
        code = dev.dtype_code(dtype)
        n = max(lib.pairattn_tri_partial_workspace_bytes(self.R, self.Jq, kn_max, self.c, H, 32, code),
                lib.pairattn_tri_partial_finish_workspace_bytes(self.R, self.Jq, self.c, H, 32, code))
        self.params = dev.make_params(params, dtype, n)
        self.o = torch.zeros((self.R, self.Jq, H * 32), dtype=torch.float32, device="cuda")
        self.lse = torch.zeros((self.R, H, self.Jq), dtype=torch.float32, device="cuda")
        self.out = torch.empty((self.R, self.Jq, self.c), dtype=dev.torch_dtype(dtype), device="cuda")

    def shard(self, kv_pairs, bias, mask, accumulate):
        lib = _lib()
        kv = _dev().to_device(kv_pairs, self.dtype)
        b = _t(bias)
        m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).to("cuda")
        lib.pairattn_tri_partial_fwd(self.q, kv, b, m, self.params, self.o, self.lse, accumulate, self.R, self.Jq,
                                     kv_pairs.shape[1], self.c, self.H, 32)
        torch.cuda.synchronize()

    def own_shard(self, bias, mask, accumulate):
        """The device's own shard: kv_pairs is the query pairs' buffer itself."""
        lib = _lib()
        b = _t(bias)
        m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).to("cuda")
        lib.pairattn_tri_partial_fwd(self.q, self.q, b, m, self.params, self.o, self.lse, accumulate, self.R,
                                     self.Jq, self.Jq, self.c, self.H, 32)
        torch.cuda.synchronize()

    def finish(self):
        _lib().pairattn_tri_partial_finish(self.q, self.o, self.params, self.out, self.R, self.Jq, self.c, self.H, 32)
        torch.cuda.synchronize()
        return self.out


def _gpu_bias(z, p, H, dtype="f32"):
    """The library's own pair bias of the whole Z (starting node), [H, I, I]:
    what the GPU path is fed.  The oracle computes its own."""
    lib, dev = _lib(), _dev()
    I, _, c = z.shape
    b = torch.empty((H, I, I), dtype=torch.float32, device="cuda")
    lib.pairattn_tri_bias(dev.to_device(z, dtype), dev.make_params(p, dtype), b, I, c, H, lib.PAIRATTN_START)
    torch.cuda.synchronize()
    return b.cpu().numpy()


def _case(I, c, H, seed, mask="random", dtype="f32"):
    case = inputs.make_tri_case(I=I, c=c, H=H, d=32, dtype=dtype, mask=mask, seed=seed, affine=True, biases=True)
    p = case.params_start
    bias_ref = oracle.attention_bias(case.z.astype(np.float64), p.as_dict(), H, oracle.START)   # [H, I, I]
    return case, p, _gpu_bias(case.z, p, H, dtype), bias_ref


@pytest.mark.parametrize("c,H", [(128, 4), (64, 8)])
def test_partial_single_shard_and_finish(c, H):
    case, p, bias, bref = _case(70, c, H, seed=80 + c + H)
    z, m = case.z, case.mask
    rows = np.arange(10, 17)
    pt = _Partial(z[rows], p, H, 70)
    pt.shard(z[rows], bias, m[rows], 0)
    o_ref, lse_ref = oracle.tri_partial(z[rows], z[rows], bref, m[rows], p.as_dict(), H)
    check(pt.o.cpu().numpy().astype(np.float64), o_ref, "f32", f"partial o c={c} H={H}")
    _check_lse(pt.lse, lse_ref, f"partial c={c} H={H}")
    out = pt.finish().cpu().numpy().astype(np.float64)
    check(out, oracle.tri_rows(z[rows], bref, m[rows], p.as_dict(), H), "f32", f"finish = row form c={c} H={H}")


def test_partial_ragged_shards_merge_on_the_gpu():
    """Keys in three ragged shards (37, 64 and 29 keys), one of them fully
    masked for a row; queries a subset of 50 columns."""
    I, H = 130, 4
    case, p, bias, bref = _case(I, 128, H, seed=91)
    z, m = case.z, case.mask.copy()
    rows = np.array([3, 64, 65, 129])
    qcols = np.arange(40, 90)
    shards = [np.arange(0, 37), np.arange(37, 101), np.arange(101, 130)]
    m[64, shards[1]] = 0
    pt = _Partial(z[rows][:, qcols], p, H, 64)
    for n, ks in enumerate(shards):
        pt.shard(z[rows][:, ks], bias[:, qcols][:, :, ks], m[rows][:, ks], n > 0)
    o_ref, lse_ref = oracle.tri_partial(z[rows][:, qcols], z[rows], bref[:, qcols], m[rows], p.as_dict(), H)
    check(pt.o.cpu().numpy().astype(np.float64), o_ref, "f32", "merged o")
    _check_lse(pt.lse, lse_ref, "merged")
    out = pt.finish().cpu().numpy().astype(np.float64)
    ref = oracle.tri_rows(z[rows], bref, m[rows], p.as_dict(), H, queries=qcols)
    check(out, ref, "f32", "merged + finish = row form")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_partial_q_ready_equals_the_full_call(dtype):
    """PAIRATTN_PARTIAL_Q_READY on the shards after the first (the workspace
    keeps the packed weights and the projected q of the query pairs) gives
    o and lse bit for bit equal to projecting q again; with the device's own
    shard second, its k and v come from the query pairs as before."""
    lib = _lib()
    I, H = 96, 4
    case, p, bias, _ = _case(I, 128, H, seed=95, dtype=dtype)
    z, m = case.z, case.mask
    rows = np.arange(30, 36)
    qcols = np.arange(0, 48)
    shards = [np.arange(48, 96), qcols]       # a foreign shard, then the query pairs' own
    runs = []
    for ready in (False, True):
        pt = _Partial(z[rows][:, qcols], p, H, 48, dtype)
        for n, ks in enumerate(shards):
            flags = (lib.PAIRATTN_PARTIAL_MERGE if n > 0 else 0) | \
                (lib.PAIRATTN_PARTIAL_Q_READY if ready and n > 0 else 0)
            b = _t(bias[:, qcols][:, :, ks])
            mk = torch.from_numpy(np.ascontiguousarray(m[rows][:, ks], np.uint8)).to("cuda")
            kv = pt.q if n == 1 else _dev().to_device(z[rows][:, ks], dtype)
            lib.pairattn_tri_partial_fwd(pt.q, kv, b, mk, pt.params, pt.o, pt.lse, flags, pt.R, pt.Jq, len(ks),
                                         pt.c, H, 32)
        torch.cuda.synchronize()
        runs.append((pt.o.clone(), pt.lse.clone()))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


def test_partial_shard_with_no_kept_key_keeps_the_others():
    """A shard whose keys are all masked leaves o and lse as they were."""
    I, H = 64, 4
    case, p, bias, _ = _case(I, 128, H, seed=93, mask="none")
    z = case.z
    rows = np.arange(0, 5)
    pt = _Partial(z[rows], p, H, 32)
    pt.shard(z[rows][:, :32], bias[:, :, :32], None, 0)
    o0, l0 = pt.o.clone(), pt.lse.clone()
    pt.shard(z[rows][:, 32:], bias[:, :, 32:], np.zeros((5, 32), np.uint8), 1)
    assert torch.equal(pt.o, o0) and torch.equal(pt.lse, l0)


def test_ring_over_a_2x2_grid_i512():
    """Z[512, 512, 128] on a simulated 2 x 2 grid: the block of rows A and
    columns B attends over the two column shards in ring order (its own
    first), then finishes; the four blocks together give starting-node
    attention (sampled rows against the oracle, all of it against the
    one-pass fp32 call)."""
    I, H, half = 512, 4, 256
    case = inputs.make_tri_case(I=I, c=128, H=H, d=32, dtype="f32", mask="random", seed=95, affine=True,
                                biases=True)
    z, m, p = case.z, case.mask, case.params_start
    full = _dev().TriRunner(z, m, p, H, "f32")(0).cpu().numpy().astype(np.float64)
    bias_all = _gpu_bias(z, p, H)   # in a grid each tile comes from the device holding those pairs
    got = np.empty_like(full)
    blocks = [np.arange(0, half), np.arange(half, I)]
    rng = np.random.default_rng(0)
    for a in range(2):
        rows = blocks[a]
        zq_all = z[rows]
        for b in range(2):
            cols = blocks[b]
            pt = _Partial(zq_all[:, cols], p, H, half)
            for step in range(2):
                kb = (b + step) % 2                         # ring order: own shard first
                ks = blocks[kb]
                bias_t = bias_all[:, cols][:, :, ks]       # the tile of (these queries, this shard)
                pt.shard(zq_all[:, ks], bias_t, m[rows][:, ks], step > 0)
            got[np.ix_(rows, cols)] = pt.finish().cpu().numpy().astype(np.float64)
    assert np.max(np.abs(got - full)) <= 1e-4
    sample = rng.choice(I, 6, replace=False)
    ref = oracle.tri_start(z, m, p.as_dict(), H, rows=sample)
    check(got[sample], ref, "f32", "2x2 ring, sampled rows")


# ----------------------------------------------------------------------------
# bf16 path (the same kernels as the one-pass bf16 attention, with a partial
# epilogue)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("c,H,mask", [(128, 4, "random"), (128, 4, "none"), (64, 8, "random"), (256, 4, "none"),
                                        (256, 8, "random")])
def test_partial_bf16_single_shard_and_finish(c, H, mask):
    """One shard holding every key (H = 4 without a mask runs the pipelined
    sweep, with one the generic sweep; H = 8 the generic sweep)."""
    case, p, bias, bref = _case(70, c, H, seed=180 + c + H, mask=mask, dtype="bf16")
    z, m = case.z, case.mask
    rows = np.arange(10, 17)
    mr = None if m is None else m[rows]
    pt = _Partial(z[rows], p, H, 70, "bf16")
    pt.shard(z[rows], bias, mr, 0)
    o_ref, lse_ref = oracle.tri_partial(z[rows], z[rows], bref, mr, p.as_dict(), H)
    check(pt.o.cpu().numpy().astype(np.float64), o_ref, "bf16", f"bf16 partial o c={c} H={H} mask={mask}")
    _check_lse(pt.lse, lse_ref, f"bf16 partial c={c} H={H} mask={mask}", "bf16")
    out = gpu_to_f64(pt.finish())
    check(out, oracle.tri_rows(z[rows], bref, mr, p.as_dict(), H), "bf16", f"bf16 finish = row form c={c} H={H}")


@pytest.mark.parametrize("masked", [True, False])
def test_partial_bf16_ragged_shards_merge(masked):
    """Keys in three ragged shards (37, 64 and 29 keys), queries a subset of
    50 columns; with a mask one row has no kept key in the middle shard."""
    I, H = 130, 4
    case, p, bias, bref = _case(I, 128, H, seed=191, mask="random" if masked else "none", dtype="bf16")
    z = case.z
    m = case.mask.copy() if masked else None
    rows = np.array([3, 64, 65, 129])
    qcols = np.arange(40, 90)
    shards = [np.arange(0, 37), np.arange(37, 101), np.arange(101, 130)]
    if masked:
        m[64, shards[1]] = 0
    pt = _Partial(z[rows][:, qcols], p, H, 64, "bf16")
    for n, ks in enumerate(shards):
        pt.shard(z[rows][:, ks], bias[:, qcols][:, :, ks], None if m is None else m[rows][:, ks], n > 0)
    mr = None if m is None else m[rows]
    o_ref, lse_ref = oracle.tri_partial(z[rows][:, qcols], z[rows], bref[:, qcols], mr, p.as_dict(), H)
    check(pt.o.cpu().numpy().astype(np.float64), o_ref, "bf16", f"bf16 merged o masked={masked}")
    _check_lse(pt.lse, lse_ref, f"bf16 merged masked={masked}", "bf16")
    out = gpu_to_f64(pt.finish())
    ref = oracle.tri_rows(z[rows], bref, mr, p.as_dict(), H, queries=qcols)
    check(out, ref, "bf16", f"bf16 merged + finish = row form masked={masked}")


@pytest.mark.parametrize("t", [-20.0, 20.0])
def test_partial_bf16_offset_bias_takes_the_shifted_sweep(t):
    """The bias offset by t for every (query, key): the softmax weights
    underflow (t < 0) or overflow (t > 0) fp16 without a shift, so the
    workgroups sweep again with per-query shifts.  o is unchanged by the
    offset and lse moves by t; two shards merge across it."""
    I, H = 96, 4
    case, p, bias, bref = _case(I, 128, H, seed=193, mask="none", dtype="bf16")
    z = case.z
    rows = np.arange(20, 26)
    pt = _Partial(z[rows], p, H, 64, "bf16")
    pt.shard(z[rows][:, :64], bias[:, :, :64] + t, None, 0)
    pt.shard(z[rows][:, 64:], bias[:, :, 64:] + t, None, 1)
    o_ref, lse_ref = oracle.tri_partial(z[rows], z[rows], bref + t, None, p.as_dict(), H)
    check(pt.o.cpu().numpy().astype(np.float64), o_ref, "bf16", f"bf16 offset o t={t}")
    _check_lse(pt.lse, lse_ref, f"bf16 offset t={t}", "bf16")
    assert abs(float(np.mean(lse_ref)) - float(np.mean(oracle.tri_partial(z[rows], z[rows], bref, None,
                                                                       p.as_dict(), H)[1])) - t) < 1e-9


def test_partial_bf16_shard_with_no_kept_key_keeps_the_others():
    I, H = 64, 8
    case, p, bias, _ = _case(I, 128, H, seed=195, mask="none", dtype="bf16")
    z = case.z
    rows = np.arange(0, 5)
    pt = _Partial(z[rows], p, H, 32, "bf16")
    pt.shard(z[rows][:, :32], bias[:, :, :32], None, 0)
    o0, l0 = pt.o.clone(), pt.lse.clone()
    pt.shard(z[rows][:, 32:], bias[:, :, 32:], np.zeros((5, 32), np.uint8), 1)
    assert torch.equal(pt.o, o0) and torch.equal(pt.lse, l0)


def test_ring_bf16_over_a_2x2_grid_i512():
    """The 2 x 2 grid of the fp32 test in bf16, without a mask (the
    pipelined sweep): the reassembled update against the one-pass bf16 call
    and, on sampled rows, against the oracle."""
    I, H, half = 512, 4, 256
    case = inputs.make_tri_case(I=I, c=128, H=H, d=32, dtype="bf16", mask="none", seed=197, affine=True,
                                biases=True)
    z, p = case.z, case.params_start
    full = gpu_to_f64(_dev().TriRunner(z, None, p, H, "bf16")(0))
    bias_all = _gpu_bias(z, p, H, "bf16")
    got = np.empty_like(full)
    blocks = [np.arange(0, half), np.arange(half, I)]
    for a in range(2):
        rows = blocks[a]
        for b in range(2):
            cols = blocks[b]
            pt = _Partial(z[rows][:, cols], p, H, half, "bf16")
            for step in range(2):
                ks = blocks[(b + step) % 2]
                pt.shard(z[rows][:, ks], bias_all[:, cols][:, :, ks], None, step > 0)
            got[np.ix_(rows, cols)] = gpu_to_f64(pt.finish())
    check(got, full, "bf16", "bf16 2x2 ring = one pass")
    sample = np.random.default_rng(1).choice(I, 5, replace=False)
    check(got[sample], oracle.tri_start(z, None, p.as_dict(), H, rows=sample), "bf16", "bf16 2x2 ring, sampled rows")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cfg_ring_i1536_grid2x2(dtype):
    """The ring step at the size and in the launch sequence the benchmark
    times: Z[1536, 1536, 128] drawn on the device, the tile of rows 0..767
    and columns 0..767 on a 2 x 2 grid, its own key shard, then the other
    (merged), then the finish.  Sampled (row, query) outputs against the
    oracle, which reads only the rows of Z it needs."""
    lib, dev = _lib(), _dev()
    I, c, H, d, half, seed = 1536, 128, 4, 32, 768, 11
    print(f"[cfg ring] {dtype}: generating Z[{I},{I},{c}] on the device", flush=True)
    z = inputs.make_z_device(I, c, seed, dtype=dtype)
    p = inputs.make_chunked_params(c, H, d, seed, dtype=dtype)
    bias = torch.empty((H, I, I), dtype=torch.float32, device="cuda")
    lib.pairattn_tri_bias(z, dev.make_params(p, dtype), bias, I, c, H, lib.PAIRATTN_START)
    zq = z[:half, :half].contiguous()
    shards = [zq, z[:half, half:].contiguous()]            # the own shard is the query pairs' buffer
    btiles = [bias[:, :half, :half].contiguous(), bias[:, :half, half:].contiguous()]
    code = dev.dtype_code(dtype)
    n = max(lib.pairattn_tri_partial_workspace_bytes(half, half, half, c, H, d, code),
            lib.pairattn_tri_partial_finish_workspace_bytes(half, half, c, H, d, code))
    prm = dev.make_params(p, dtype, n)
    o = torch.empty((half, half, H * d), dtype=torch.float32, device="cuda")
    lse = torch.empty((half, H, half), dtype=torch.float32, device="cuda")
    out = torch.empty((half, half, c), dtype=dev.torch_dtype(dtype), device="cuda")
    for sidx in range(2):
        lib.pairattn_tri_partial_fwd(zq, shards[sidx], btiles[sidx], None, prm, o, lse, sidx > 0, half, half, half,
                                     c, H, d)
    lib.pairattn_tri_partial_finish(zq, o, prm, out, half, half, c, H, d)
    torch.cuda.synchronize()
    # both rows of 5 workgroup pairs across the tile; queries in 6 of its 24 query blocks
    rows = np.array([0, 1, 200, 201, 383, 384, 590, 591, half - 2, half - 1])
    queries = np.array([0, 5, 31, 32, 300, 511, 512, 700, half - 1])
    g = out[torch.as_tensor(rows, device="cuda")][:, torch.as_tensor(queries, device="cuda")]
    pd = p.as_dict()
    zr = z[torch.as_tensor(rows, device="cuda")].float().cpu().numpy().astype(np.float64)
    zqr = z[torch.as_tensor(queries, device="cuda")].float().cpu().numpy().astype(np.float64)
    bias_q = oracle.attention_bias(zqr, pd, H, oracle.START)         # [H, Q, I] for these queries
    ref = oracle.tri_rows(zr, bias_q, None, pd, H, queries=queries, bias_restricted=True)
    check(gpu_to_f64(g), ref, dtype, f"cfg ring_{dtype}_i1536_grid2x2 rows={rows.tolist()}")
    del z, bias, zq, shards, btiles, o, lse, out, prm
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("masked", [False, True])
def test_own_shard_from_the_query_buffer_bitwise(dtype, masked):
    """kv_pairs given as the query pairs' own buffer (one projection pass for
    q, k and v) gives the same o and lse, bit for bit, as a copy of it."""
    case, p, bias, _ = _case(70, 128, 4, seed=199, mask="random" if masked else "none", dtype=dtype)
    z = case.z
    rows = np.arange(3, 9)
    m = None if not masked else case.mask[rows]
    a = _Partial(z[rows], p, 4, 70, dtype)
    a.own_shard(bias, m, 0)
    b = _Partial(z[rows], p, 4, 70, dtype)
    b.shard(z[rows], bias, m, 0)
    assert torch.equal(a.o, b.o) and torch.equal(a.lse, b.lse)
