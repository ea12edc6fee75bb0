"""GPU parity of partial attention (one key shard with its log-sum-exp) and
its finish, the local step of ring attention over a 2D device grid, against
the fp64 oracle through the C ABI.  fp32 path; bar max abs error <= 1e-4 on
o, lse and the finished output.

Run on an MI355X:  python -m pytest tests -m gpu
"""
import numpy as np
import pytest

import oracle
from pair_representation_attention_amd import inputs
from parity_common import check

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


def _check_lse(got, ref, what):
    got = got.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isinf(got), np.isinf(ref)), f"{what}: -inf pattern differs"
    fin = np.isfinite(ref)
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    print(f"[parity] {what} lse max_abs={err:.3e}", flush=True)
    assert err <= 1e-4


class _Partial:
    """Device buffers for one (rows, queries) block across key shards."""

    def __init__(self, q_pairs, params, H, kn_max):
        lib, dev = _lib(), _dev()
        self.R, self.Jq, self.c = q_pairs.shape
        self.H = H
        self.q = _t(q_pairs)
        n = max(lib.pairattn_tri_partial_workspace_bytes(self.R, self.Jq, kn_max, self.c, H, 32, lib.PAIRATTN_F32),
                lib.pairattn_tri_partial_finish_workspace_bytes(self.R, self.Jq, self.c, H, 32, lib.PAIRATTN_F32))
        self.params = dev.make_params(params, "f32", n)
        self.o = torch.zeros((self.R, self.Jq, H * 32), dtype=torch.float32, device="cuda")
        self.lse = torch.zeros((self.R, H, self.Jq), dtype=torch.float32, device="cuda")
        self.out = torch.empty((self.R, self.Jq, self.c), dtype=torch.float32, device="cuda")

    def shard(self, kv_pairs, bias, mask, accumulate):
        lib = _lib()
        kv = _t(kv_pairs)
        b = _t(bias)
        m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).to("cuda")
        lib.pairattn_tri_partial_fwd(self.q, kv, b, m, self.params, self.o, self.lse, accumulate, self.R, self.Jq,
                                     kv_pairs.shape[1], self.c, self.H, 32)
        torch.cuda.synchronize()

    def finish(self):
        _lib().pairattn_tri_partial_finish(self.q, self.o, self.params, self.out, self.R, self.Jq, self.c, self.H, 32)
        torch.cuda.synchronize()
        return self.out


def _gpu_bias(z, p, H):
    """The library's own pair bias of the whole Z (starting node), [H, I, I]:
    what the GPU path is fed.  The oracle computes its own."""
    lib, dev = _lib(), _dev()
    I, _, c = z.shape
    b = torch.empty((H, I, I), dtype=torch.float32, device="cuda")
    lib.pairattn_tri_bias(_t(z), dev.make_params(p, "f32"), b, I, c, H, lib.PAIRATTN_START)
    torch.cuda.synchronize()
    return b.cpu().numpy()


def _case(I, c, H, seed, mask="random"):
    case = inputs.make_tri_case(I=I, c=c, H=H, d=32, dtype="f32", mask=mask, seed=seed, affine=True, biases=True)
    p = case.params_start
    bias_ref = oracle.attention_bias(case.z.astype(np.float64), p.as_dict(), H, oracle.START)   # [H, I, I]
    return case, p, _gpu_bias(case.z, p, H), bias_ref


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
