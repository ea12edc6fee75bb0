"""GPU runs of the debug build (libpairattn_debug.so: the same sources at
-O1 with -DPA_DEBUG).  Its kernels check every index they compute against
the extents of their buffers (copy sources and LDS stages of the
attention, q / gate tiles, the staged output tile, the projection's stores,
the keep-bits words) and set a flag bit instead of trapping.  Small cases of
each path run through it: parity against the oracle as in the release
tests, and no failed check (pairattn_debug_status).

Run on an MI355X:  python -m pytest tests -m gpu
"""
import os

import numpy as np
import pytest

import oracle
from pair_representation_attention_amd import inputs
from parity_common import check, gpu_to_f64
from test_gpu_parity import _block_mix_mask

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _debug_library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from pair_representation_attention_amd import lib
    if not os.path.exists(lib.DEBUG_LIB_PATH):
        pytest.fail(f"{lib.DEBUG_LIB_PATH} missing: the build makes it beside the release library")
    prev = lib._lib
    lib._lib = None
    lib.load(lib.DEBUG_LIB_PATH)
    flags, checking = lib.pairattn_debug_status()
    assert checking == 1, "the debug library reports no index checks"
    yield lib
    lib._lib = prev   # the release library for the test modules that follow


def _no_failed_check(lib, what):
    torch.cuda.synchronize()
    flags, _ = lib.pairattn_debug_status()
    assert flags == 0, f"{what}: index checks failed, flag bits {flags:#x}"


def _dev():
    from pair_representation_attention_amd import device
    return device


@pytest.mark.parametrize("H,I", [(4, 100), (8, 70)])
def test_debug_tri_block_masks(_debug_library, H, I):
    lib = _debug_library
    case = inputs.make_tri_case(I=I, c=128, H=H, d=32, dtype="bf16", mask="none", seed=600 + I, affine=True,
                                biases=True)
    rows = _block_mix_mask(I, seed=I + 3)
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        mask = rows if ori == 0 else np.ascontiguousarray(rows.T)
        got = gpu_to_f64(_dev().TriRunner(case.z, mask, p, H, "bf16")(ori))
        _no_failed_check(lib, f"tri H={H} I={I} ori={ori}")
        check(got, oracle.tri_fwd(case.z, mask, p.as_dict(), H, ori), "bf16", f"debug tri H={H} ori={ori}")


def test_debug_tri_unmasked_and_fp32(_debug_library):
    lib = _debug_library
    for dtype, I in (("bf16", 96), ("bf16", 33), ("f32", 40)):
        case = inputs.make_tri_case(I=I, c=128, H=4, d=32, dtype=dtype, mask="none", seed=620 + I, affine=True,
                                    biases=True)
        got = gpu_to_f64(_dev().TriRunner(case.z, None, case.params_start, 4, dtype)(0))
        _no_failed_check(lib, f"tri {dtype} I={I}")
        check(got, oracle.tri_fwd(case.z, None, case.params_start.as_dict(), 4, 0), dtype, f"debug tri {dtype} I={I}")


@pytest.mark.parametrize("mask", ["bernoulli", "none"])
def test_debug_msa(_debug_library, mask):
    lib = _debug_library
    case = inputs.make_msa_case(S=6, I=70, c_m=256, c_z=128, H=8, d=32, dtype="bf16", mask=mask, seed=640,
                                affine=True, biases=True)
    got = gpu_to_f64(_dev().MsaRunner(case.m, case.z, case.mask, case.params, 8, "bf16")())
    _no_failed_check(lib, f"msa mask={mask}")
    check(got, oracle.msa_row(case.m, case.z, case.mask, case.params.as_dict(), 8), "bf16", f"debug msa {mask}")


def test_debug_msa_streamed_projection_batches(_debug_library):
    """c_m = 256: the streamed projection, with more batches of 8 tiles (300)
    than workgroups, so that the copies of the next batch's first operand
    slice and the loads of its rows run under the current batch."""
    lib = _debug_library
    case = inputs.make_msa_case(S=200, I=384, c_m=256, c_z=128, H=4, d=32, dtype="bf16", mask="bernoulli",
                                seed=641, affine=True, biases=True)
    got = gpu_to_f64(_dev().MsaRunner(case.m, case.z, case.mask, case.params, 4, "bf16")())
    _no_failed_check(lib, "msa streamed projection")
    seqs = np.array([0, 77, 199])
    ref = oracle.msa_row(case.m, case.z, case.mask, case.params.as_dict(), 4, seqs=seqs)
    check(got[seqs], ref, "bf16", "debug msa streamed projection")


def test_debug_chunked(_debug_library):
    lib = _debug_library
    case = inputs.make_tri_case(I=90, c=64, H=4, d=32, dtype="bf16", mask="random", seed=660, affine=True,
                                biases=True)
    dev = _dev()
    ch = dev.TriChunkedRunner(dev.to_device(case.z, "bf16"), dev.mask_to_device(case.mask), case.params_start, 4,
                              "bf16", 37)
    got = gpu_to_f64(ch(0))
    _no_failed_check(lib, "chunked")
    check(got, oracle.tri_fwd(case.z, case.mask, case.params_start.as_dict(), 4, 0), "bf16", "debug chunked")


def test_debug_partial_shards_and_finish(_debug_library):
    """bf16 partial attention over two key shards (the second merged), then
    the finish: the one-pass kernel's modes 1 and 2 and the fused finish."""
    lib = _debug_library
    dev = _dev()
    I, H, c = 96, 4, 128
    case = inputs.make_tri_case(I=I, c=c, H=H, d=32, dtype="bf16", mask="random", seed=680, affine=True,
                                biases=True)
    p = case.params_start
    z, m = case.z, case.mask
    zd = dev.to_device(z, "bf16")
    bias = torch.empty((H, I, I), dtype=torch.float32, device="cuda")
    lib.pairattn_tri_bias(zd, dev.make_params(p, "bf16"), bias, I, c, H, lib.PAIRATTN_START)
    rows = np.arange(20, 30)
    qp = dev.to_device(z[rows], "bf16")
    code = dev.dtype_code("bf16")
    n = max(lib.pairattn_tri_partial_workspace_bytes(len(rows), I, 64, c, H, 32, code),
            lib.pairattn_tri_partial_finish_workspace_bytes(len(rows), I, c, H, 32, code))
    prm = dev.make_params(p, "bf16", n)
    o = torch.zeros((len(rows), I, H * 32), dtype=torch.float32, device="cuda")
    lse = torch.zeros((len(rows), H, I), dtype=torch.float32, device="cuda")
    out = torch.empty((len(rows), I, c), dtype=torch.bfloat16, device="cuda")
    for n_s, ks in enumerate((np.arange(0, 64), np.arange(64, I))):
        kv = dev.to_device(np.ascontiguousarray(z[rows][:, ks]), "bf16")
        b = bias[:, :, ks].contiguous()   # [H, queries (all I positions), keys of the shard]
        mk = torch.from_numpy(np.ascontiguousarray(m[rows][:, ks], np.uint8)).to("cuda")
        lib.pairattn_tri_partial_fwd(qp, kv, b, mk, prm, o, lse, n_s > 0, len(rows), I, len(ks), c, H, 32)
    lib.pairattn_tri_partial_finish(qp, o, prm, out, len(rows), I, c, H, 32)
    got = gpu_to_f64(out)
    _no_failed_check(lib, "partial + finish")
    bref = oracle.attention_bias(z.astype(np.float64), p.as_dict(), H, oracle.START)
    check(got, oracle.tri_rows(z[rows], bref, m[rows], p.as_dict(), H), "bf16", "debug partial + finish")
