"""GPU checks of pairattn_tri_chunked_fwd, the low-memory form of triangle
attention: the pair bias of the whole Z once, then blocks of rows (START) or
columns (END).  Small sizes: bit for bit equal to the one-pass call (even
blocks) and within tolerance of the oracle; full size: I = 16384, which the
one-pass workspace cannot hold beside Z and the update on one device, on
sampled rows and columns against the oracle.

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


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("I,block", [(100, 32), (100, 2), (160, 64), (97, 200)])
def test_chunked_equals_one_pass_bitwise(dtype, I, block):
    case = inputs.make_tri_case(I=I, c=128, H=4, d=32, dtype=dtype, mask="random", seed=60 + I + block,
                                affine=True, biases=True)
    dev = _dev()
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        full = dev.TriRunner(case.z, case.mask, p, 4, dtype)(ori).clone()
        ch = dev.TriChunkedRunner(dev.to_device(case.z, dtype), dev.mask_to_device(case.mask), p, 4, dtype, block)
        got = ch(ori)
        assert torch.equal(got, full), f"I={I} block={block} ori={ori}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunked_odd_block_against_oracle(dtype):
    """An odd block pairs rows differently in the bf16 kernel, so only the
    tolerance applies there."""
    case = inputs.make_tri_case(I=90, c=64, H=8, d=32, dtype=dtype, mask="random", seed=71, affine=True,
                                biases=True)
    dev = _dev()
    for ori, p in ((0, case.params_start), (1, case.params_end)):
        ch = dev.TriChunkedRunner(dev.to_device(case.z, dtype), dev.mask_to_device(case.mask), p, 8, dtype, 37)
        got = gpu_to_f64(ch(ori))
        ref = oracle.tri_fwd(case.z, case.mask, p.as_dict(), 8, ori)
        check(got, ref, dtype, f"chunked odd block ori={ori}")


def test_cfg_tri_bf16_i16384_chunked():
    """Z[16384, 16384, 128] bf16 (drawn on the device), blocks of 1024 rows or
    columns.  Sampled outputs against the oracle, which reads only the rows
    (START) or columns (END) of Z it needs: END is START on Z^T."""
    cfg = inputs.CONFIGS["tri_bf16_i16384_chunked"]
    I, c, H, d, block = cfg["I"], cfg["c"], cfg["H"], cfg["d"], cfg["block"]
    print(f"[cfg chunked] generating Z[{I},{I},{c}] on the device", flush=True)
    z = inputs.make_z_device(I, c, cfg["seed"])
    p = inputs.make_chunked_params(c, H, d, cfg["seed"])
    run = _dev().TriChunkedRunner(z, None, p, H, "bf16", block)
    print(f"[cfg chunked] workspace {run.workspace_bytes / 1e9:.1f} GB", flush=True)
    # two lines (an even row and the next, the bf16 kernel's workgroup pair)
    # in each of the 16 blocks, at positions that move through the block
    lines = np.array(sorted({b * block + off + e for b in range(I // block)
                             for off in [(b * 389) % (block - 1) & ~1] for e in (0, 1)} | {0, I - 1}))
    assert all(len([x for x in lines if x // block == b]) >= 2 for b in range(I // block))
    queries = np.array([0, 5, 1023, 1024, 4097, 8190, 12001, I - 2])
    pd = p.as_dict()
    for ori in (0, 1):
        got = run(ori)
        torch.cuda.synchronize()
        print(f"[cfg chunked] orientation {ori} done", flush=True)
        li = torch.as_tensor(lines, device="cuda")
        qi = torch.as_tensor(queries, device="cuda")
        if ori == 0:
            view_rows = z[li]                           # rows of the START view
            view_q = z[qi]
            g = got[li][:, qi]
        else:
            view_rows = z[:, li].transpose(0, 1)        # rows of Z^T = columns of Z
            view_q = z[:, qi].transpose(0, 1)
            g = got[:, li][qi].transpose(0, 1)
        zr = view_rows.float().cpu().numpy().astype(np.float64)
        zq = view_q.float().cpu().numpy().astype(np.float64)
        bias_q = oracle.attention_bias(zq, pd, H, oracle.START)      # [H, Q, I] for these queries
        ref = oracle.tri_rows(zr, bias_q, None, pd, H, queries=queries, bias_restricted=True)
        check(gpu_to_f64(g), ref, "bf16", f"cfg tri_bf16_i16384_chunked ori={ori}")
    del run, z
    torch.cuda.empty_cache()
