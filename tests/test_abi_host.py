"""Host-side checks of the C ABI (no GPU needed).

The library must load and export every function declared in
include/pairattn.h; argument validation runs on the host and returns the
documented status codes before any device work.  Pointers below are fake
addresses: validation never dereferences them.
"""
import ctypes

import pytest

from pair_representation_attention_amd import lib

A = 0x7F0000000000          # a 256-byte aligned fake device address
MB = 1 << 20


@pytest.fixture(scope="module")
def L():
    return lib.load()


def _params(dtype=lib.PAIRATTN_BF16, ws=None, ws_bytes=0, msa=False, **over):
    base = dict(ln_gamma=A + 1 * MB, ln_beta=A + 2 * MB, w_q=A + 3 * MB, w_k=A + 4 * MB, w_v=A + 5 * MB,
                w_g=A + 6 * MB, w_b=A + 7 * MB, w_o=A + 8 * MB, b_g=None, b_o=None)
    if msa:
        base.update(lnz_gamma=A + 9 * MB, lnz_beta=A + 10 * MB)
    base.update(over)
    eps = base.pop("eps", 1e-5)
    return lib.Params(dtype, eps=eps, workspace=ws, workspace_bytes=ws_bytes, **base)


Z = A + 64 * MB
OUT = A + 4096 * MB
WS = A + 8192 * MB


def test_exports_every_declared_symbol(L):
    names = lib.header_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), f"{n} declared in pairattn.h but not exported"


def test_version_and_status_strings(L):
    assert L.pairattn_version() >= 10000
    for st in range(6):
        assert lib.status_string(st) not in ("", "unknown status")
    assert lib.status_string(99) == "unknown status"


def test_workspace_sizes():
    w = lib.pairattn_tri_workspace_bytes(384, 128, 4, 32, lib.PAIRATTN_BF16)
    # q, k, v (padded to 384) + g + bias + packed weights, each 256-aligned
    assert w >= 3 * 384 * 4 * 384 * 32 * 2 + 384 * 384 * 128 * 2 + 4 * 384 * 384 * 2
    assert lib.pairattn_tri_workspace_bytes(384, 128, 4, 32, lib.PAIRATTN_F32) >= 4 * 384 * 384 * 128 * 4
    assert lib.pairattn_tri_workspace_bytes(384, 128, 4, 64, lib.PAIRATTN_BF16) == 0
    assert lib.pairattn_tri_workspace_bytes(384, 128, 3, 32, lib.PAIRATTN_BF16) == 0
    assert lib.pairattn_tri_workspace_bytes(384, 96, 4, 32, lib.PAIRATTN_BF16) == 0
    assert lib.pairattn_tri_workspace_bytes(0, 128, 4, 32, lib.PAIRATTN_BF16) == 0
    assert lib.pairattn_tri_workspace_bytes(8, 128, 4, 32, 7) == 0
    assert lib.pairattn_msa_workspace_bytes(512, 384, 256, 128, 8, 32, lib.PAIRATTN_BF16) > 0
    assert lib.pairattn_rows_workspace_bytes(512, 4096, 128, 4, 32, lib.PAIRATTN_BF16) > 0
    # a block of 16 rows needs less than all 64 rows
    assert lib.pairattn_rows_workspace_bytes(16, 64, 128, 4, 32, lib.PAIRATTN_BF16) < \
        lib.pairattn_tri_workspace_bytes(64, 128, 4, 32, lib.PAIRATTN_BF16)
    assert lib.pairattn_rows_workspace_bytes(16, 64, 128, 4, 32, lib.PAIRATTN_F32) < \
        lib.pairattn_tri_workspace_bytes(64, 128, 4, 32, lib.PAIRATTN_F32)
    # both paths copy the caller's bias into the attention's own layout: a
    # block of all rows needs the same workspace as the whole call
    for dt in (lib.PAIRATTN_BF16, lib.PAIRATTN_F32):
        assert lib.pairattn_rows_workspace_bytes(64, 64, 128, 4, 32, dt) == \
            lib.pairattn_tri_workspace_bytes(64, 128, 4, 32, dt)


def _tri_ok_params(I=64, c=128, H=4, dtype=lib.PAIRATTN_BF16):
    n = lib.pairattn_tri_workspace_bytes(I, c, H, 32, dtype)
    return _params(dtype, ws=WS, ws_bytes=n)


def test_validate_tri_ok():
    assert lib.pairattn_validate_tri(Z, None, _tri_ok_params(), OUT, 64, 128, 4, 32, 0) == lib.PAIRATTN_OK
    assert lib.pairattn_validate_tri(Z, A + 999 * MB, _tri_ok_params(), OUT, 64, 128, 4, 32, 1) == lib.PAIRATTN_OK
    p = _tri_ok_params(dtype=lib.PAIRATTN_F32)
    assert lib.pairattn_validate_tri(Z, None, p, OUT, 64, 128, 4, 32, 0) == lib.PAIRATTN_OK


@pytest.mark.parametrize("kw,status", [
    (dict(z=None), lib.PAIRATTN_ERR_ARG),
    (dict(out=None), lib.PAIRATTN_ERR_ARG),
    (dict(z=Z + 8), lib.PAIRATTN_ERR_ARG),
    (dict(orientation=2), lib.PAIRATTN_ERR_ARG),
    (dict(I=0), lib.PAIRATTN_ERR_ARG),
    (dict(d=64), lib.PAIRATTN_ERR_UNSUPPORTED),
    (dict(H=3), lib.PAIRATTN_ERR_UNSUPPORTED),
    (dict(c=96), lib.PAIRATTN_ERR_UNSUPPORTED),
    (dict(I=(1 << 20) + 1), lib.PAIRATTN_ERR_UNSUPPORTED),
    (dict(out=Z + 4096), lib.PAIRATTN_ERR_ARG),          # out overlaps z
    (dict(out=WS + 256), lib.PAIRATTN_ERR_ARG),          # out overlaps the workspace
])
def test_validate_tri_rejects(kw, status):
    args = dict(z=Z, mask=None, out=OUT, I=64, c=128, H=4, d=32, orientation=0)
    args.update(kw)
    p = _tri_ok_params()
    st = lib.pairattn_validate_tri(args["z"], args["mask"], p, args["out"], args["I"], args["c"], args["H"],
                                   args["d"], args["orientation"])
    assert st == status, lib.last_error()
    assert lib.last_error() != ""
    # the entry point returns the same status without touching a device
    st2 = lib.pairattn_tri_fwd(args["z"], args["mask"], p, args["out"], args["I"], args["c"], args["H"],
                               args["d"], args["orientation"], stream=0, check=False)
    assert st2 == status


@pytest.mark.parametrize("over,status", [
    (dict(w_q=None), lib.PAIRATTN_ERR_ARG),
    (dict(ln_gamma=None), lib.PAIRATTN_ERR_ARG),
    (dict(w_o=A + 3), lib.PAIRATTN_ERR_ARG),             # misaligned weight
    (dict(eps=-1.0), lib.PAIRATTN_ERR_ARG),
    (dict(eps=float("nan")), lib.PAIRATTN_ERR_ARG),
])
def test_validate_params(over, status):
    n = lib.pairattn_tri_workspace_bytes(64, 128, 4, 32, lib.PAIRATTN_BF16)
    p = _params(lib.PAIRATTN_BF16, ws=WS, ws_bytes=n, **over)
    assert lib.pairattn_validate_tri(Z, None, p, OUT, 64, 128, 4, 32, 0) == status


def test_validate_dtype_and_null_params(L):
    p = _tri_ok_params()
    p.dtype = 5
    assert lib.pairattn_validate_tri(Z, None, p, OUT, 64, 128, 4, 32, 0) == lib.PAIRATTN_ERR_ARG
    st = L.pairattn_validate_tri(Z, None, None, OUT, 64, 128, 4, 32, 0)
    assert st == lib.PAIRATTN_ERR_ARG


def test_validate_workspace():
    n = lib.pairattn_tri_workspace_bytes(64, 128, 4, 32, lib.PAIRATTN_BF16)
    for ws, nb in ((None, n), (WS, n - 1), (WS + 16, n)):
        p = _params(lib.PAIRATTN_BF16, ws=ws, ws_bytes=nb)
        assert lib.pairattn_validate_tri(Z, None, p, OUT, 64, 128, 4, 32, 0) == lib.PAIRATTN_ERR_WORKSPACE


def test_validate_msa_and_rows():
    n = lib.pairattn_msa_workspace_bytes(8, 40, 256, 128, 8, 32, lib.PAIRATTN_BF16)
    p = _params(lib.PAIRATTN_BF16, ws=WS, ws_bytes=n, msa=True)
    M = A + 512 * MB
    assert lib.pairattn_validate_msa(M, Z, None, p, OUT, 8, 40, 256, 128, 8, 32) == lib.PAIRATTN_OK
    assert lib.pairattn_validate_msa(M, Z, None, p, OUT, 0, 40, 256, 128, 8, 32) == lib.PAIRATTN_ERR_ARG
    assert lib.pairattn_validate_msa(M, Z, None, p, OUT, 8, 40, 256, 100, 8, 32) == lib.PAIRATTN_ERR_UNSUPPORTED
    p2 = _params(lib.PAIRATTN_BF16, ws=WS, ws_bytes=n, msa=False)     # missing pair LayerNorm
    assert lib.pairattn_validate_msa(M, Z, None, p2, OUT, 8, 40, 256, 128, 8, 32) == lib.PAIRATTN_ERR_ARG
    nr = lib.pairattn_rows_workspace_bytes(16, 100, 128, 4, 32, lib.PAIRATTN_BF16)
    pr = _params(lib.PAIRATTN_BF16, ws=WS, ws_bytes=nr)
    B = A + 2048 * MB
    assert lib.pairattn_validate_rows(Z, B, None, pr, OUT, 16, 100, 128, 4, 32) == lib.PAIRATTN_OK
    assert lib.pairattn_validate_rows(Z, None, None, pr, OUT, 16, 100, 128, 4, 32) == lib.PAIRATTN_ERR_ARG
    assert lib.pairattn_validate_rows(Z, B, None, pr, OUT, 16, 100, 128, 4, 16) == lib.PAIRATTN_ERR_UNSUPPORTED
    pr_small = _params(lib.PAIRATTN_BF16, ws=WS, ws_bytes=nr - 256)
    assert lib.pairattn_validate_rows(Z, B, None, pr_small, OUT, 16, 100, 128, 4, 32) == \
        lib.PAIRATTN_ERR_WORKSPACE


def test_bias_entry_validation():
    p = _params(lib.PAIRATTN_BF16)
    B = A + 2048 * MB
    assert lib.pairattn_tri_bias(Z, p, B, 64, 128, 4, 3, stream=0, check=False) == lib.PAIRATTN_ERR_ARG
    assert lib.pairattn_tri_bias(Z, p, None, 64, 128, 4, 0, stream=0, check=False) == lib.PAIRATTN_ERR_ARG
    assert lib.pairattn_tri_bias(Z, p, B, 64, 100, 4, 0, stream=0, check=False) == lib.PAIRATTN_ERR_UNSUPPORTED


def test_no_device_is_reported():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = lib.pairattn_tri_fwd(Z, None, _tri_ok_params(), OUT, 64, 128, 4, 32, 0, stream=0, check=False)
    assert st == lib.PAIRATTN_ERR_DEVICE, lib.last_error()


def test_python_binding_raises_on_error():
    with pytest.raises(lib.PairAttnError) as ei:
        lib.pairattn_tri_fwd(Z, None, _tri_ok_params(), OUT, 64, 128, 4, 48, 0, stream=0)
    assert ei.value.status == lib.PAIRATTN_ERR_UNSUPPORTED


# ----------------------------------------------------------------------------
# chunked triangle attention: workspace and argument rules
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("dt", [lib.PAIRATTN_BF16, lib.PAIRATTN_F32])
def test_chunked_workspace_sizes(dt):
    full = lib.pairattn_tri_workspace_bytes(1024, 128, 4, 32, dt)
    sizes = [lib.pairattn_tri_chunked_workspace_bytes(1024, 128, 4, 32, dt, b) for b in (1, 64, 256, 1024)]
    assert all(x > 0 for x in sizes)
    assert sizes == sorted(sizes) and sizes[0] < sizes[-1]
    # one block of all rows is the one-pass layout; more never costs more
    assert sizes[-1] == full
    assert lib.pairattn_tri_chunked_workspace_bytes(1024, 128, 4, 32, dt, 4096) == full
    # a block of 64 rows needs about 64/1024 of the projections plus the whole bias
    assert sizes[1] < full / 8
    assert lib.pairattn_tri_chunked_workspace_bytes(1024, 128, 4, 32, dt, 0) == 0
    assert lib.pairattn_tri_chunked_workspace_bytes(1024, 96, 4, 32, dt, 64) == 0


def test_chunked_at_i16384_fits_where_one_pass_does_not():
    """I = 16384, c = 128, H = 4, bf16: Z and the update take 68.7 GB each.
    The one-pass workspace (about 277 GB) cannot sit beside them on a 288 GB
    device; blocks of 1024 rows need about 19 GB (17.2 GB of projections,
    2.1 GB of bias)."""
    one = lib.pairattn_tri_workspace_bytes(16384, 128, 4, 32, lib.PAIRATTN_BF16)
    chunk = lib.pairattn_tri_chunked_workspace_bytes(16384, 128, 4, 32, lib.PAIRATTN_BF16, 1024)
    zb = 16384 * 16384 * 128 * 2
    assert one + 2 * zb > 288e9
    assert chunk < 20e9 and chunk + 2 * zb < 160e9


@pytest.mark.parametrize("kw,status", [
    (dict(block=0), lib.PAIRATTN_ERR_ARG),
    (dict(block=-3), lib.PAIRATTN_ERR_ARG),
    (dict(z=None), lib.PAIRATTN_ERR_ARG),
    (dict(orientation=7), lib.PAIRATTN_ERR_ARG),
    (dict(H=5), lib.PAIRATTN_ERR_UNSUPPORTED),
    (dict(out=Z + 4096), lib.PAIRATTN_ERR_ARG),
    (dict(ws_bytes=-1), lib.PAIRATTN_ERR_WORKSPACE),      # one byte short
])
def test_validate_tri_chunked(kw, status):
    args = dict(z=Z, mask=None, out=OUT, I=300, c=128, H=4, d=32, orientation=1, block=64)
    args.update({k: v for k, v in kw.items() if k != "ws_bytes"})
    need = lib.pairattn_tri_chunked_workspace_bytes(300, 128, 4, 32, lib.PAIRATTN_BF16, 64)
    p = _params(lib.PAIRATTN_BF16, ws=WS, ws_bytes=need + kw.get("ws_bytes", 0))
    st = lib.pairattn_validate_tri_chunked(args["z"], args["mask"], p, args["out"], args["I"], args["c"], args["H"],
                                           args["d"], args["orientation"], args["block"])
    assert st == status, lib.last_error()
    st2 = lib.pairattn_tri_chunked_fwd(args["z"], args["mask"], p, args["out"], args["I"], args["c"], args["H"],
                                       args["d"], args["orientation"], args["block"], stream=0, check=False)
    assert st2 == status


def test_validate_tri_chunked_ok():
    need = lib.pairattn_tri_chunked_workspace_bytes(300, 128, 4, 32, lib.PAIRATTN_F32, 64)
    p = _params(lib.PAIRATTN_F32, ws=WS, ws_bytes=need)
    assert lib.pairattn_validate_tri_chunked(Z, None, p, OUT, 300, 128, 4, 32, 0, 64) == lib.PAIRATTN_OK


# ----------------------------------------------------------------------------
# partial attention (one key shard) and its finish
# ----------------------------------------------------------------------------
QP, KP, BIAS, O_, LSE = A + 100 * MB, A + 200 * MB, A + 300 * MB, A + 400 * MB, A + 500 * MB


def test_partial_workspace_sizes():
    for dt in (lib.PAIRATTN_F32, lib.PAIRATTN_BF16):
        assert lib.pairattn_tri_partial_workspace_bytes(4, 64, 96, 128, 4, 32, dt) > 0
        assert lib.pairattn_tri_partial_workspace_bytes(4, 64, 0, 128, 4, 32, dt) == 0
        a = lib.pairattn_tri_partial_workspace_bytes(4, 64, 96, 128, 4, 32, dt)
        b = lib.pairattn_tri_partial_workspace_bytes(4, 64, 192, 128, 4, 32, dt)
        assert b > a
        assert lib.pairattn_tri_partial_finish_workspace_bytes(4, 64, 128, 4, 32, dt) > 0
    assert lib.pairattn_tri_partial_workspace_bytes(4, 64, 96, 128, 4, 32, 7) == 0   # unknown dtype
    # the bf16 path keeps single fp16 planes (no lo planes): a smaller workspace
    assert lib.pairattn_tri_partial_workspace_bytes(4, 64, 96, 128, 4, 32, lib.PAIRATTN_BF16) < \
        lib.pairattn_tri_partial_workspace_bytes(4, 64, 96, 128, 4, 32, lib.PAIRATTN_F32)


@pytest.mark.parametrize("kw,status", [
    (dict(), lib.PAIRATTN_OK),
    (dict(dtype=lib.PAIRATTN_BF16), lib.PAIRATTN_OK),
    (dict(dtype=lib.PAIRATTN_BF16, ws_short=True), lib.PAIRATTN_ERR_WORKSPACE),
    (dict(o=None), lib.PAIRATTN_ERR_ARG),
    (dict(lse=LSE + 4), lib.PAIRATTN_ERR_ARG),               # misaligned
    (dict(Kn=0), lib.PAIRATTN_ERR_ARG),
    (dict(o=QP), lib.PAIRATTN_ERR_ARG),                      # o overlaps the query pairs
    (dict(lse=O_ + 64), lib.PAIRATTN_ERR_ARG),               # lse overlaps o
    (dict(ws_short=True), lib.PAIRATTN_ERR_WORKSPACE),
])
def test_validate_tri_partial(kw, status):
    dt = kw.get("dtype", lib.PAIRATTN_F32)
    need = lib.pairattn_tri_partial_workspace_bytes(3, 40, 70, 128, 4, 32, dt)
    p = _params(dt, ws=WS, ws_bytes=need - (256 if kw.get("ws_short") else 0))
    a = dict(q=QP, k=KP, b=BIAS, m=None, o=O_, lse=LSE, R=3, Jq=40, Kn=70)
    a.update({k: v for k, v in kw.items() if k in a})
    st = lib.pairattn_validate_tri_partial(a["q"], a["k"], a["b"], a["m"], p, a["o"], a["lse"], a["R"], a["Jq"],
                                           a["Kn"], 128, 4, 32)
    assert st == status, lib.last_error()
    if status != lib.PAIRATTN_OK:
        st2 = lib.pairattn_tri_partial_fwd(a["q"], a["k"], a["b"], a["m"], p, a["o"], a["lse"], 0, a["R"], a["Jq"],
                                           a["Kn"], 128, 4, 32, stream=0, check=False)
        assert st2 == status


@pytest.mark.parametrize("flags", [4, 8, -1, 7])
def test_partial_flags_outside_merge_and_q_ready_are_rejected(flags):
    """accumulate holds PAIRATTN_PARTIAL_MERGE | PAIRATTN_PARTIAL_Q_READY only;
    any other bit is refused before anything is launched."""
    need = lib.pairattn_tri_partial_workspace_bytes(3, 40, 70, 128, 4, 32, lib.PAIRATTN_BF16)
    p = _params(lib.PAIRATTN_BF16, ws=WS, ws_bytes=need)
    st = lib.pairattn_tri_partial_fwd(QP, KP, BIAS, None, p, O_, LSE, flags, 3, 40, 70, 128, 4, 32, stream=0,
                                      check=False)
    assert st == lib.PAIRATTN_ERR_ARG and "accumulate" in lib.last_error()


def test_validate_tri_partial_finish():
    need = lib.pairattn_tri_partial_finish_workspace_bytes(3, 40, 128, 4, 32, lib.PAIRATTN_F32)
    p = _params(lib.PAIRATTN_F32, ws=WS, ws_bytes=need)
    assert lib.pairattn_validate_tri_partial_finish(QP, O_, p, OUT, 3, 40, 128, 4, 32) == lib.PAIRATTN_OK
    assert lib.pairattn_validate_tri_partial_finish(QP, O_, p, QP, 3, 40, 128, 4, 32) == lib.PAIRATTN_ERR_ARG
    nb = lib.pairattn_tri_partial_finish_workspace_bytes(3, 40, 128, 4, 32, lib.PAIRATTN_BF16)
    pb = _params(lib.PAIRATTN_BF16, ws=WS, ws_bytes=nb)
    assert lib.pairattn_validate_tri_partial_finish(QP, O_, pb, OUT, 3, 40, 128, 4, 32) == lib.PAIRATTN_OK
    pb = _params(lib.PAIRATTN_BF16, ws=WS, ws_bytes=nb - 256)
    assert lib.pairattn_validate_tri_partial_finish(QP, O_, pb, OUT, 3, 40, 128, 4, 32) == \
        lib.PAIRATTN_ERR_WORKSPACE


# ----------------------------------------------------------------------------
# allocation-free triangle attention: host checks before any device call
# ----------------------------------------------------------------------------
def test_noalloc_host_checks(L):
    p = _params(lib.PAIRATTN_BF16)   # no workspace: the call ignores those fields
    # the largest bf16 problem at H = 4 that fits the static scratch, and the next
    assert lib.pairattn_tri_workspace_bytes(507, 128, 4, 32, lib.PAIRATTN_BF16) <= lib.NOALLOC_SCRATCH_BYTES
    assert lib.pairattn_tri_workspace_bytes(508, 128, 4, 32, lib.PAIRATTN_BF16) > lib.NOALLOC_SCRATCH_BYTES
    st = lib.pairattn_tri_fwd_noalloc(Z, None, p, OUT, 508, 128, 4, 32, 0, stream=0, check=False)
    assert st == lib.PAIRATTN_ERR_UNSUPPORTED and "scratch" in lib.last_error()
    assert lib.pairattn_tri_fwd_noalloc(Z, None, p, OUT, 64, 128, 4, 32, 3, stream=0, check=False) == \
        lib.PAIRATTN_ERR_ARG
    assert lib.pairattn_tri_fwd_noalloc(Z, None, p, OUT, 64, 128, 4, 48, 0, stream=0, check=False) == \
        lib.PAIRATTN_ERR_UNSUPPORTED
    assert lib.pairattn_tri_fwd_noalloc(Z, None, p, Z, 64, 128, 4, 32, 0, stream=0, check=False) == \
        lib.PAIRATTN_ERR_ARG   # out overlaps z
    f = _params(lib.PAIRATTN_F32)
    st = lib.pairattn_tri_fwd_noalloc(Z, None, f, OUT, 353, 128, 4, 32, 1, stream=0, check=False)
    assert st == lib.PAIRATTN_ERR_UNSUPPORTED


def test_noalloc_without_device_reports_it():
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    st = lib.pairattn_tri_fwd_noalloc(Z, None, _params(lib.PAIRATTN_BF16), OUT, 64, 128, 4, 32, 0, stream=0,
                                      check=False)
    assert st == lib.PAIRATTN_ERR_DEVICE, lib.last_error()
