"""Seeded synthetic inputs for pair-biased attention.

This module only draws random numbers and rounds them to the storage
precision.  It performs none of the attention arithmetic, so both the
fp64 reference implementation and the HIP path can take their inputs
from here without sharing any part of the method.

Every array is drawn with ``numpy.random.Generator(PCG64)``.  One
``SeedSequence(seed)`` per case is split into independent child streams
(pair tensor, MSA tensor, weights, masks), so changing one part of a
case never shifts the random numbers of another.

Values are drawn in float32.  For the bf16 path they are rounded to
bfloat16 with round-to-nearest-even and handed out both as the exact
float32 value of that bf16 number (``*_f32``) and as its 16-bit pattern
(``*_bits``); bf16 -> float is exact, so every consumer sees the same
numbers.

Workload recipes (the pages publish no dataset for this operator; these
synthetic tensors stand in for the residue counts the pages mention):
  * triangle, fp32:  Z[64,64,128] ~ N(0,1), H=4, d=32, no mask
  * triangle, bf16:  Z[384,384,128], H=4, d=32, last 10% of residues padded
  * MSA row + pair bias: M[512,384,256], Z[384,384,128], H=8, d=32,
    Bernoulli(0.95) per-entry key mask
  * triangle, bf16:  Z[1536,1536,128], H=4, d=32, no mask
  * row block: rows 0..511 of Z[4096,4096,128] built from one 171-residue
    block tiled 24 times (cropped) plus N(0, 0.1^2) noise
Weights are N(0, 1/fan_in); LayerNorm gamma=1, beta=0; gate and output
biases 0 unless a case asks for random affine/bias terms.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

START = 0
END = 1


# ----------------------------------------------------------------------------
# bf16 rounding (storage format only)
# ----------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 -> bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # NaN is not produced by the generators; keep the plain RNE formula.
    rounding_bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding_bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact bfloat16 -> float32 widening."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly representable in bf16 (RNE)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ----------------------------------------------------------------------------
# parameter sets
# ----------------------------------------------------------------------------
PARAM_NAMES = ("ln_gamma", "ln_beta", "w_q", "w_k", "w_v", "w_g", "b_g",
               "w_b", "w_o", "b_o", "lnz_gamma", "lnz_beta")


@dataclasses.dataclass
class Params:
    """Weights of one gated pair-biased attention module (float32 values).

    Shapes (c = input channels, H heads, d head width, cz = pair channels):
      ln_gamma, ln_beta: [c]           w_q, w_k, w_v, w_g: [c, H*d]
      b_g: [H*d]                       w_b: [cz, H]
      w_o: [H*d, c]                    b_o: [c]
      lnz_gamma, lnz_beta: [cz] (MSA only: LayerNorm of the pair input)
    Linear maps act as ``y = x @ W``.
    """
    ln_gamma: np.ndarray
    ln_beta: np.ndarray
    w_q: np.ndarray
    w_k: np.ndarray
    w_v: np.ndarray
    w_g: np.ndarray
    b_g: np.ndarray
    w_b: np.ndarray
    w_o: np.ndarray
    b_o: np.ndarray
    lnz_gamma: Optional[np.ndarray] = None
    lnz_beta: Optional[np.ndarray] = None
    eps: float = 1e-5

    def as_dict(self) -> Dict[str, object]:
        """Plain mapping of the arrays plus ``eps`` (the form the fp64 reference takes)."""
        d: Dict[str, object] = {k: getattr(self, k) for k in PARAM_NAMES if getattr(self, k) is not None}
        d["eps"] = self.eps
        return d

    def replace(self, **kw) -> "Params":
        return dataclasses.replace(self, **kw)


def _normal(rng: np.random.Generator, shape, std: float) -> np.ndarray:
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _maybe_bf16(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_to_bf16(x) if dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


def make_params(rng: np.random.Generator, c: int, H: int, d: int, dtype: str,
                cz: Optional[int] = None, affine: bool = False,
                biases: bool = False) -> Params:
    """Draw one weight set: W ~ N(0, 1/fan_in).

    ``affine`` draws gamma = 1 + 0.1 N(0,1), beta = 0.1 N(0,1) instead of 1/0;
    ``biases`` draws b_g, b_o ~ N(0,1) instead of zeros.  ``cz`` (MSA) adds
    the pair-input LayerNorm and sizes w_b as [cz, H].
    """
    hd = H * d
    cb = c if cz is None else cz
    w_q = _normal(rng, (c, hd), 1.0 / np.sqrt(c))
    w_k = _normal(rng, (c, hd), 1.0 / np.sqrt(c))
    w_v = _normal(rng, (c, hd), 1.0 / np.sqrt(c))
    w_g = _normal(rng, (c, hd), 1.0 / np.sqrt(c))
    w_b = _normal(rng, (cb, H), 1.0 / np.sqrt(cb))
    w_o = _normal(rng, (hd, c), 1.0 / np.sqrt(hd))
    if affine:
        g = 1.0 + _normal(rng, (c,), 0.1)
        b = _normal(rng, (c,), 0.1)
    else:
        g = np.ones((c,), np.float32)
        b = np.zeros((c,), np.float32)
    if biases:
        b_g = _normal(rng, (hd,), 1.0)
        b_o = _normal(rng, (c,), 1.0)
    else:
        b_g = np.zeros((hd,), np.float32)
        b_o = np.zeros((c,), np.float32)
    lnz_g = lnz_b = None
    if cz is not None:
        if affine:
            lnz_g = 1.0 + _normal(rng, (cz,), 0.1)
            lnz_b = _normal(rng, (cz,), 0.1)
        else:
            lnz_g = np.ones((cz,), np.float32)
            lnz_b = np.zeros((cz,), np.float32)
    f = lambda a: None if a is None else _maybe_bf16(a, dtype)
    return Params(ln_gamma=f(g), ln_beta=f(b), w_q=f(w_q), w_k=f(w_k), w_v=f(w_v),
                  w_g=f(w_g), b_g=f(b_g), w_b=f(w_b), w_o=f(w_o), b_o=f(b_o),
                  lnz_gamma=f(lnz_g), lnz_beta=f(lnz_b))


# ----------------------------------------------------------------------------
# masks
# ----------------------------------------------------------------------------
def residue_padding(I: int, frac: float = 0.1) -> np.ndarray:
    """r[a] = 1 for real residues, 0 for the last floor(frac*I) (padding)."""
    r = np.ones((I,), np.uint8)
    npad = int(np.floor(frac * I))
    if npad:
        r[I - npad:] = 0
    return r


def pair_mask_from_residues(r: np.ndarray) -> np.ndarray:
    """M[a,b] = r[a] * r[b]."""
    r = r.astype(np.uint8)
    return np.ascontiguousarray(np.outer(r, r).astype(np.uint8))


def key_only_mask(r: np.ndarray) -> np.ndarray:
    """M[a,b] = r[b] (every row masks the same keys)."""
    I = r.shape[0]
    return np.ascontiguousarray(np.broadcast_to(r.astype(np.uint8)[None, :], (I, I)).copy())


def bernoulli_mask(rng: np.random.Generator, shape, keep: float) -> np.ndarray:
    return (rng.random(size=shape, dtype=np.float32) < np.float32(keep)).astype(np.uint8)


# ----------------------------------------------------------------------------
# cases
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class TriCase:
    I: int
    c: int
    H: int
    d: int
    dtype: str
    z: np.ndarray                       # [I, I, c] float32 values
    mask: Optional[np.ndarray]          # [I, I] uint8 or None
    params_start: Params
    params_end: Params
    seed: int


@dataclasses.dataclass
class MsaCase:
    S: int
    I: int
    c_m: int
    c_z: int
    H: int
    d: int
    dtype: str
    m: np.ndarray                       # [S, I, c_m]
    z: np.ndarray                       # [I, I, c_z]
    mask: Optional[np.ndarray]          # [S, I] uint8 or None
    params: Params
    seed: int


def _children(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def make_tri_case(I: int, c: int = 128, H: int = 4, d: int = 32, dtype: str = BF16,
                  mask: str = "none", seed: int = 0, affine: bool = False,
                  biases: bool = False, z_std: float = 1.0) -> TriCase:
    """Triangle-attention case.

    mask: "none"; "pad" (M = r r^T with the last 10% of residues padded);
    "keypad" (M[a,b] = r[b]); "random" (Bernoulli(0.8) per pair, with a
    fully masked row and a single-key row planted for edge coverage).
    """
    r_z, r_ws, r_we, r_m = _children(seed, 4)
    z = _maybe_bf16(_normal(r_z, (I, I, c), z_std), dtype)
    ps = make_params(r_ws, c, H, d, dtype, affine=affine, biases=biases)
    pe = make_params(r_we, c, H, d, dtype, affine=affine, biases=biases)
    if mask == "none":
        mk = None
    elif mask == "pad":
        mk = pair_mask_from_residues(residue_padding(I))
    elif mask == "keypad":
        mk = key_only_mask(residue_padding(I))
    elif mask == "random":
        mk = bernoulli_mask(r_m, (I, I), 0.8)
        if I >= 3:
            mk[1, :] = 0
            mk[:, 1] = 0
            mk[2, :] = 0
            mk[2, I - 1] = 1
            mk[0, 2] = 1
    else:
        raise ValueError(f"unknown mask kind {mask!r}")
    return TriCase(I=I, c=c, H=H, d=d, dtype=dtype, z=z, mask=mk,
                   params_start=ps, params_end=pe, seed=seed)


def make_msa_case(S: int, I: int, c_m: int = 256, c_z: int = 128, H: int = 8, d: int = 32,
                  dtype: str = BF16, mask: str = "bernoulli", seed: int = 0,
                  affine: bool = False, biases: bool = False) -> MsaCase:
    """MSA row attention case.

    mask: "none"; "bernoulli" (Mm[s,j] ~ Bernoulli(0.95) per entry);
    "columns" (the same 5% of columns masked in every row).
    """
    r_m, r_z, r_w, r_k = _children(seed, 4)
    m = _maybe_bf16(_normal(r_m, (S, I, c_m), 1.0), dtype)
    z = _maybe_bf16(_normal(r_z, (I, I, c_z), 1.0), dtype)
    p = make_params(r_w, c_m, H, d, dtype, cz=c_z, affine=affine, biases=biases)
    if mask == "none":
        mk = None
    elif mask == "bernoulli":
        mk = bernoulli_mask(r_k, (S, I), 0.95)
    elif mask == "columns":
        ncol = max(1, int(round(0.05 * I)))
        cols = r_k.choice(I, size=ncol, replace=False)
        mk = np.ones((S, I), np.uint8)
        mk[:, cols] = 0
    else:
        raise ValueError(f"unknown mask kind {mask!r}")
    return MsaCase(S=S, I=I, c_m=c_m, c_z=c_z, H=H, d=d, dtype=dtype, m=m, z=z,
                   mask=mk, params=p, seed=seed)


def make_assembly_z_bits(I: int, c: int, asu: int, noise_std: float, seed: int,
                         rows: Optional[slice] = None, workers: Optional[int] = None) -> np.ndarray:
    """bf16 bits of a repeated-block pair tensor, generated row by row.

    Z[a,b] = A[a mod asu, b mod asu] + noise_std * eps, A ~ N(0,1)^[asu,asu,c],
    eps ~ N(0,1) drawn per row from a per-row child stream, so any row can be
    regenerated on its own (and rows are filled in parallel threads without
    changing a bit).  Returns uint16 [n_rows, I, c].
    """
    import concurrent.futures as cf
    import os

    seq = np.random.SeedSequence(seed)
    s_asu, s_rows = seq.spawn(2)
    A = np.random.Generator(np.random.PCG64(s_asu)).standard_normal((asu, asu, c), dtype=np.float32)
    rows = rows or slice(0, I)
    idx = list(range(*rows.indices(I)))
    out = np.empty((len(idx), I, c), np.uint16)
    reps = -(-I // asu)

    def fill(n: int) -> None:
        a = idx[n]
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1, a])))
        base = np.tile(A[a % asu], (reps, 1))[:I]
        noise = rng.standard_normal((I, c), dtype=np.float32) * np.float32(noise_std)
        out[n] = f32_to_bf16_bits(base + noise)

    workers = workers or min(16, os.cpu_count() or 1)
    if workers <= 1 or len(idx) < 8:
        for n in range(len(idx)):
            fill(n)
    else:
        with cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(len(idx))))
    return out


@dataclasses.dataclass
class RowsCase:
    I: int
    R: int
    c: int
    H: int
    d: int
    zbits: np.ndarray                   # [I, I, c] bf16 bits of the whole pair tensor
    r0: int                             # the block holds rows r0 .. r0+R-1
    params: Params
    seed: int


def make_rows_case(I: int, R: int, c: int = 128, H: int = 4, d: int = 32, asu: int = 171,
                   noise: float = 0.1, seed: int = 0, r0: Optional[int] = None) -> RowsCase:
    """A block of R starting-node rows of a large repeated-block pair tensor
    (bf16), with random LayerNorm affine terms and biases.  The block holds
    rows r0 .. r0+R-1 (rows 0 .. R-1 by default)."""
    zbits = make_assembly_z_bits(I, c, asu, noise, seed)
    r_w = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2])))
    params = make_params(r_w, c, H, d, BF16, affine=True, biases=True)
    r0 = 0 if r0 is None else r0
    return RowsCase(I=I, R=R, c=c, H=H, d=d, zbits=zbits, r0=r0, params=params, seed=seed)


def make_z_device(I: int, c: int, seed: int, dtype: str = BF16, device: str = "cuda"):
    """Z[I, I, c] ~ N(0, 1) drawn on the device, for pair tensors too large
    to generate on the host (I = 16384: 68.7 GB in bf16).  Row blocks are
    drawn in order from one torch generator seeded with `seed`, so the tensor
    depends only on (I, c, seed, dtype); the values are rounded to the dtype."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    z = torch.empty((I, I, c), dtype=torch.bfloat16 if dtype == BF16 else torch.float32, device=device)
    step = max(1, (1 << 27) // (I * c))
    for r0 in range(0, I, step):
        r1 = min(I, r0 + step)
        z[r0:r1] = torch.randn((r1 - r0, I, c), generator=g, device=device, dtype=torch.float32).to(z.dtype)
    return z


def make_chunked_params(c: int, H: int, d: int, seed: int, dtype: str = BF16) -> Params:
    """Weights of the device-generated pair tensor workloads (host, seeded)."""
    r_w = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
    return make_params(r_w, c, H, d, dtype, affine=True, biases=True)


# ----------------------------------------------------------------------------
# the workload table
# ----------------------------------------------------------------------------
CONFIGS = {
    "tri_fp32_i64": dict(kind="tri", I=64, c=128, H=4, d=32, dtype=F32, mask="none", seed=1),
    "tri_bf16_i384_pad": dict(kind="tri", I=384, c=128, H=4, d=32, dtype=BF16, mask="pad", seed=2),
    "msa_bf16_s512_i384": dict(kind="msa", S=512, I=384, c_m=256, c_z=128, H=8, d=32, dtype=BF16,
                               mask="bernoulli", seed=3),
    "tri_bf16_i1536": dict(kind="tri", I=1536, c=128, H=4, d=32, dtype=BF16, mask="none", seed=4),
    "rows_bf16_i4096_r512": dict(kind="rows", I=4096, R=512, c=128, H=4, d=32, dtype=BF16,
                                 asu=171, noise=0.1, seed=5),
    # I far beyond the one-pass workspace: Z drawn on the device, attention in blocks of 1024 rows
    "tri_bf16_i16384_chunked": dict(kind="tri_chunked", I=16384, c=128, H=4, d=32, dtype=BF16, mask="none",
                                    block=1024, seed=7),
    # extra-MSA row attention: 5120 sequences of 64 channels, fp32 end to end
    "msa_fp32_s5120_i384": dict(kind="msa", S=5120, I=384, c_m=64, c_z=128, H=8, d=32, dtype=F32,
                                mask="bernoulli", seed=6),
}
