"""fp64 CPU reference for gated, pair-biased attention.  TEST INFRASTRUCTURE.

This module is the parity oracle for the HIP library.  Only the test suite,
the smoke check and the CPU-baseline leg of the benchmark may import it; the
product path never calls it, and it imports nothing from the product path.

It evaluates the dense definition, in float64, with numpy.  It is slow on
purpose: every logit, softmax weight and output is formed exactly as the
definition states, without tiling, fusion or online (streaming) softmax.

Sources (the pages print no formula, so the equations are a reading; see the
list of readings at the bottom of this docstring):
  * Pair representation Z[I, I, c] with O(I^2) memory; attention that takes
    queries along one axis and keys/values along the other without forming
    the I x I score matrix -- "Resumo Tecnico: Design-CP", Declaracao do
    Problema and Metodologia 1 (1D row sharding / 2D grid sharding).
  * Triangle-geometry self-attention over the pair representation inside the
    48-block Evoformer, MSA and pair representations influencing each other
    -- Intel "AlphaFold2 throughput" page, DL-inference bullet, and the Dell
    XE8545 page, EvoFormer paragraph ("triple attention").
  * The attention bias is produced by tensor matrix products, and the
    dominant operators are Einsum followed by Add (logits plus bias) --
    Intel page, Step 4 (slicing the attention module, operator fusion).
  * The attention interface takes (q_data, m_data, bias, nonbatched_bias):
    the per-row ``bias`` is sliced together with the query rows while the
    ``nonbatched_bias`` is shared by every slice -- Intel page, Step 4 code
    example.  This fixes the pair bias as a function of (query, key) only,
    independent of the row being attended.
  * Sliced evaluation over row chunks equals the unsliced call -- Intel page,
    Step 4.

Equations (c channels, H heads, d head width):
  LN(x)   = (x - mean(x)) / sqrt(var(x) + eps) * gamma + beta,
            mean/var over the channel axis, var the biased (1/c) estimate.
  q, k, v = LN(x) W_q, LN(x) W_k, LN(x) W_v            (split into H x d)
  g       = sigmoid(LN(x) W_g + b_g)
  B       = LN(Z) W_b                                   (one scalar per head)
  logit   = q . k / sqrt(d) + B[query, key]; masked keys get weight 0
  o       = sum_k softmax(logit)_k v_k;  o = 0 if every key is masked
  out     = (g * concat_h o_h) W_o + b_o

  Triangle attention, starting node (row i, query j, key k):
      logit = q[i,j].k[i,k]/sqrt(d) + B[j,k];  key k kept iff mask[i,k] != 0
      o[i,j] = sum_k w_k v[i,k]
  Triangle attention, ending node (column j, query i, key k):
      logit = q[i,j].k[k,j]/sqrt(d) + B[k,i];  key k kept iff mask[k,j] != 0
      o[i,j] = sum_k w_k v[k,j]
  MSA row attention with pair bias (sequence s, query i, key j):
      logit = q[s,i].k[s,j]/sqrt(d) + B[i,j] with B from LN_z(Z) W_b;
      key j kept iff mask[s,j] != 0
      o[s,i] = sum_j w_j v[s,j]

Readings where the pages are silent (also listed in the design notes):
  scale 1/sqrt(d); LN eps 1e-5, biased variance; no bias on q/k/v/B
  projections, biases b_g and b_o on gate and output; masked keys carry
  exactly zero weight (not a finite additive penalty) and a query with no
  kept key yields o = 0 (out = b_o); the output is the attention update
  (no residual add); the START bias is B[j,k] (the edge closing the
  triangle i-j-k) and the END bias is B[k,i].

Array conventions: inputs may be any float dtype (they are widened to
float64); masks are integer/bool arrays where nonzero means "keep".
Parameters are a mapping with the keys ln_gamma, ln_beta, w_q, w_k, w_v,
w_g, b_g, w_b, w_o, b_o (and lnz_gamma, lnz_beta for MSA) plus "eps";
linear maps act as y = x @ W.
"""
from __future__ import annotations

import math
from typing import Mapping, Optional, Sequence

import numpy as np

START = 0
END = 1


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _param(p: Mapping, name: str) -> np.ndarray:
    return _f64(p[name])


def _eps(p: Mapping) -> float:
    return float(p.get("eps", 1e-5)) if hasattr(p, "get") else 1e-5


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------
def layer_norm(x, gamma, beta, eps: float) -> np.ndarray:
    """LayerNorm over the last axis with the biased variance estimate."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


def sigmoid(t) -> np.ndarray:
    t = _f64(t)
    return 1.0 / (1.0 + np.exp(-t))


def heads(y: np.ndarray, H: int) -> np.ndarray:
    """[..., H*d] -> [..., H, d]."""
    return y.reshape(y.shape[:-1] + (H, y.shape[-1] // H))


def masked_softmax_weights(logits: np.ndarray, keep: np.ndarray) -> np.ndarray:
    """softmax over the last axis restricted to kept keys.

    ``keep`` broadcasts against ``logits``.  Dropped keys get weight exactly 0;
    a slice with no kept key gets all-zero weights.
    """
    keep = np.broadcast_to(keep.astype(bool), logits.shape)
    x = np.where(keep, logits, -np.inf)
    mx = x.max(axis=-1, keepdims=True)
    mx = np.where(np.isfinite(mx), mx, 0.0)
    e = np.where(keep, np.exp(x - mx), 0.0)
    s = e.sum(axis=-1, keepdims=True)
    return np.where(s > 0, e / np.where(s > 0, s, 1.0), 0.0)


def pair_bias(z, p: Mapping, H: int, ln_prefix: str = "ln") -> np.ndarray:
    """B[a, b, h] = LN(Z[a, b]) . W_b[:, h]  (natural [I, I, H] layout).

    ``ln_prefix`` selects the LayerNorm used: "ln" (triangle attention, the
    same LN as the projections) or "lnz" (MSA: separate LN of the pair input).
    """
    zh = layer_norm(z, p[f"{ln_prefix}_gamma"], p[f"{ln_prefix}_beta"], _eps(p))
    return zh @ _param(p, "w_b")


def attention_bias(z, p: Mapping, H: int, orientation: int = START,
                   ln_prefix: str = "ln", queries: Optional[Sequence[int]] = None) -> np.ndarray:
    """Additive logit term indexed [h, query, key] for one orientation.

    START: bias[h, j, k] = B[j, k, h];  END: bias[h, i, k] = B[k, i, h].
    ``queries`` restricts the query axis (only the pairs it needs are read).
    """
    z = np.asarray(z)
    I = z.shape[0]
    q_i = _as_index(queries, I)
    if orientation == START:
        B = pair_bias(z[q_i], p, H, ln_prefix)          # [Q, I(k), H] = B[j, k]
        return np.ascontiguousarray(B.transpose(2, 0, 1))
    if orientation == END:
        B = pair_bias(z[:, q_i], p, H, ln_prefix)       # [I(k), Q, H] = B[k, i]
        return np.ascontiguousarray(B.transpose(2, 1, 0))
    raise ValueError("orientation must be START (0) or END (1)")


def gated_output(o: np.ndarray, g_pre: np.ndarray, p: Mapping) -> np.ndarray:
    """out = (sigmoid(g_pre + b_g) * o) W_o + b_o with o, g_pre [..., H*d]."""
    g = sigmoid(g_pre + _param(p, "b_g"))
    return (g * o) @ _param(p, "w_o") + _param(p, "b_o")


def _attend_one_row(x_row, bias_hqk, keep_k, p: Mapping, H: int,
                    queries: Optional[np.ndarray]) -> np.ndarray:
    """One attention row: x_row [P, c] supplies queries, keys and values.

    bias_hqk [H, Q, P] (rows already restricted to ``queries``), keep_k [P].
    Returns out [Q, c] for the selected query positions.
    """
    xh = layer_norm(x_row, p["ln_gamma"], p["ln_beta"], _eps(p))
    xq = xh if queries is None else xh[queries]
    q = heads(xq @ _param(p, "w_q"), H)                 # [Q, H, d]
    k = heads(xh @ _param(p, "w_k"), H)                 # [P, H, d]
    v = heads(xh @ _param(p, "w_v"), H)                 # [P, H, d]
    g_pre = xq @ _param(p, "w_g")                       # [Q, H*d]
    d = q.shape[-1]
    logits = np.einsum("qhd,khd->hqk", q, k) / math.sqrt(d) + bias_hqk
    w = masked_softmax_weights(logits, keep_k[None, None, :])
    o = np.einsum("hqk,khd->qhd", w, v).reshape(q.shape[0], -1)
    return gated_output(o, g_pre, p)


def _as_index(sel, n: int) -> np.ndarray:
    return np.arange(n) if sel is None else np.asarray(sel, dtype=np.int64).reshape(-1)


# ----------------------------------------------------------------------------
# triangle attention
# ----------------------------------------------------------------------------
def tri_start(z, mask, p: Mapping, H: int, rows: Optional[Sequence[int]] = None,
              queries: Optional[Sequence[int]] = None) -> np.ndarray:
    """Triangle attention around the starting node.

    z [I, I, c]; mask [I, I] or None.  Returns out[rows][:, queries] with
    shape [len(rows), len(queries), c] (all rows / queries by default).
    Attention row i uses pairs (i, *): queries j, keys k along the row, and
    the bias B[j, k] of the edge that closes the triangle (i, j, k).
    """
    z = np.asarray(z)
    I = z.shape[0]
    rows_i = _as_index(rows, I)
    q_i = _as_index(queries, I)
    bias = attention_bias(z, p, H, START, queries=q_i)
    keep = np.ones((I, I), bool) if mask is None else np.asarray(mask) != 0
    out = np.empty((len(rows_i), len(q_i), z.shape[-1]))
    for n, i in enumerate(rows_i):
        out[n] = _attend_one_row(z[i], bias, keep[i], p, H, q_i)
    return out


def tri_end(z, mask, p: Mapping, H: int, cols: Optional[Sequence[int]] = None,
            queries: Optional[Sequence[int]] = None) -> np.ndarray:
    """Triangle attention around the ending node, written in index form.

    Attention column j uses pairs (*, j): query i is the pair (i, j), key k
    the pair (k, j), the bias is B[k, i] and key k is kept iff mask[k, j].
    Returns out[queries][:, cols] with shape [len(queries), len(cols), c].
    """
    z = np.asarray(z)
    I = z.shape[0]
    cols_j = _as_index(cols, I)
    q_i = _as_index(queries, I)
    keep = np.ones((I, I), bool) if mask is None else np.asarray(mask) != 0
    bias = attention_bias(z, p, H, END, queries=q_i)      # [H, Q(i), I(k)]
    out = np.empty((len(q_i), len(cols_j), z.shape[-1]))
    for n, j in enumerate(cols_j):
        zc = _f64(z[:, j, :])                            # pairs (k, j) for all k
        xh = layer_norm(zc, p["ln_gamma"], p["ln_beta"], _eps(p))
        q = heads(xh[q_i] @ _param(p, "w_q"), H)         # q[i, j]
        k = heads(xh @ _param(p, "w_k"), H)              # k[k, j]
        v = heads(xh @ _param(p, "w_v"), H)              # v[k, j]
        g_pre = xh[q_i] @ _param(p, "w_g")
        d = q.shape[-1]
        # logit[h, i, k] = q[i,j].k[k,j]/sqrt(d) + B[k, i, h]
        logits = np.einsum("ihd,khd->hik", q, k) / math.sqrt(d) + bias
        w = masked_softmax_weights(logits, keep[:, j][None, None, :])
        o = np.einsum("hik,khd->ihd", w, v).reshape(len(q_i), -1)
        out[:, n, :] = gated_output(o, g_pre, p)
    return out


def tri_fwd(z, mask, p: Mapping, H: int, orientation: int) -> np.ndarray:
    """Full triangle attention output [I, I, c] for either orientation."""
    if orientation == START:
        return tri_start(z, mask, p, H)
    if orientation == END:
        return tri_end(z, mask, p, H)
    raise ValueError("orientation must be START (0) or END (1)")


def tri_points(z, mask, p: Mapping, H: int, orientation: int, points) -> np.ndarray:
    """out[a, b] for a list of pair indices (a, b), each evaluated on its own.

    For START the attention row is a and the query b; for END the attention
    column is b and the query a.  Returns [n, c].
    """
    pts = np.asarray(points, dtype=np.int64).reshape(-1, 2)
    res = np.empty((pts.shape[0], np.asarray(z).shape[-1]))
    for n, (a, b) in enumerate(pts):
        if orientation == START:
            res[n] = tri_start(z, mask, p, H, rows=[a], queries=[b])[0, 0]
        else:
            res[n] = tri_end(z, mask, p, H, cols=[b], queries=[a])[0, 0]
    return res


def tri_rows(z_rows, bias_hqk, mask_rows, p: Mapping, H: int,
             queries: Optional[Sequence[int]] = None, bias_restricted: bool = False) -> np.ndarray:
    """Starting-node attention for a block of rows with a given bias.

    z_rows [R, I, c] are rows of Z; bias_hqk [H, I, I] is the full-length
    additive term (query, key) computed from the whole Z; mask_rows [R, I]
    or None.  This is one device's share when the query rows are split
    across devices while keys/values stay whole (self-attention recast as
    cross-attention: Design-CP, Metodologia 1).  Returns [R, Q, c].
    With ``bias_restricted`` the bias holds only the rows of ``queries``
    ([H, Q, I], e.g. from attention_bias over those rows of Z).
    """
    z_rows = np.asarray(z_rows)
    R, I = z_rows.shape[0], z_rows.shape[1]
    q_i = _as_index(queries, I)
    bias = _f64(bias_hqk) if bias_restricted else _f64(bias_hqk)[:, q_i, :]
    if bias.shape[1] != len(q_i):
        raise ValueError("bias rows do not match the selected queries")
    keep = np.ones((R, I), bool) if mask_rows is None else np.asarray(mask_rows) != 0
    out = np.empty((R, len(q_i), z_rows.shape[-1]))
    for r in range(R):
        out[r] = _attend_one_row(z_rows[r], bias, keep[r], p, H, q_i)
    return out


# ----------------------------------------------------------------------------
# MSA row attention with pair bias
# ----------------------------------------------------------------------------
def msa_row(m, z, mask, p: Mapping, H: int, seqs: Optional[Sequence[int]] = None,
            queries: Optional[Sequence[int]] = None) -> np.ndarray:
    """Row-wise gated attention over the MSA with a bias from the pair tensor.

    m [S, I, c_m], z [I, I, c_z], mask [S, I] or None.  Sequence s attends
    over its own residues; the bias B[i, j] = LN_z(Z[i, j]) W_b is shared by
    every sequence.  Returns out[seqs][:, queries] as [len(seqs), Q, c_m].
    """
    m = np.asarray(m)
    S, I = m.shape[0], m.shape[1]
    s_i = _as_index(seqs, S)
    q_i = _as_index(queries, I)
    bias = attention_bias(z, p, H, START, ln_prefix="lnz", queries=q_i)
    keep = np.ones((S, I), bool) if mask is None else np.asarray(mask) != 0
    out = np.empty((len(s_i), len(q_i), m.shape[-1]))
    for n, s in enumerate(s_i):
        out[n] = _attend_one_row(m[s], bias, keep[s], p, H, q_i)
    return out


# ----------------------------------------------------------------------------
# one key shard at a time (2D grid sharding with ring attention)
# ----------------------------------------------------------------------------
def tri_partial(q_pairs, kv_pairs, bias_hqk, mask_rows, p: Mapping, H: int):
    """Starting-node attention of R rows' query pairs against one shard of
    key pairs of the same rows.

    In the 2D grid of the Design-CP page (Metodologia 1, 2D grid sharding)
    a device holds the pairs of its rows and columns: its queries.  Keys and
    values arrive shard by shard around the ring, and the softmax is
    assembled across shards without ever forming the I x I scores.
    q_pairs [R, Jq, c] and kv_pairs [R, Kn, c]; bias_hqk [H, Jq, Kn]
    (query, key) for these queries and keys; mask_rows [R, Kn] or None.

    Returns (o, lse):
      o   [R, Jq, H*d]  per head, the softmax-weighted sum of v over this
                        shard's kept keys (0 when it has none);
      lse [R, H, Jq]    ln sum_k exp(logit_k) over the same keys (-inf when
                        none), so that shards combine by
                        lse = ln sum_s exp(lse_s),  o = sum_s exp(lse_s - lse) o_s.
    """
    qp, kp = _f64(q_pairs), _f64(kv_pairs)
    R, Jq, Kn = qp.shape[0], qp.shape[1], kp.shape[1]
    bias = _f64(bias_hqk)
    keep = np.ones((R, Kn), bool) if mask_rows is None else np.asarray(mask_rows) != 0
    hd = _param(p, "w_q").shape[1]
    o = np.empty((R, Jq, hd))
    lse = np.empty((R, H, Jq))
    for r in range(R):
        xq = layer_norm(qp[r], p["ln_gamma"], p["ln_beta"], _eps(p))
        xk = layer_norm(kp[r], p["ln_gamma"], p["ln_beta"], _eps(p))
        q = heads(xq @ _param(p, "w_q"), H)
        k = heads(xk @ _param(p, "w_k"), H)
        v = heads(xk @ _param(p, "w_v"), H)
        logits = np.einsum("qhd,khd->hqk", q, k) / math.sqrt(q.shape[-1]) + bias
        kept = keep[r][None, None, :]
        w = masked_softmax_weights(logits, kept)
        o[r] = np.einsum("hqk,khd->qhd", w, v).reshape(Jq, hd)
        x = np.where(kept, logits, -np.inf)
        mx = x.max(axis=-1)
        safe = np.where(np.isfinite(mx), mx, 0.0)
        tot = np.where(kept, np.exp(x - safe[..., None]), 0.0).sum(axis=-1)
        lse[r] = np.where(tot > 0, safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    return o, lse


def tri_partial_finish(q_pairs, o, p: Mapping, H: int) -> np.ndarray:
    """out [R, Jq, c] = (sigmoid(LN(q_pairs) W_g + b_g) * o) W_o + b_o, with o
    the per-head outputs assembled over every key shard."""
    qp = _f64(q_pairs)
    xq = layer_norm(qp, p["ln_gamma"], p["ln_beta"], _eps(p))
    return gated_output(_f64(o), xq @ _param(p, "w_g"), p)


# ----------------------------------------------------------------------------
# error metrics used by the parity bar
# ----------------------------------------------------------------------------
def max_abs_err(y, ref) -> float:
    return float(np.max(np.abs(_f64(y) - _f64(ref)))) if np.size(ref) else 0.0


def mean_rel_err(y, ref) -> float:
    """sum |y - ref| / sum |ref| (aggregate relative error)."""
    num = np.sum(np.abs(_f64(y) - _f64(ref)))
    den = np.sum(np.abs(_f64(ref)))
    return float(num / den) if den > 0 else float(num)
