"""Sparse MLA decode over NVFP4 cache rows.  TEST INFRASTRUCTURE ONLY (see package doc).

Source: "Prime Intellect Launches Prime Inference, Serving 600B Tokens Daily",
section "Four-bit caches make room": for each decode token the native kernel
loads only the cache rows named by the sparse indexer's 2,048-position list,
unpacks them on chip and runs attention with FP16 operands and FP32
accumulation; empty entries of the list are handled specially.  A staged
implementation instead unpacked NVFP4 into FP8 buffers first.

What is computed here is the plain definition (float64 throughout), which the
kernel reaches up to the rounding of its FP16 probabilities and FP32 sums:

  for token t and head h, over the valid entries J = {j : idx[t, j] >= 0}
  (a multiset: a repeated row counts once per entry),
      K_j   = dequant(pool[idx[t, j]])            576 values (latent | rope)
      V_j   = K_j[0:512]                          the latent (MLA: K and V share it)
      s_j   = softmax_scale * sum_k q[t, h, k] * K_j[k]
      lse   = ln sum_j exp(s_j)                   natural log, scale included
      out   = sum_j exp(s_j - lse) * V_j          rounded once to fp16
  and for an empty J: out = 0, lse = -inf.

Readings taken here where the page leaves the step open:
  * An empty entry (index -1) is masked: it takes no part in the softmax.  A
    zero row that did take part would add exp(0 - m) to the denominator and
    make the result depend on how many empties pad the list.
  * The query's first 512 values pair with the latent and its last 64 with
    the rope part (the absorbed form of multi-head latent attention).
"""

import numpy as np

from .formats import (HEAD_DIM, LATENT_DIM, ROW_BYTES, nvfp4_unpack_rows_ref,
                      fp8_stage_rows_ref, fp8_unpack_rows_ref, e4m3_table)

_E4M3 = e4m3_table()


def dense_rows_for(pool, ids):
    """Exact float64 [len(ids), 576] values of the cache rows `ids` of `pool`.

    `pool` is anything that maps an int64 id array to uint8 [n, 352] rows by
    indexing (a numpy array, or an object that builds rows on demand).
    """
    rows = np.asarray(pool[np.asarray(ids, dtype=np.int64)], dtype=np.uint8)
    if rows.ndim != 2 or rows.shape[1] != ROW_BYTES:
        raise ValueError("pool rows must be uint8 [n, 352]")
    return nvfp4_unpack_rows_ref(rows)


def _attend(q_th, K, softmax_scale):
    """One token: q_th float64 [H, 576], K float64 [n, 576] -> (out float64 [H, 512], lse float64 [H])."""
    H = q_th.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, LATENT_DIM)), np.full(H, -np.inf)
    s = softmax_scale * (K @ q_th.T)                  # [n, H] scores
    m = np.max(s, axis=0)                             # [H]
    lse = m + np.log(np.sum(np.exp(s - m), axis=0))   # [H]
    w = np.exp(s - lse)                               # [n, H] softmax weights
    out = w.T @ K[:, :LATENT_DIM]                     # [H, 512]
    return out, lse


def sparse_mla_decode_ref(q, pool, indices, softmax_scale, tokens=None, rows_fn=None):
    """Sparse MLA decode: q fp16 [T, H, 576], pool uint8 rows, indices int32 [T, K].

    Returns (out float16 [len(tokens), H, 512], lse float64 [len(tokens), H])
    for the requested `tokens` (default: all).  `rows_fn(ids)` may replace the
    default NVFP4 row decode (used by the staged variant).
    """
    q = np.asarray(q)
    if q.dtype != np.float16 or q.ndim != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be float16 [T, H, 576]")
    indices = np.asarray(indices)
    T, H, _ = q.shape
    if indices.ndim != 2 or indices.shape[0] != T:
        raise ValueError("indices must be int32 [T, K]")
    if tokens is None:
        tokens = range(T)
    tokens = list(tokens)
    decode = rows_fn if rows_fn is not None else (lambda ids: dense_rows_for(pool, ids))
    out = np.zeros((len(tokens), H, LATENT_DIM), dtype=np.float16)
    lse = np.zeros((len(tokens), H), dtype=np.float64)
    for i, t in enumerate(tokens):
        ids = indices[t][indices[t] >= 0].astype(np.int64)
        K = decode(ids) if len(ids) else np.zeros((0, HEAD_DIM))
        o, l = _attend(q[t].astype(np.float64), K, float(softmax_scale))
        out[i] = o.astype(np.float16)          # one round-to-nearest-even
        lse[i] = l
    return out, lse


def lse_combine_ref(partial_out, partial_lse):
    """Merge split results: partial_out float [S, ..., 512], partial_lse float [S, ...].

    Each split s carries its normalized output O_s and its log-sum-exp lse_s.
    lse = ln sum_s exp(lse_s); out = sum_s exp(lse_s - lse) * O_s.  Splits with
    lse_s = -inf weigh zero; if every split is -inf, out = 0 and lse = -inf.
    Returns (out float64 [..., 512], lse float64 [...]).
    """
    po = np.asarray(partial_out, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    m = np.max(pl, axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(pl), np.exp(pl - m_safe), 0.0)          # [S, ...]
    tot = np.sum(w, axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), -np.inf)
    out = np.where(finite[..., None],
                   np.sum(w[..., None] * np.where(np.isfinite(pl)[..., None], po, 0.0), axis=0)
                   / np.where(finite, tot, 1.0)[..., None],
                   0.0)
    return out, lse


def sparse_mla_decode_fp8rows_ref(q, pool, indices, softmax_scale, tokens=None):
    """Staged variant: each gathered row is first re-encoded as 576 E4M3 values
    (fp8_stage_rows_ref), then attention runs over those FP8 rows exactly as in
    sparse_mla_decode_ref.  The result differs from the fused path because the
    FP8 re-encoding rounds the 6-bit NVFP4 products."""
    def rows_fn(ids):
        rows = np.asarray(pool[np.asarray(ids, dtype=np.int64)], dtype=np.uint8)
        return _E4M3[fp8_stage_rows_ref(rows)]
    return sparse_mla_decode_ref(q, pool, indices, softmax_scale, tokens=tokens, rows_fn=rows_fn)


def sparse_mla_decode_fp8pool_ref(q, pool, indices, softmax_scale, tokens=None):
    """Decode over a pool of 576-byte FP8 rows (the cache format before NVFP4): the same
    definition as sparse_mla_decode_ref, with K_j the E4M3 values of pool row idx[t, j].
    `pool` maps an int64 id array to uint8 [n, 576] rows by indexing."""
    def rows_fn(ids):
        return fp8_unpack_rows_ref(np.asarray(pool[np.asarray(ids, dtype=np.int64)], dtype=np.uint8))
    return sparse_mla_decode_ref(q, pool, indices, softmax_scale, tokens=tokens, rows_fn=rows_fn)
