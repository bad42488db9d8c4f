"""Sparse attention over the indexer's selection (the path's consumer), float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (pages, not code):
  [PAT] "DeepSeek-V4 on ATOM" tracker, "CSA": the sparse attention kernel is
        an index gather, an online softmax and an attention-sink bias.
  [P27] "xkernels #27 -- [AMD/MI300A] DeepSeek-V4 DSA indexer + attention":
        the sparse-MLA attention kernel consumes the indexer's top-k indices.
  [P28] "xkernels #28 -- DeepSeek-V4 serving support": the selected rows
        live in the paged mxfp4 cache the gather reads.

Readings (the pages name the parts only; also listed in the design notes):
  * MQA over a latent: the row gathered for a selected position serves as
    both key and value for every head (the MLA arrangement), decoded
    exactly as the gather decodes it;
  * score s[r,h,j] = scale * (q[r,h,:] . v[r,j,:]) over the row's valid
    slots (sel_pos >= 0); the sink is one extra logit sink[h] per head with
    no value: p = exp(s) / (sum_j exp(s_j) + exp(sink[h]));
  * out[r,h,:] = sum_j p[r,h,j] v[r,j,:]; a row with no valid slot gives 0;
  * an online softmax is an evaluation order of this quantity, not another
    definition.
"""
from __future__ import annotations

import numpy as np

from .formats import bf16_bits_to_f64


def sparse_attention(q_bits, rows_bits, sel_pos, sink, scale):
    """out [R,H,D] float64.

    q_bits     [R,H,D] uint16 bf16 bits (the queries)
    rows_bits  [R,k,D] uint16 bf16 bits (the gathered rows, e.g. the output
               of mxfp4_paged_gather for the same sel_pos)
    sel_pos    [R,k]   int; slots < 0 take no part
    sink       [H]     float, or None (no sink: exp(sink) = 0)
    scale      float   the softmax scale
    """
    q = bf16_bits_to_f64(np.asarray(q_bits))
    v = bf16_bits_to_f64(np.asarray(rows_bits))
    valid = np.asarray(sel_pos) >= 0                                  # [R,k]
    s = float(scale) * np.einsum("rhd,rjd->rhj", q, v)               # [R,H,k]
    s = np.where(valid[:, None, :], s, -np.inf)
    sk = np.full(q.shape[1], -np.inf) if sink is None else np.asarray(sink, dtype=np.float64)
    m = np.maximum(s.max(axis=-1), sk[None, :])                      # [R,H], finite if a sink
    m = np.where(np.isfinite(m), m, 0.0)                             # no slot and no sink
    e = np.exp(s - m[..., None])                                     # exp(-inf) = 0
    den = e.sum(axis=-1) + np.exp(sk[None, :] - m)
    num = np.einsum("rhj,rjd->rhd", e, v)
    return np.where(den[..., None] > 0, num / np.where(den > 0, den, 1.0)[..., None], 0.0)
