"""The whole indexer hot path on one stream: logits -> top-k -> mxfp4 gather.

IndexerStep preallocates every output and validates every argument once, so
repeated calls only enqueue the three kernels of libxk (no allocation, no
host synchronisation, no per-call checks). The calls can also be captured
into a HIP graph (torch.cuda.graph) and replayed.
"""
from __future__ import annotations

import torch

from . import (_check, _lib, _stream, gather_args, logits_args, logits_paged_args, logits_topk_args,
               topk_args)


class IndexerStep:
    """One batch's launches. `outputs` = (logits, idx, gathered) of another
    step with the same shapes makes this step write into those buffers.
    With k None and a paged key cache (k_cache, k_cache_scale, K) the logits
    read the keys through block_table from that cache."""

    def __init__(self, q, k, w, limit, topk, kv_fp4, kv_scale, block_table, row_seq,
                 q_scale=None, k_scale=None, outputs=None, k_cache=None, k_cache_scale=None,
                 K=None):
        self.q, self.k, self.w, self.limit = q, k, w, limit
        self.q_scale, self.k_scale = q_scale, k_scale
        self.topk = topk
        self.kv_fp4, self.kv_scale = kv_fp4, kv_scale
        self.block_table, self.row_seq = block_table, row_seq
        # the C arguments below hold raw pointers: every tensor they name stays referenced here
        self.k_cache, self.k_cache_scale = k_cache, k_cache_scale
        lg, ix, ga = outputs if outputs is not None else (None, None, None)
        self.paged = k is None
        if self.paged:
            self._logits_args, self.logits = logits_paged_args(q, q_scale, w, k_cache, k_cache_scale,
                                                               block_table, limit, K, out=lg)
        else:
            self._logits_args, self.logits = logits_args(q, k, w, limit, q_scale, k_scale, out=lg)
        self._topk_args, self.idx, self.workspace = topk_args(self.logits, topk, limit, out=ix)
        self._gather_args, self.gathered = gather_args(kv_fp4, kv_scale, block_table, self.idx,
                                                       row_seq, out=ga)

    def outputs(self):
        return self.logits, self.idx, self.gathered

    def run_logits(self, stream=None):
        if self.paged:
            _check(_lib.xk_indexer_logits_paged(*self._logits_args, _stream(stream)))
        else:
            _check(_lib.xk_indexer_logits(*self._logits_args, _stream(stream)))
        return self.logits

    def run_topk(self, stream=None):
        _check(_lib.xk_indexer_topk(*self._topk_args, _stream(stream)))
        return self.idx

    def run_gather(self, stream=None):
        _check(_lib.xk_mxfp4_paged_gather(*self._gather_args, _stream(stream)))
        return self.gathered

    def enable_fused(self, workspace=None):
        """Prepare run_logits_topk (dense keys only): the same top-k written to
        self.idx by xk_indexer_logits_topk, which for prefill shapes does not
        write the score matrix. Steps run in order on one stream may share a
        workspace; returns the one this step uses."""
        if self.paged:
            raise ValueError("the fused call reads dense keys")
        self._fused_args, _, self.fused_workspace = logits_topk_args(
            self.q, self.k, self.w, self.topk, self.limit, self.q_scale, self.k_scale, out=self.idx,
            workspace=workspace)
        return self.fused_workspace

    def run_logits_topk(self, stream=None):
        _check(_lib.xk_indexer_logits_topk(*self._fused_args, _stream(stream)))
        return self.idx

    def run_fused(self, stream=None):
        """Top-k straight from q and k, then the gather (self.logits untouched)."""
        self.run_logits_topk(stream)
        self.run_gather(stream)
        return self.idx, self.gathered

    def __call__(self, stream=None):
        self.run_logits(stream)
        self.run_topk(stream)
        self.run_gather(stream)
        return self.logits, self.idx, self.gathered
