"""The whole indexer hot path on one stream: logits -> top-k -> mxfp4 gather.

IndexerStep preallocates every output once, so repeated calls only enqueue
the three kernels of libxk (no allocation, no host synchronisation).
"""
from __future__ import annotations

import torch

from . import xk_indexer_logits, xk_indexer_topk, xk_mxfp4_paged_gather, \
    xk_indexer_topk_workspace_size


class IndexerStep:
    def __init__(self, q, k, w, limit, topk, kv_fp4, kv_scale, block_table, row_seq,
                 q_scale=None, k_scale=None):
        self.q, self.k, self.w, self.limit = q, k, w, limit
        self.q_scale, self.k_scale = q_scale, k_scale
        self.topk = topk
        self.kv_fp4, self.kv_scale = kv_fp4, kv_scale
        self.block_table, self.row_seq = block_table, row_seq
        B, T = q.shape[0], q.shape[1]
        K = k.shape[1]
        dev = q.device
        self.logits = torch.empty((B, T, K), dtype=torch.float32, device=dev)
        self.idx = torch.empty((B * T, topk), dtype=torch.int32, device=dev)
        self.gathered = torch.empty((B * T, topk, 2 * kv_fp4.shape[2]), dtype=torch.int16,
                                    device=dev)
        ws = xk_indexer_topk_workspace_size(B * T, K, topk)
        self.workspace = torch.empty(ws, dtype=torch.uint8, device=dev) if ws else None

    def run_logits(self, stream=None):
        return xk_indexer_logits(self.q, self.k, self.w, self.limit, self.q_scale, self.k_scale,
                                 out=self.logits, stream=stream)

    def run_topk(self, stream=None):
        return xk_indexer_topk(self.logits, self.topk, self.limit, out=self.idx,
                               workspace=self.workspace, stream=stream)

    def run_gather(self, sel_pos=None, stream=None):
        return xk_mxfp4_paged_gather(self.kv_fp4, self.kv_scale, self.block_table,
                                     self.idx if sel_pos is None else sel_pos, self.row_seq,
                                     out=self.gathered, stream=stream)

    def __call__(self, stream=None):
        self.run_logits(stream)
        self.run_topk(stream)
        self.run_gather(stream=stream)
        return self.logits, self.idx, self.gathered
