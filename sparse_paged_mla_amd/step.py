"""One decode step of one sparse MLA layer on device tensors: indexer ->
top-k -> split-KV decode -> LSE merge, four library calls on one stream.

This module only allocates the step's buffers and sequences the calls."""
from dataclasses import dataclass
from typing import Optional

import torch

from . import (dsa_indexer_scores, lse_merge, mla_paged_decode, topk_select, topk_workspace_bytes)


@dataclass
class DeviceBatch:
    """Device-resident inputs of one step (see include/sparse_mla.h for layouts)."""
    q: torch.Tensor               # [B, H, D] bf16 / fp32
    kv: torch.Tensor              # [num_pages, P, D] bf16 / fp32 / float8_e4m3fn
    kv_scale: Optional[torch.Tensor]
    block_table: torch.Tensor     # int32 [B, bt_stride]
    lens: torch.Tensor            # int32 [B]
    max_len: int
    score_stride: int
    d_latent: int
    sm_scale: float
    topk: int                     # 0: dense attention (no indexer)
    q_idx: Optional[torch.Tensor] = None
    w: Optional[torch.Tensor] = None
    k_idx: Optional[torch.Tensor] = None
    k_idx_scale: Optional[torch.Tensor] = None


# KV splits per workload as timed: enough (request, split, head group)
# workgroups to fill 256 compute units without splitting short token lists.
DEFAULT_SPLITS = {"c1": 1, "c2": 4, "c3": 2, "c3f": 2, "c4": 2, "c5": 8}


class DecodeStep:
    """Holds the step's output and scratch buffers for a fixed batch shape."""

    def __init__(self, batch: DeviceBatch, num_splits: int = 1):
        dev = batch.q.device
        B, H, _ = batch.q.shape
        self.batch = batch
        self.num_splits = num_splits
        self.sparse = batch.topk > 0
        self.status = torch.zeros(B, dtype=torch.int32, device=dev)
        if self.sparse:
            self.scores = torch.empty(B, batch.score_stride, dtype=torch.float32, device=dev)
            self.idx = torch.empty(B, batch.topk, dtype=torch.int32, device=dev)
            ws = topk_workspace_bytes(B, batch.max_len, batch.topk)
            self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.o_part = torch.empty(B, num_splits, H, batch.d_latent, dtype=torch.float32, device=dev)
        self.lse_part = torch.empty(B, num_splits, H, dtype=torch.float32, device=dev)
        if num_splits > 1:
            self.o = torch.empty(B, H, batch.d_latent, dtype=torch.float32, device=dev)
            self.lse = torch.empty(B, H, dtype=torch.float32, device=dev)
        else:
            self.o = self.o_part[:, 0]
            self.lse = self.lse_part[:, 0]

    def indexer(self, stream=None):
        b = self.batch
        dsa_indexer_scores(b.q_idx, b.w, b.k_idx, b.k_idx_scale, b.block_table, b.lens, b.max_len, self.scores,
                           self.status, stream)

    def select(self, stream=None):
        b = self.batch
        topk_select(self.scores, b.lens, b.max_len, b.topk, self.idx, self.workspace, self.status, stream)

    def attend(self, stream=None):
        b = self.batch
        mla_paged_decode(b.q, b.kv, b.kv_scale, b.block_table, b.lens, b.max_len,
                         self.idx if self.sparse else None, b.d_latent, b.sm_scale, self.o_part, self.lse_part,
                         self.status, stream)

    def merge(self, stream=None):
        if self.num_splits > 1:
            lse_merge(self.o_part, self.lse_part, self.o, self.lse, stream)

    def run(self, stream=None):
        if self.sparse:
            self.indexer(stream)
            self.select(stream)
        self.attend(stream)
        self.merge(stream)
