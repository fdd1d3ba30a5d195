"""One decode step of one sparse MLA layer on device tensors: indexer ->
top-k -> split-KV decode -> LSE merge, four library calls on one stream.

This module only allocates the step's buffers and sequences the calls."""
from dataclasses import dataclass
from typing import Optional

import torch

from . import (dsa_indexer_scores, dsa_indexer_scores_mq, lse_merge, mla_paged_decode, mq_expand_requests,
               topk_select, topk_workspace_bytes)


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
# "balanced": one split length for the whole batch (balanced_splits), so a
# ragged dense batch's long requests take more splits than its short ones.
# Measured on the box: c4 (128 requests) runs 201 µs per step with one split
# (256 workgroups, one round) against 224 with two; c2 is best at 4 and c5 at
# 8 of {2, 4, 8} and {4, 8, 16}.
DEFAULT_SPLITS = {"c1": 1, "c2": "balanced", "c3": 2, "c3f": 2, "c4": 1, "c5": 8}


def _busy_per_xcd(lens, c, num_splits, n_hg, xcds=8):
    """Workgroups with work per XCD when a fixed split length c is used: the
    decode kernels' order for that case (decode_ws.h, wg_coord): pairs
    split-major with the requests of split s rotated by s, dealt to the XCDs
    round-robin, a pair's n_hg workgroups on one XCD."""
    B = len(lens)
    pairs = B * num_splits
    full = pairs // xcds
    busy = [0] * xcds
    for p in range(pairs):
        s = p // B
        b = (p - s % B + B) % B
        if s * c < lens[b]:
            if p < full * xcds:
                busy[p % xcds] += n_hg
            else:  # the last, partial round: ids in order, dealt round-robin
                for hg in range(n_hg):
                    busy[(full * xcds * n_hg + (p - full * xcds) * n_hg + hg) % xcds] += 1
    return busy


def balanced_splits(lens, n_heads, cus=256, heads_per_group=64, tile=32, max_splits=64, min_tokens=512, xcds=8):
    """(num_splits, split_tokens) for a ragged dense batch: one split length c
    for every request, so that a long request takes more splits than a short
    one and every workgroup gets about the same work whatever the length mix.
    c is the smallest multiple of `tile`, and at least min_tokens (every
    workgroup pays a fixed start-up of several microseconds), for which no
    XCD gets more workgroups with work than it has compute units (cus / xcds;
    one per (request, split) pair and group of heads_per_group heads): the
    whole batch then runs in one round.  `lens` are the host-side context
    lengths (a serving loop's scheduler knows them)."""
    lens = [max(0, int(x)) for x in lens]
    if not lens or max(lens) == 0:
        return 1, 0
    n_hg = -(-n_heads // heads_per_group)
    target = max(1, cus // n_hg)
    c = max(min_tokens, tile, -(-max(1, sum(lens) // target) // tile) * tile)
    c = -(-c // tile) * tile
    while c < max(lens):
        S = max(1, max(-(-L // c) for L in lens))
        if S <= max_splits and max(_busy_per_xcd(lens, c, S, n_hg, xcds)) <= cus // xcds:
            break
        c += tile
    return max(1, min(max_splits, max(-(-L // c) for L in lens))), c


def default_splits(name, lens, n_heads, override=0):
    """(num_splits, split_tokens) of a workload as timed: `override` splits of
    equal count when given, else DEFAULT_SPLITS (balanced_splits for
    "balanced")."""
    if override:
        return int(override), 0
    d = DEFAULT_SPLITS.get(name, 1)
    return balanced_splits(lens, n_heads) if d == "balanced" else (int(d), 0)


class DecodeStep:
    """Holds the step's output and scratch buffers for a fixed batch shape."""

    def __init__(self, batch: DeviceBatch, num_splits: int = 1, split_tokens: int = 0):
        dev = batch.q.device
        B, H, _ = batch.q.shape
        self.batch = batch
        self.num_splits = num_splits
        self.split_tokens = split_tokens
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
                         self.status, stream, split_tokens=self.split_tokens)

    def merge(self, stream=None):
        if self.num_splits > 1:
            lse_merge(self.o_part, self.lse_part, self.o, self.lse, stream)

    def run(self, stream=None):
        if self.sparse:
            self.indexer(stream)
            self.select(stream)
        self.attend(stream)
        self.merge(stream)


class MultiQueryStep:
    """A verification step over n_q new tokens per request (already in the
    cache): query i of request b attends causally, to the tokens before
    position L_b - n_q + i + 1, with its own indexer scores and top-k.

    q [B, n_q, H, D], q_idx [B, n_q, H_I, d_I], w [B, n_q, H_I] on the device;
    `batch` supplies the pools, block table and lengths of the B requests.
    One mq_expand_requests call builds the expanded batch (B * n_q requests);
    the indexer scores both queries per key read when n_q is 2
    (dsa_indexer_scores_mq on the real requests), else runs on the expanded
    batch; top-k, decode and merge run on the expanded batch.  Outputs o [B, n_q, H, d_c],
    lse [B, n_q, H], idx [B, n_q, k] and status [B, n_q] are views of the
    expanded step's buffers."""

    def __init__(self, batch: DeviceBatch, q, q_idx, w, num_splits: int = 1):
        B, n_q = q.shape[0], q.shape[1]
        dev = q.device
        self.B, self.n_q = B, n_q
        self.real_bt, self.real_lens = batch.block_table, batch.lens
        self.bt = torch.empty(B * n_q, batch.block_table.shape[1], dtype=torch.int32, device=dev)
        self.lens = torch.empty(B * n_q, dtype=torch.int32, device=dev)
        ex = DeviceBatch(q=q.reshape(B * n_q, *q.shape[2:]), kv=batch.kv, kv_scale=batch.kv_scale,
                         block_table=self.bt, lens=self.lens, max_len=batch.max_len,
                         score_stride=batch.score_stride, d_latent=batch.d_latent, sm_scale=batch.sm_scale,
                         topk=batch.topk, q_idx=q_idx.reshape(B * n_q, *q_idx.shape[2:]),
                         w=w.reshape(B * n_q, w.shape[2]), k_idx=batch.k_idx, k_idx_scale=batch.k_idx_scale)
        self.step = DecodeStep(ex, num_splits=num_splits)
        self.real = batch
        self.q_idx_mq, self.w_mq = q_idx, w
        H_I = q_idx.shape[2]
        self.two_query_indexer = batch.topk > 0 and n_q == 2 and H_I in (16, 32, 64) and q_idx.dtype == torch.bfloat16

    def expand(self, stream=None):
        mq_expand_requests(self.real_bt, self.real_lens, self.n_q, self.bt, self.lens, stream)

    def indexer(self, stream=None):
        if self.two_query_indexer:
            r = self.real
            dsa_indexer_scores_mq(self.q_idx_mq, self.w_mq, r.k_idx, r.k_idx_scale, r.block_table, r.lens, r.max_len,
                                  self.step.scores, self.step.status, stream)
        else:
            self.step.indexer(stream)

    def run(self, stream=None):
        self.expand(stream)
        if self.step.sparse:
            self.indexer(stream)
            self.step.select(stream)
        self.step.attend(stream)
        self.step.merge(stream)

    def _view(self, t):
        return t.reshape(self.B, self.n_q, *t.shape[1:])

    @property
    def o(self):
        return self._view(self.step.o)

    @property
    def lse(self):
        return self._view(self.step.lse)

    @property
    def idx(self):
        return self._view(self.step.idx)

    @property
    def scores(self):
        return self._view(self.step.scores)

    @property
    def status(self):
        return self._view(self.step.status)


class PrefillChunkStep:
    """Attention of a prefill chunk: n_q new tokens per request (already in
    the cache, at positions L - n_q .. L - 1), each attending densely and
    causally to the tokens up to itself, computed block by block: the context
    of every query is cut into num_blocks KV splits, each giving a partial
    (o, lse), and the partials are merged with the online-softmax algebra
    (the blockwise ring-attention structure on one GPU).

    q [B, n_q, H, D] on the device; `batch` supplies the latent pool, block
    table and lengths.  Outputs o [B, n_q, H, d_c], lse [B, n_q, H] and
    status [B, n_q]."""

    def __init__(self, batch: DeviceBatch, q, num_blocks: int = 1):
        B, n_q = q.shape[0], q.shape[1]
        dev = q.device
        self.B, self.n_q = B, n_q
        self.real_bt, self.real_lens = batch.block_table, batch.lens
        self.bt = torch.empty(B * n_q, batch.block_table.shape[1], dtype=torch.int32, device=dev)
        self.lens = torch.empty(B * n_q, dtype=torch.int32, device=dev)
        ex = DeviceBatch(q=q.reshape(B * n_q, *q.shape[2:]), kv=batch.kv, kv_scale=batch.kv_scale,
                         block_table=self.bt, lens=self.lens, max_len=batch.max_len,
                         score_stride=batch.score_stride, d_latent=batch.d_latent, sm_scale=batch.sm_scale, topk=0)
        self.step = DecodeStep(ex, num_splits=num_blocks)

    def run(self, stream=None):
        mq_expand_requests(self.real_bt, self.real_lens, self.n_q, self.bt, self.lens, stream)
        self.step.attend(stream)
        self.step.merge(stream)

    def _view(self, t):
        return t.reshape(self.B, self.n_q, *t.shape[1:])

    @property
    def o(self):
        return self._view(self.step.o)

    @property
    def lse(self):
        return self._view(self.step.lse)

    @property
    def status(self):
        return self._view(self.step.status)
