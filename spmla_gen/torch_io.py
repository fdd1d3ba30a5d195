"""Move generator inputs into torch tensors (host or device).

bf16 bit patterns (uint16) become torch.bfloat16 views, FP8 codes (uint8)
become torch.float8_e4m3fn views; nothing is rounded or recomputed."""
import numpy as np
import torch


def tensor(a, device, fp8=False):
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    elif a.dtype == np.uint8 and fp8:
        t = t.view(torch.float8_e4m3fn)
    return t.to(device) if device is not None else t


def device_batch(inp, device="cuda"):
    """Generator Inputs -> sparse_paged_mla_amd.step.DeviceBatch."""
    from sparse_paged_mla_amd.step import DeviceBatch
    cfg = inp.cfg
    return DeviceBatch(
        q=tensor(inp.q, device), kv=tensor(inp.kv, device, fp8=True), kv_scale=tensor(inp.kv_scale, device),
        block_table=tensor(inp.block_table, device), lens=tensor(inp.lens, device), max_len=inp.max_len,
        score_stride=inp.score_stride, d_latent=cfg.d_latent, sm_scale=cfg.softmax_scale,
        topk=0 if cfg.dense else cfg.topk,
        q_idx=tensor(inp.q_idx, device), w=tensor(inp.w, device), k_idx=tensor(inp.k_idx, device, fp8=True),
        k_idx_scale=tensor(inp.k_idx_scale, device))
