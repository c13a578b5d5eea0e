"""Test-side helpers for the GPU parity tests: moving caches between the
oracle's logical layout and the library's paged layout, and building models.

The paged layout (include/cad.h): ``k [cache][block][Hkv][16][hd]`` and
``v [cache][block][Hkv][hd][16]``; token t of sequence b sits in block
``table[b][t // 16]`` at slot ``t % 16``.
"""
import numpy as np
import torch

import verify_forward_amd as cad

BLK = cad.CAD_KV_BLOCK


def write_prefix(kv: cad.KVCache, k_log: torch.Tensor, v_log: torch.Tensor, seq: int = 0):
    """Copy logical ``[cache][Hkv][L][hd]`` K/V into sequence ``seq`` of a paged cache."""
    CL, H, L, hd = k_log.shape
    table = kv.block_table.view(-1, kv.max_blocks_per_seq)[seq].long()
    nb = (L + BLK - 1) // BLK
    pad = nb * BLK - L
    kp = torch.nn.functional.pad(k_log, (0, 0, 0, pad)).view(CL, H, nb, BLK, hd).permute(0, 2, 1, 3, 4)
    vp = torch.nn.functional.pad(v_log, (0, 0, 0, pad)).view(CL, H, nb, BLK, hd).permute(0, 2, 1, 4, 3)
    blocks = table[:nb].to(kv.k.device)
    # the last block may be partial: write only its valid slots
    full = L // BLK
    if full:
        kv.k[:, blocks[:full]] = kp[:, :full].to(kv.k.dtype)
        kv.v[:, blocks[:full]] = vp[:, :full].to(kv.v.dtype)
    if pad:
        r = L - full * BLK
        b = int(blocks[full])
        kv.k[:, b, :, :r] = kp[:, full, :, :r].to(kv.k.dtype)
        kv.v[:, b, :, :, :r] = vp[:, full, :, :, :r].to(kv.v.dtype)


def read_seq(kv: cad.KVCache, n_tokens: int, seq: int = 0):
    """Logical ``[cache][Hkv][n][hd]`` float64 numpy copies of a sequence's K/V."""
    table = kv.block_table.view(-1, kv.max_blocks_per_seq)[seq].long()
    nb = (n_tokens + BLK - 1) // BLK
    blocks = table[:nb].to(kv.k.device)
    k = kv.k[:, blocks].permute(0, 2, 1, 3, 4).reshape(kv.k.shape[0], kv.k.shape[2], nb * BLK, -1)
    v = kv.v[:, blocks].permute(0, 2, 1, 4, 3).reshape(kv.v.shape[0], kv.v.shape[2], nb * BLK, -1)
    f = lambda t: t[:, :, :n_tokens].to(torch.float64).cpu().numpy()
    return f(k), f(v)


def tensors_i32(a, device="cuda"):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=device)


def outputs(N: int, vocab: int, n_seq: int = 1, device="cuda"):
    return dict(argmax=torch.full((N,), -7, dtype=torch.int32, device=device),
                accepted=torch.full((n_seq,), -7, dtype=torch.int32, device=device),
                logits=torch.empty((N, vocab), dtype=torch.float32, device=device),
                status=torch.zeros(1, dtype=torch.int32, device=device))
