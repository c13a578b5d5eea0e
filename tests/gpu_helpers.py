"""Test-side helpers for the GPU parity tests: moving caches between the
oracle's logical layout and the library's paged layout, building models, and
masks under which the looped block's decisions have clear margins.

The paged layout (include/cad.h): ``k [cache][block][Hkv][16][hd]`` and
``v [cache][block][Hkv][hd][16]``; token t of sequence b sits in block
``table[b][t // 16]`` at slot ``t % 16``.
"""
import numpy as np
import torch

import synth
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


def read_span(kv: cad.KVCache, first: int, n: int, seq: int = 0):
    """Logical ``[cache][Hkv][n][hd]`` float64 copies of tokens
    ``first .. first + n - 1`` of a sequence (only the blocks that hold them
    are read back)."""
    table = kv.block_table.view(-1, kv.max_blocks_per_seq)[seq].long()
    b0, b1 = first // BLK, (first + n - 1) // BLK + 1
    blocks = table[b0:b1].to(kv.k.device)
    k = kv.k[:, blocks].permute(0, 2, 1, 3, 4).reshape(kv.k.shape[0], kv.k.shape[2], (b1 - b0) * BLK, -1)
    v = kv.v[:, blocks].permute(0, 2, 1, 4, 3).reshape(kv.v.shape[0], kv.v.shape[2], (b1 - b0) * BLK, -1)
    o = first - b0 * BLK
    f = lambda t: t[:, :, o:o + n].to(torch.float64).cpu().numpy()
    return f(k), f(v)


def tensors_i32(a, device="cuda"):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device=device)


def outputs(N: int, vocab: int, n_seq: int = 1, device="cuda"):
    return dict(argmax=torch.full((N,), -7, dtype=torch.int32, device=device),
                accepted=torch.full((n_seq,), -7, dtype=torch.int32, device=device),
                logits=torch.empty((N, vocab), dtype=torch.float32, device=device),
                status=torch.zeros(1, dtype=torch.int32, device=device))


def bf16_ulp(x):
    """Spacing of bfloat16 numbers at |x| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def kv_close(gpu, ref, tol):
    """Cache entries are stored in bfloat16: a GPU value matches an exact
    reference value within ``tol`` plus half a bfloat16 spacing at the
    reference (the rounding that storing any value in the cache applies)."""
    gpu, ref = np.asarray(gpu, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    excess = np.abs(gpu - ref) - (tol + 0.5 * bf16_ulp(ref))
    return float(np.max(excess)) <= 0.0, float(np.max(np.abs(gpu - ref)))


def kv_close_stored(a, b, tol):
    """Two bfloat16 caches agree within ``tol`` or one bfloat16 spacing (a
    value close to a rounding boundary may land on either neighbour)."""
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    lim = np.maximum(tol, bf16_ulp(np.maximum(np.abs(a), np.abs(b))))
    return bool(np.all(np.abs(a - b) <= lim)), float(np.max(np.abs(a - b)))


def clear_margin_mask(screen_logits, full_logits, gap):
    """A per-position mask under which every masked decision of both
    readouts has a top-2 margin of at least ``gap``, built from the oracle's
    unmasked logits.  Row k allows its screening argmax a_s; its full-depth
    argmax a_f too when the two readouts separate them by ``gap`` each way
    (rows past ``full_logits`` have no full-depth readout); and every id at
    least ``gap`` below the allowed leaders in both readouts.  The screening
    argmax is unchanged by the mask, so the survivors are too."""
    N, V = screen_logits.shape
    allowed = np.zeros((N, V), dtype=bool)
    for k in range(N):
        s = screen_logits[k]
        a_s = int(np.argmax(s))
        lead = [a_s]
        ok = s <= s[a_s] - gap
        if k < len(full_logits):
            f = full_logits[k]
            a_f = int(np.argmax(f))
            if a_f != a_s and s[a_s] - s[a_f] >= gap and f[a_f] - f[a_s] >= gap:
                lead.append(a_f)
            ok &= f <= max(f[i] for i in lead) - gap
        allowed[k] = ok
        allowed[k, lead] = True
    return synth.pack_mask(allowed)
