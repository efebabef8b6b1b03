"""Host-side view of the paged cache layout that libkvlr reads and writes.

Physical arrays have shape [num_phys_pages, H_kv, R / CH, P, CH]: a chunk is
16 bytes of elements (8 bf16 or 4 f32), or 8 bytes for 8-bit latents (8 FP8
E4M3 values); for each KV head, the P tokens of one chunk column are
contiguous. Logical page j of a sequence lives in physical
page page_table[b, j]. These helpers only move data (staging a prefix into
pages, reading pages back); they compute nothing.
"""

from __future__ import annotations

import torch

CHUNK_BYTES = 16


def chunk_elems(dtype: torch.dtype) -> int:
    es = torch.empty(0, dtype=dtype).element_size()
    return 8 if es == 1 else CHUNK_BYTES // es


def _bytes(t: torch.Tensor) -> torch.Tensor:
    """8-bit tensors are moved as bytes (torch has no indexed copies for them)."""
    return t.view(torch.uint8) if t.element_size() == 1 else t


def alloc_pages(num_phys: int, num_kv_heads: int, width: int, page_size: int, dtype: torch.dtype,
                device, fill: float | None = 0.0) -> torch.Tensor:
    ch = chunk_elems(dtype)
    if width % ch:
        raise ValueError(f"width {width} is not a multiple of {ch}")
    shape = (num_phys, num_kv_heads, width // ch, page_size, ch)
    if fill is None:
        return torch.empty(shape, dtype=dtype, device=device)
    return torch.full(shape, fill, dtype=dtype, device=device)


def pack_sequence(phys: torch.Tensor, page_ids: torch.Tensor, rows: torch.Tensor,
                  tail_fill: float = 0.0) -> None:
    """Write logical tokens 0 .. L-1 of one sequence, rows [H, L, R], into its pages.

    page_ids: the sequence's physical page ids (logical order), at least ceil(L / P).
    Slots past L on the last page get tail_fill.
    """
    n_pages_total, H, nch, P, ch = phys.shape
    Hr, L, R = rows.shape
    if Hr != H or R != nch * ch:
        raise ValueError("rows do not match the page array")
    if L == 0:
        return
    n_pg = -(-L // P)
    x = torch.full((H, n_pg * P, R), tail_fill, dtype=phys.dtype, device=phys.device)
    x[:, :L] = rows.to(device=phys.device, dtype=phys.dtype)
    x = x.view(H, n_pg, P, nch, ch).permute(1, 0, 3, 2, 4).contiguous()
    idx = page_ids[:n_pg].to(device=phys.device, dtype=torch.long)
    _bytes(phys).index_copy_(0, idx, _bytes(x))


def unpack_sequence(phys: torch.Tensor, page_ids: torch.Tensor, L: int, start: int = 0) -> torch.Tensor:
    """Read logical tokens start .. L-1 of one sequence back as rows [H, L - start, R]."""
    n_pages_total, H, nch, P, ch = phys.shape
    if L <= start:
        return phys.new_zeros((H, 0, nch * ch))
    n_pg = -(-L // P)
    idx = page_ids[:n_pg].to(device=phys.device, dtype=torch.long)
    x = _bytes(phys).index_select(0, idx).view(phys.dtype)  # [n_pg, H, nch, P, ch]
    x = x.permute(1, 0, 3, 2, 4).reshape(H, n_pg * P, nch * ch)
    return x[:, start:L]
