"""NaN and Inf bit patterns for the cache slots no call may read (test helper)."""

import numpy as np

POISON_BF16 = np.array([0x7FC0, 0xFFFF, 0x7F80, 0xFF80], np.uint16)  # NaN, NaN, +Inf, -Inf
POISON_F32 = np.array([0x7FC00000, 0xFFFFFFFF, 0x7F800000, 0xFF800000], np.uint32)


def poison_from(k_pages, v_pages, block_table, start, npos):
    """In place: every slot of sequence b at positions [start[b], npos[b]) gets a NaN or Inf pattern,
    K and V (only the pages of b's block-table row that cover those positions)."""
    words = POISON_BF16 if k_pages.dtype == np.uint16 else POISON_F32
    kw = k_pages.view(words.dtype)
    vw = v_pages.view(words.dtype)
    D = k_pages.shape[-1]
    pat = np.resize(words, D)
    for b in range(len(start)):
        for pos in range(int(start[b]), int(npos[b])):
            page = int(block_table[b, pos // 16])
            kw[page, :, pos % 16, :] = np.roll(pat, pos)
            vw[page, :, pos % 16, :] = np.roll(pat, pos + 1)


def bits(a):
    """Bit patterns of a storage array (NaN-safe equality)."""
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)
