"""Rows that drive an MX block quantiser through every (element, shared
exponent) pair it can meet: for every biased bf16 exponent field f of the block
maximum (0..254), the maximum m_f is the largest bf16 magnitude with that field,
and the other 31 elements of the blocks run through every finite bf16 pattern
whose magnitude does not exceed m_f (both signs, zeros and subnormals included).
The block maximum moves through the 32 positions and alternates in sign.

Input construction only: no quantiser arithmetic lives here."""
import numpy as np

BLOCK = 32


def exhaustive_mx_rows(hidden: int = 1024):
    """Returns (x_bits uint16 [T, hidden], max_field int [T, hidden/32]): every
    block's maximum magnitude has bf16 exponent field max_field.  Padding
    blocks at the end repeat the last field with zero fill."""
    assert hidden % BLOCK == 0
    blocks, fields = [], []
    pos = 0
    for f in range(255):
        m = np.uint16((f << 7) | 0x7F)
        mag = np.arange(0, (f + 1) << 7, dtype=np.uint32).astype(np.uint16)
        vals = np.concatenate([mag, mag | np.uint16(0x8000)])
        nblk = -(-vals.size // (BLOCK - 1))
        fill = np.zeros(nblk * (BLOCK - 1), np.uint16)
        fill[:vals.size] = vals
        fill = fill.reshape(nblk, BLOCK - 1)
        for b in range(nblk):
            p = pos % BLOCK
            mx = m | np.uint16(0x8000) if pos & 1 else m
            blocks.append(np.concatenate([fill[b, :p], [mx], fill[b, p:]]).astype(np.uint16))
            fields.append(f)
            pos += 1
    per_row = hidden // BLOCK
    pad = (-len(blocks)) % per_row
    for _ in range(pad):
        blk = np.zeros(BLOCK, np.uint16)
        blk[0] = np.uint16((254 << 7) | 0x7F)
        blocks.append(blk)
        fields.append(254)
    x = np.stack(blocks).reshape(-1, hidden)
    return x, np.array(fields, np.int64).reshape(-1, per_row)


def floor_log2_of_max(field: np.ndarray) -> np.ndarray:
    """floor(log2 m_f) for the block maxima built above: f - 127 for normal
    fields; for field 0 the maximum is 127 * 2^-133, whose floor(log2) is -127."""
    return np.where(field >= 1, field - 127, -127)
