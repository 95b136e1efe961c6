"""Helpers for the GPU parity tests: numpy bf16 bits <-> torch device tensors."""

import numpy as np


def torch_mod():
    import torch
    return torch


def to_dev(bits):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda")


def bits_of(t):
    return t.view(torch_mod().int16).cpu().numpy().view(np.uint16)


def bytes_to_dev(a):
    return torch_mod().from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def f32_dev(v):
    return torch_mod().tensor([float(v)], dtype=torch_mod().float32, device="cuda")


def rel_frobenius(y_bits, ref_bits):
    from oracle.formats import bf16_bits_to_f32
    y = bf16_bits_to_f32(y_bits).astype(np.float64)
    r = bf16_bits_to_f32(ref_bits).astype(np.float64)
    den = np.linalg.norm(r)
    return float(np.linalg.norm(y - r) / den) if den > 0 else float(np.linalg.norm(y))


def ulp_diff(y_bits, ref_bits):
    """|difference| in bf16 units of last place (same-sign values; zeros of either sign equal)."""
    a = y_bits.astype(np.int32)
    b = ref_bits.astype(np.int32)
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(a - b)


def stratified_rows(M, tile=256, block=32):
    """Rows to compare at full size: one in every `tile`-row band of the
    output (so every tile row of a 256x256-tiled GEMM, every band of K-split
    tail tiles and every workgroup of the XCD-ordered grid is touched), the
    32-row MFMA block inside the band and the row inside that block rotating
    from band to band, plus the first and last rows."""
    bands = -(-M // tile)
    rows = [b * tile + block * (b % (tile // block)) + (7 * b + 3) % block for b in range(bands)]
    return np.unique(np.clip(np.array(rows + [0, M - 1]), 0, M - 1))
