"""Host-side permutations between the oracle's plain packed layout -- codes
[rows][K*bits/8], scales [rows][K/32] -- and the library's K-group-major
layout: codes [ceil(K/128)][rows][16*bits], scales [ceil(K/128)][rows][4]
(block b of a row in byte b % 4 of K group b // 4).  Inside an E2M3 group
the 24 bytes of block b are split: the first 16 at byte 16 b, the last 8 at
64 + 8 (b ^ s), s = bit 4 of the row.  Pad bytes of a partial last K group
are 0.  Pure byte moves: no
arithmetic of the method happens here."""
import numpy as np


def _to_groups(plain: np.ndarray, per_group: int) -> np.ndarray:
    *lead, rows, nbytes = plain.shape
    ng = (nbytes + per_group - 1) // per_group
    pad = np.zeros((*lead, rows, ng * per_group), np.uint8)
    pad[..., :nbytes] = plain
    return np.ascontiguousarray(np.swapaxes(pad.reshape(*lead, rows, ng, per_group), -3, -2))


def _from_groups(grouped: np.ndarray, nbytes: int, per_group: int) -> np.ndarray:
    *lead, ng, rows, pg = grouped.shape
    assert pg == per_group and ng == (nbytes + per_group - 1) // per_group, (grouped.shape, nbytes)
    flat = np.swapaxes(grouped, -3, -2).reshape(*lead, rows, ng * per_group)
    assert not np.any(flat[..., nbytes:]), "nonzero pad bytes in a partial K group"
    return np.ascontiguousarray(flat[..., :nbytes])


def blocked(plain: np.ndarray) -> np.ndarray:
    """scales [..., rows, nb] -> [..., ceil(nb/4), rows, 4]."""
    return _to_groups(plain, 4)


def unblocked(blk: np.ndarray, nb: int) -> np.ndarray:
    """scales [..., ng, rows, 4] -> [..., rows, nb]; the pad bytes must be 0."""
    return _from_groups(blk, nb, 4)


# stored byte j of an E2M3 group holds plain byte E2M3_ORDER[s][j], s = bit 4 of the row
E2M3_ORDER = [np.array([24 * b + i for b in range(4) for i in range(16)] +
                       [24 * (c ^ s) + 16 + i for c in range(4) for i in range(8)]) for s in (0, 1)]


def _swap_rows(rows: int) -> np.ndarray:
    return ((np.arange(rows) >> 4) & 1).astype(bool)


def tiled(plain: np.ndarray, bits: int) -> np.ndarray:
    """codes [..., rows, K*bits/8] -> [..., ceil(K/128), rows, 16*bits]."""
    g = _to_groups(plain, 16 * bits)
    if bits == 6:
        odd = _swap_rows(g.shape[-2])
        out = g[..., E2M3_ORDER[0]]
        out[..., odd, :] = g[..., odd, :][..., E2M3_ORDER[1]]
        g = out
    return np.ascontiguousarray(g)


def untiled(t: np.ndarray, k: int, bits: int) -> np.ndarray:
    """codes [..., ng, rows, 16*bits] -> [..., rows, k*bits/8]; pad bytes must be 0."""
    if bits == 6:
        odd = _swap_rows(t.shape[-2])
        g = np.empty_like(t)
        g[..., E2M3_ORDER[0]] = t
        sub = np.empty_like(t[..., odd, :])
        sub[..., E2M3_ORDER[1]] = t[..., odd, :]
        g[..., odd, :] = sub
        t = g
    return _from_groups(t, k * bits // 8, 16 * bits)


def blocked_shape(rows: int, K: int, batch=None):
    s = ((K // 32 + 3) // 4, rows, 4)
    return s if batch is None else (batch, *s)


def tiled_shape(rows: int, K: int, bits: int, batch=None):
    s = ((K + 127) // 128, rows, 16 * bits)
    return s if batch is None else (batch, *s)
