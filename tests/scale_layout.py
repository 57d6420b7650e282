"""Host-side permutations between the oracle's plain scale layout
[rows][K/32] and the library's blocked layout [ceil(K/128)][rows][4]
(block b of a row in byte b % 4 of K group b // 4; pad bytes 0).  Pure
byte moves: no arithmetic of the method happens here."""
import numpy as np


def blocked(plain: np.ndarray) -> np.ndarray:
    """[..., rows, nb] -> [..., ceil(nb/4), rows, 4]."""
    *lead, rows, nb = plain.shape
    ng = (nb + 3) // 4
    pad = np.zeros((*lead, rows, ng * 4), np.uint8)
    pad[..., :nb] = plain
    return np.ascontiguousarray(np.swapaxes(pad.reshape(*lead, rows, ng, 4), -3, -2))


def unblocked(blk: np.ndarray, nb: int) -> np.ndarray:
    """[..., ng, rows, 4] -> [..., rows, nb]; the pad bytes must be 0."""
    *lead, ng, rows, four = blk.shape
    assert four == 4 and ng == (nb + 3) // 4, (blk.shape, nb)
    flat = np.swapaxes(blk, -3, -2).reshape(*lead, rows, ng * 4)
    assert not np.any(flat[..., nb:]), "nonzero pad bytes in the blocked scales"
    return np.ascontiguousarray(flat[..., :nb])


def blocked_shape(rows: int, K: int, batch=None):
    s = ((K // 32 + 3) // 4, rows, 4)
    return s if batch is None else (batch, *s)
