"""Test helper: 16-token K/V pages built lane by lane.

Written from the attention kernel's point of view (lane l = 16 g + c reads its
16-byte chunk h at byte 1024 h + 16 l), independently of the generator's
tensor permutes and of the oracle's per-element offset formulas, so that a
test comparing either of them against these pages checks the layout itself.
"""
import numpy as np


def k_pages(vals: np.ndarray) -> np.ndarray:
    """vals: element bytes [n, 16 key, 128 dim, e] -> pages [n, 2048 e].
    Chunk h of lane (g, c): key c, dims 32 g + (16/e) h ... (16/e) consecutive dims."""
    n, _, _, e = vals.shape
    dpc = 16 // e
    out = np.zeros((n, 2048 * e), dtype=np.uint8)
    for h in range(32 // dpc):
        for g in range(4):
            for c in range(16):
                lane = 16 * g + c
                dims = 32 * g + dpc * h + np.arange(dpc)
                out[:, 1024 * h + 16 * lane: 1024 * h + 16 * lane + 16] = vals[:, c, dims, :].reshape(n, 16)
    return out


def v_pages(vals: np.ndarray) -> np.ndarray:
    """vals: element bytes [n, 16 key, 128 dim, e] -> pages [n, 2048 e].
    Chunk h of lane (g, c): for the dim tiles dt = (4/e) h + q, keys 4 g .. 4 g + 3
    of dim 16 dt + c."""
    n, _, _, e = vals.shape
    tpc = 4 // e
    out = np.zeros((n, 2048 * e), dtype=np.uint8)
    for h in range(8 // tpc):
        for g in range(4):
            for c in range(16):
                lane = 16 * g + c
                pieces = []
                for q in range(tpc):
                    dt = tpc * h + q
                    pieces.append(vals[:, 4 * g: 4 * g + 4, 16 * dt + c, :].reshape(n, 4 * e))
                out[:, 1024 * h + 16 * lane: 1024 * h + 16 * lane + 16] = np.concatenate(pieces, axis=1)
    return out


def read_back(pages: np.ndarray, e: int, which: str) -> np.ndarray:
    """Inverse of k_pages / v_pages: pages [n, 2048 e] -> element bytes [n, 16, 128, e]."""
    probe = np.arange(16 * 128 * e, dtype=np.int64).reshape(1, 16, 128, e)
    # build the page with logical byte indices as values (as int64: run the
    # builders on every byte position via a uint8 split of the index)
    pos = np.zeros(2048 * e, dtype=np.int64)
    for shift in (0, 8, 16):
        plane = ((probe >> shift) & 0xFF).astype(np.uint8)
        built = (k_pages if which == "k" else v_pages)(plane)[0].astype(np.int64)
        pos |= built << shift
    logical = np.empty_like(pages)
    logical[:, pos] = pages
    return logical.reshape(pages.shape[0], 16, 128, e)
