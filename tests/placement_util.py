"""Check of a placed KV buffer (shared by the CPU and GPU exchange tests)."""
import numpy as np

BLOCK = 128          # KV rows per block of the placement's zero fill, counted from kv_lo


def check_placement(buf, want, need, sentinel, tag):
    """Rows a query may attend hold the global rows; the other rows of every
    128-row block (from kv_lo) holding such a row are zero; the rest are
    untouched (still `sentinel`)."""
    n = buf.shape[0]
    blk = np.zeros(n, dtype=bool)
    for b in np.unique(np.nonzero(need)[0] // BLOCK):
        blk[b * BLOCK:(b + 1) * BLOCK] = True
    assert np.array_equal(buf[need], want[need]), f"{tag}: needed rows"
    assert np.all(buf[blk & ~need] == 0), f"{tag}: block rows not zero"
    assert np.all(buf[~blk] == sentinel), f"{tag}: rows outside the blocks written"
