"""Launch geometry of the 16-byte boundary transpose, modelled on the host.

transpose8_kernel (conv3d_kernels.hip) gives each thread one 8 x 8 block of
a [n][A][B] -> [n][B][A] transpose: wave w of the grid (work-groups of four
waves, rounded up) covers 8 x 8 blocks of batch w / (ga * gb), lane l the
block (8 * ga_w + l / 8, 8 * gb_w + l % 8); blocks past A or B, and the
spare waves of the last work-group, touch nothing. This model repeats that
index arithmetic with the launch's own grid and checks, for shapes that
take each load path, that every access lies inside its batch's slice and
that every output element is written exactly once (a first GPU version
without the spare-wave guard wrote one batch past the tensors).
"""
import numpy as np
import pytest


def model(n, A, B):
    ga = (A // 8 + 7) // 8
    gb = ((B + 7) // 8 + 7) // 8
    waves = n * ga * gb
    grid = (waves + 3) // 4
    written = np.zeros(n * A * B, np.int32)
    for blk in range(grid):
        for t in range(256):
            lane, wave = t & 63, blk * 4 + (t >> 6)
            nn = wave // (ga * gb)
            if nn >= n:
                continue
            rest = wave - nn * ga * gb
            a0 = ((rest // gb) * 8 + (lane >> 3)) * 8
            b0 = ((rest % gb) * 8 + (lane & 7)) * 8
            if a0 >= A or b0 >= B:
                continue
            lo, hi = nn * A * B, (nn + 1) * A * B
            cols = range(8) if (b0 + 8 <= B and B % 4 == 0) else range(min(8, B - b0))
            for c in cols:
                for r in range(8):
                    src = lo + (a0 + r) * B + b0 + c
                    dst = lo + (b0 + c) * A + a0 + r
                    assert lo <= src < hi and lo <= dst < hi, (n, A, B, blk, t)
                    written[dst] += 1
    return written


@pytest.mark.parametrize("n,A,B", [(1, 160, 44), (2, 24, 60), (1, 8, 8), (3, 16, 13),
                                   (1, 72, 117), (1, 320, 36), (2, 40, 64), (1, 16, 252),
                                   (2, 24, 105), (3, 8, 1), (1, 160, 1004)])
def test_every_element_written_once_inside_the_batch(n, A, B):
    w = model(n, A, B)
    assert w.min() == 1 and w.max() == 1
