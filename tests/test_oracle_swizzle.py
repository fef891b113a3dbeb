"""Pins of the oracle's 128x4 scale swizzle.  The pages name the layout
without its index map, so these check it against the public layout's
closed-form byte offset, its block structure and its zero padding."""
import numpy as np

import oracle as orc


def _offset(r, c, cols_pad):
    # the public layout: 512-byte blocks of 128 rows x 4 columns, row-major over
    # the blocks; inside one, 16 bytes per row modulo 32, 4 per group of 32 rows
    return ((r // 128) * (cols_pad // 4) + c // 4) * 512 + (r % 32) * 16 + ((r // 32) % 4) * 4 + c % 4


def test_every_scale_at_its_closed_form_offset():
    rng = np.random.default_rng(5)
    for rows, cols in ((1, 1), (127, 3), (128, 4), (300, 17), (513, 64)):
        s = rng.integers(1, 256, size=(rows, cols), dtype=np.uint8)
        buf = orc.swizzle_scales_128x4(s)
        cp = -(-cols // 4) * 4
        assert buf.size == -(-rows // 128) * 128 * cp
        hit = np.zeros(buf.size, dtype=bool)
        for r in range(rows):
            for c in range(cols):
                o = _offset(r, c, cp)
                assert buf[o] == s[r, c]
                hit[o] = True
        assert (buf[~hit] == 0).all()  # padding rows and columns are zero
        assert (orc.unswizzle_scales_128x4(buf, rows, cols) == s).all()


def test_first_block_pattern():
    # a 128 x 4 matrix is one 512-byte block: its first 16 bytes are columns
    # 0..3 of rows 0, 32, 64 and 96; bytes 16..31 the same for rows 1, 33, 65, 97
    s = np.arange(512, dtype=np.int64).reshape(128, 4).astype(np.uint8)
    buf = orc.swizzle_scales_128x4(s)
    assert list(buf[:16]) == [int(s[r, c]) for r in (0, 32, 64, 96) for c in range(4)]
    assert list(buf[16:32]) == [int(s[r, c]) for r in (1, 33, 65, 97) for c in range(4)]
    # the block holds every scale once
    assert sorted(buf.tolist()) == sorted(s.reshape(-1).tolist())


def test_second_column_block_follows_the_first():
    # 128 x 8: the block of columns 4..7 is the next 512 bytes, same pattern
    s = np.random.default_rng(6).integers(0, 256, size=(128, 8), dtype=np.uint8)
    buf = orc.swizzle_scales_128x4(s)
    assert (buf[:512] == orc.swizzle_scales_128x4(s[:, :4])).all()
    assert (buf[512:] == orc.swizzle_scales_128x4(s[:, 4:])).all()
