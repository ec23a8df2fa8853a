"""Pins of the oracle's tiled scale order (the arrangement the C header states
under moe_layout), checked against what the arrangement is for rather than its
own formula: it is a bijection on every row, it leaves a partial trailing
window in place, and in a full window the 16-byte word of piece g holds piece
g of steps 0..7 in step order (a row whose pairs name their own (step, piece)
is rearranged and read back word by word)."""
import numpy as np

from oracle import formats as F


def test_tiled_order_is_a_bijection_that_keeps_the_tail():
    for nc in (4, 16, 32, 36, 64, 96, 100, 128):
        pos = F.tiled_scale_order(nc)
        assert sorted(pos.tolist()) == list(range(nc))
        full = nc // 32 * 32
        assert pos[full:].tolist() == list(range(full, nc))


def test_tiled_window_words_hold_one_piece_of_each_step():
    nc = 96 + 8                                      # three full windows and a partial one
    row = np.zeros(2 * nc, np.uint8)
    for c in range(nc):                              # pair c names its window, step and piece
        w, cw = divmod(c, 32)
        row[2 * c] = 16 * w + cw // 4                # window and step
        row[2 * c + 1] = cw % 4                      # piece
    t = F.tiled_scales(row[None, :])[0]
    for w in range(3):
        for g in range(4):
            word = t[64 * w + 16 * g: 64 * w + 16 * g + 16]
            assert word[1::2].tolist() == [g] * 8                        # one piece ...
            assert word[0::2].tolist() == [16 * w + i for i in range(8)]  # ... steps 0..7 in order
    assert np.array_equal(t[192:], row[192:])        # the partial window as it was


def test_tiled_scales_is_a_pure_rearrangement():
    rng = np.random.default_rng(71)
    s = rng.integers(0, 256, size=(3, 5, 2 * 72), dtype=np.uint8)
    t = F.tiled_scales(s)
    pos = F.tiled_scale_order(72)                    # canonical pair c sits at pos[c]
    back = t.reshape(3, 5, 72, 2)[:, :, pos, :].reshape(s.shape)
    assert np.array_equal(back, s)
    assert np.array_equal(np.sort(t, axis=-1), np.sort(s, axis=-1))
