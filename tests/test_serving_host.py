"""Host logic of the serving helpers: multi-level padding levels and padded batch layout."""
import pytest

from long_context_attention_attn_amd import serving


def test_multilevel_levels():
    lv = serving.multilevel(5000, first_step=64, steps_per_level=4)
    assert lv[:4] == [64, 128, 192, 256]
    assert lv[4:8] == [320, 384, 448, 512]   # octave (256, 512] in steps of 64
    assert lv[8:12] == [640, 768, 896, 1024]  # octave (512, 1024] in steps of 128
    assert lv[-1] >= 5000 and all(a < b for a, b in zip(lv, lv[1:]))


@pytest.mark.parametrize("spl", [2, 4, 8])
def test_multilevel_padding_bound(spl):
    """Every size pads by less than max(first_step, size / steps_per_level)."""
    lv = serving.multilevel(1 << 20, first_step=64, steps_per_level=spl)
    for n in list(range(1, 3000)) + [4097, 65535, 65536, 65537, 1000000]:
        p = serving.pad_to_level(n, lv)
        assert p >= n
        assert p - n < max(64, n / spl), (n, p)


def test_pad_to_level_limits():
    with pytest.raises(ValueError):
        serving.pad_to_level(10 ** 9, serving.multilevel(1000))


def test_padded_batch_layout():
    tl = serving.multilevel(1 << 16)
    sl = [1, 2, 4, 8, 16, 32]
    T_pad, S_pad, cu = serving.padded_batch([100, 0, 37], tl, sl)
    assert T_pad == 192 and S_pad == 4
    assert cu == [0, 100, 100, 137, 192]        # real sequences, then the filler
    T_pad, S_pad, cu = serving.padded_batch([64, 64], tl, sl)
    assert (T_pad, S_pad, cu) == (128, 2, [0, 64, 128])  # exact fit: no filler
    T_pad, S_pad, cu = serving.padded_batch([5, 6, 7], tl, sl)
    assert (T_pad, S_pad) == (64, 4) and cu == [0, 5, 11, 18, 64]
    T_pad, S_pad, cu = serving.padded_batch([1] * 5, tl, sl)
    assert S_pad == 8 and cu == [0, 1, 2, 3, 4, 5, 64, 64, 64]  # filler then empties
    with pytest.raises(ValueError):
        serving.padded_batch([-1], tl, sl)
