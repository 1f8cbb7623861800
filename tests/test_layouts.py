"""CPU checks of the host-side layout helpers the GPU tests use to read the
library's outputs, against the layouts include/vsmooth.h documents."""
import numpy as np

from gpu_util import V_TOKEN_OF_POS, v4_rows, v8_rows


def test_e4m3_v_layout_helper():
    rng = np.random.default_rng(0)
    nb, D = 2, 8
    codes = rng.integers(0, 256, size=(nb * 128, D), dtype=np.uint8)
    tiles = np.zeros((nb, D, 128), dtype=np.uint8)
    for j in range(nb):
        for p in range(128):      # row position p holds token t(p)
            tiles[j, :, p] = codes[j * 128 + V_TOKEN_OF_POS[p]]
    np.testing.assert_array_equal(v8_rows(tiles), codes)
    assert sorted(V_TOKEN_OF_POS.tolist()) == list(range(128))


def test_mxfp4_v_layout_helper():
    """Forward packing written from the header's wording: group g of channel
    d in bytes 16g..16g+15, nibble q (low first) = token 32g + 8((q%16)/4) +
    4(q/16) + q%4; scale byte g = e + 127."""
    rng = np.random.default_rng(1)
    nb, D = 3, 16
    codes = rng.integers(0, 16, size=(nb * 128, D), dtype=np.uint8)
    exps = rng.integers(-127, 128, size=(nb * 4, D), dtype=np.int32)
    tiles = np.zeros((nb, D, 64), dtype=np.uint8)
    scales = np.zeros((nb, D, 4), dtype=np.uint8)
    for j in range(nb):
        for d in range(D):
            for g in range(4):
                scales[j, d, g] = exps[4 * j + g, d] + 127
                for q in range(32):
                    tok = j * 128 + 32 * g + 8 * ((q % 16) // 4) + 4 * (q // 16) + q % 4
                    tiles[j, d, 16 * g + q // 2] |= codes[tok, d] << (4 * (q % 2))
    got_codes, got_exps = v4_rows(tiles, scales)
    np.testing.assert_array_equal(got_codes, codes)
    np.testing.assert_array_equal(got_exps, exps)
