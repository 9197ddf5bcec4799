"""The workgroup-shape rule (vattn_launch_shape), host-only: no GPU needed.

W = n_heads * ceil(n_patches / 256) wide blocks, S = n_heads *
ceil(n_patches / 64) small blocks, C compute units:
  16 waves if 2W > C (rotary: 2W >= C); rotary: else 4 waves;
  8 waves if 2W >= C; split-key if S <= C; else 8 waves.
"""
from __future__ import annotations

import pytest

import non_causal_flash_amd as vattn

SK, W4, W8, W16 = (vattn.SHAPE_SPLIT_KEYS, vattn.SHAPE_4_WAVES, vattn.SHAPE_8_WAVES,
                   vattn.SHAPE_16_WAVES)


@pytest.mark.parametrize("h,n,d,rope,cus,shape", [
    # the five benchmark configurations on 256 CUs
    (4, 64, 64, False, 256, SK),       # 4 small blocks
    (16, 256, 64, False, 256, SK),     # 64 small blocks
    (16, 1024, 64, False, 256, SK),    # S = 256 = C: still one small block per CU
    (12, 4097, 32, False, 256, W16),   # W = 12 * 17 = 204 > 128
    (128, 4096, 64, False, 256, W16),
    # edges of the 16- and 8-wave steps
    (32, 1000, 64, False, 256, W8),    # W = 128: 2W = C, not above
    (33, 1000, 64, False, 256, W16),   # W = 132
    (20, 800, 64, False, 256, W8),     # W = 80, S = 260 > C
    (16, 1025, 64, False, 256, W8),    # W = 80, S = 272
    (64, 256, 64, False, 256, SK),     # W = 64, S = 256
    (65, 256, 64, False, 256, W8),     # S = 260
    # rotary kernels: no 8-wave or split-key step
    (16, 1024, 64, True, 256, W4),     # W = 64
    (32, 1024, 64, True, 256, W16),    # W = 128: 2W >= C
    (31, 1024, 64, True, 256, W4),
    # other CU counts (a device with more CUs, a partition with fewer)
    (12, 4097, 32, False, 304, W16),   # 2W = 408 > 304
    (16, 1024, 64, False, 304, SK),    # S = 256 <= 304
    (16, 1024, 64, False, 80, W16),    # 2W = 128 > 80
    (4, 64, 64, False, 1, W16),        # 2W = 8 > 1
    (1, 1, 1, False, 4, SK),
])
def test_shape(h, n, d, rope, cus, shape):
    assert vattn.launch_shape(h, n, d, rope, cus) == shape


def test_head_dim_does_not_change_the_shape():
    for d in (1, 17, 32, 33, 64):
        assert vattn.launch_shape(12, 4097, d, False, 256) == W16
        assert vattn.launch_shape(16, 1024, d, False, 256) == SK


@pytest.mark.parametrize("args", [(0, 64, 64, 0, 256), (4, 0, 64, 0, 256), (4, 64, 0, 0, 256),
                                  (4, 64, 65, 0, 256), (4, 64, 64, 0, 0), (-1, 64, 64, 0, 256)])
def test_invalid_sizes(args):
    assert vattn.launch_shape(*args) == -vattn.VATTN_ERR_SIZE
