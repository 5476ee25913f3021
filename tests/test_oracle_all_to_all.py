"""Pins for the oracle's all-to-all + reduce (every rank's share on one host).

The index map is checked by closed forms that a transposed or shifted map
breaks, by exactness of the grand total, and by locality.
"""

import numpy as np
import pytest

import workloads
from oracle.decode import GROUP_SIZE
from oracle.reduce import all_shares, all_to_all, reduce_scatter_share


@pytest.mark.parametrize("w", [2, 4, 8])
def test_block_codes_closed_form(w):
    """Rank r's row block k holds INT8 code r*W + k everywhere, unit scales:
    share j is sum_r (r*W + j) = W*j + W*W*(W-1)/2 in every element. The
    transposed map (block r of rank j) would give W*W*j + W*(W-1)/2."""
    rows, h = 3, 256
    xs = []
    for r in range(w):
        x = np.concatenate([np.full((rows, h), r * w + k, dtype=np.uint8) for k in range(w)])
        xs.append(x)
    ss = [np.ones((w * rows, h // 128), dtype=np.float32) for _ in range(w)]
    outs = all_shares(xs, ss, "int8", "f32_group128", "f32")
    assert len(outs) == w
    for j, o in enumerate(outs):
        assert o.shape == (rows, h)
        assert np.all(o == np.float32(w * j + w * w * (w - 1) // 2)), j


def test_grand_total_is_exact():
    """INT8 with power-of-two scales: every product and sum is exact, so the
    sum of all shares' outputs equals the sum of every rank's whole input."""
    w, rows, h = 4, 5, 1024
    rng = np.random.default_rng(8)
    xs = [rng.integers(-127, 128, size=(w * rows, h), dtype=np.int8).view(np.uint8) for _ in range(w)]
    ks = [rng.integers(-10, -4, size=(w * rows, h // 128)) for _ in range(w)]
    ss = [np.ldexp(np.float32(1.0), k).astype(np.float32) for k in ks]
    outs = all_shares(xs, ss, "int8", "f32_group128", "f32")
    got = sum(int(v) for o in outs for v in (o.astype(np.float64) * 2**10).astype(np.int64).ravel())
    want = 0
    for x, k in zip(xs, ks):
        want += int(np.sum(x.view(np.int8).astype(np.int64) * (2 ** (np.repeat(k, 128, axis=1) + 10)).astype(np.int64)))
    assert got == want


def test_share_depends_only_on_its_row_block():
    wl = workloads.WORKLOADS["w8_bs16384_h8192_mx_e4m3_bf16"].with_(bs=4 * 3, world_size=4, h=1024)
    xs, ss = workloads.generate_full(wl)
    base = all_shares(xs, ss, wl.x_format, wl.scale_layout, "f32")
    xs2 = [x.copy() for x in xs]
    # change rank 2's row 7 (block 7 // 3 = 2), column 100
    xs2[2][7, 100] ^= 0x08
    after = all_shares(xs2, ss, wl.x_format, wl.scale_layout, "f32")
    for j in range(4):
        d = base[j].view(np.uint32) != after[j].view(np.uint32)
        if j == 2:
            assert d[1, 100] and d.sum() == 1
        else:
            assert not d.any()


def test_received_slices_are_in_rank_order():
    w, rows, h = 4, 2, 128
    xs = [np.full((w * rows, h), r, dtype=np.uint8) for r in range(w)]
    ss = [np.zeros((w * rows, h // 128), dtype=np.float32) + r for r in range(w)]
    for j, (rx, rs) in enumerate(all_to_all(xs, ss)):
        assert [int(x[0, 0]) for x in rx] == list(range(w))
        assert [float(s[0, 0]) for s in rs] == list(range(w))


def test_single_block_equals_share():
    """With the all-to-all done by hand, the result is reduce_scatter_share."""
    wl = workloads.WORKLOADS["w8_bs65536_h5120_mx_e5m2_f32"].with_(bs=8 * 2, h=1024)
    xs, ss = workloads.generate_full(wl)
    outs = all_shares(xs, ss, wl.x_format, wl.scale_layout, wl.out_dtype)
    g = GROUP_SIZE[wl.scale_layout]
    assert ss[0].shape == (wl.bs, wl.h // g)
    for j in range(8):
        ref = reduce_scatter_share([x[2 * j:2 * j + 2] for x in xs], [s[2 * j:2 * j + 2] for s in ss],
                                   wl.x_format, wl.scale_layout, wl.out_dtype)
        assert np.array_equal(outs[j].view(np.uint32), ref.view(np.uint32))
