"""Pins of the oracle's whole-block copy (oracle.copy_blocks), the checker of the
library's copy-on-write copies.

"KV Cache: capacity, layout, lifecycle", "Reference counting and tail-block COW":
when a sequence moves off a shared tail block, the old block's committed K/V and
its quantisation scales are copied into the fresh block before the new table is
published.  The expected arrays below are written out by hand from that statement
(whole blocks move; a scale that belongs to no block stays; pairs naming no block
of the pool, and a block copied onto itself, change nothing), so a copy that moves
the wrong block, skips the scales, or touches a block it should not fails here.
"""
import numpy as np

import oracle


def _pool():
    # 4 blocks; K and V pages of 2 heads x 3 values; every value distinct
    k = np.arange(24, dtype=np.int16).reshape(4, 2, 3)
    v = (100 + np.arange(24, dtype=np.int16)).reshape(4, 2, 3)
    return k, v


def test_copy_moves_whole_blocks_and_skips_bad_pairs():
    k, v = _pool()
    # (0 -> 2) copies; (1 -> 1) is a self copy; (5 -> 0) and (3 -> -1) leave the pool
    oracle.copy_blocks(k, v, None, None, [[0, 2], [1, 1], [5, 0], [3, -1]])
    want_k = np.array([[[0, 1, 2], [3, 4, 5]],
                       [[6, 7, 8], [9, 10, 11]],
                       [[0, 1, 2], [3, 4, 5]],
                       [[18, 19, 20], [21, 22, 23]]], np.int16)
    want_v = np.array([[[100, 101, 102], [103, 104, 105]],
                       [[106, 107, 108], [109, 110, 111]],
                       [[100, 101, 102], [103, 104, 105]],
                       [[118, 119, 120], [121, 122, 123]]], np.int16)
    assert np.array_equal(k, want_k)
    assert np.array_equal(v, want_v)


def test_copy_moves_block_scales():
    # one scale per (block, head): block 3's scales go to block 1, K and V apart
    k, v = _pool()
    ks = np.array([[0.5, 0.25], [1.0, 2.0], [4.0, 8.0], [16.0, 32.0]], np.float32)
    vs = -ks
    oracle.copy_blocks(k, v, ks, vs, [[3, 1]])
    assert np.array_equal(ks, np.array([[0.5, 0.25], [16.0, 32.0], [4.0, 8.0], [16.0, 32.0]],
                                        np.float32))
    assert np.array_equal(vs, -np.array([[0.5, 0.25], [16.0, 32.0], [4.0, 8.0], [16.0, 32.0]],
                                         np.float32))
    assert np.array_equal(k[1], np.array([[18, 19, 20], [21, 22, 23]], np.int16))
    assert np.array_equal(v[1], np.array([[118, 119, 120], [121, 122, 123]], np.int16))


def test_copy_moves_token_scales():
    # one scale per (block, head, token): every token's scale of the source block moves
    k, v = _pool()
    ks = np.arange(4 * 2 * 2, dtype=np.float32).reshape(4, 2, 2)
    vs = 1000 + ks
    oracle.copy_blocks(k, v, ks, vs, [[2, 0], [0, 0]])
    want = np.array([[[8, 9], [10, 11]], [[4, 5], [6, 7]], [[8, 9], [10, 11]],
                     [[12, 13], [14, 15]]], np.float32)
    assert np.array_equal(ks, want)
    assert np.array_equal(vs, 1000 + want)


def test_copy_leaves_a_pool_wide_scale_alone():
    # one scale for the whole pool belongs to no block: the caller passes none, and the
    # pool's scale array is untouched while the block itself moves
    k, v = _pool()
    tensor_scale = np.array([0.125], np.float32)
    oracle.copy_blocks(k, v, None, None, [[1, 3]])
    assert tensor_scale[0] == np.float32(0.125)
    assert np.array_equal(k[3], np.array([[6, 7, 8], [9, 10, 11]], np.int16))
    assert np.array_equal(v[3], np.array([[106, 107, 108], [109, 110, 111]], np.int16))
    assert np.array_equal(k[:3], _pool()[0][:3]) and np.array_equal(v[:3], _pool()[1][:3])


def test_copy_pairs_apply_in_order():
    # pairs are applied one after another: a block copied into a destination that a
    # later pair reads is read after the copy (the library requires distinct
    # destinations that are nobody's source; the model states the sequential meaning)
    k, v = _pool()
    oracle.copy_blocks(k, v, None, None, [[0, 1], [1, 2]])
    assert np.array_equal(k[2], np.array([[0, 1, 2], [3, 4, 5]], np.int16))
