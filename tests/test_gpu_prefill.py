"""GPU parity of chunked prefill (matrix cores) against the oracle.

Method: "03 | PagedAttention and the KV-cache memory system" §4 — prefill over the
paged cache with the block table; query row i of an n-token chunk sits at
a = ctx - n + i and sees keys 0..a (every key when not causal).  Tolerance as for
decode: |gpu - oracle| <= 2e-3 + 1e-2|oracle| per element, oracle in fp64 on the
same stored values.  Pools are NaN-filled (0xFF) before the library's write path
fills them, so a read of any slot outside the context fails the finiteness check.
"""
import numpy as np
import pytest

import oracle
from helpers import GpuCase, assert_close, oracle_pool, peaked, to_f64
import workloads as W

pytestmark = pytest.mark.gpu


def _run(wl, causal=True, rows=None):
    case = GpuCase(wl)
    opool = oracle_pool(wl)
    ref = oracle.paged_prefill(wl.q, wl.q_dtype, wl.cu_seqlens_q, opool, wl.block_table,
                               wl.context_lens, wl.scale, causal=causal, rows=rows)
    out = to_f64(case.prefill(causal=causal), wl.q_dtype)
    if rows is not None:
        out = out[rows]
    return assert_close(out, ref, "%s causal=%d" % (wl.name, causal))


def test_fp8_prefill_small_causal():
    print(_run(W.fp8_chunked_prefill(small=True), causal=True))


def test_fp8_prefill_small_not_causal():
    print(_run(W.fp8_chunked_prefill(small=True), causal=False))


def test_bf16_prefill_small():
    wl = W.make_prefill("bf16 KV prefill (S=3)", 21, 3, [250, 0, 64], [70, 33, 1], 32, 8, 128, 16,
                        kv_dtype="bf16")
    print(_run(wl, causal=True))


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("kv", ["fp8", "bf16", "f16"])
def test_prefill_group_sizes(G, kv):
    # chunk lengths that end mid-tile and mid-workgroup, a chunk with no cache; f16 pools
    # take f16 queries
    Hkv = 2
    wl = W.make_prefill("prefill G=%d %s" % (G, kv), 30 + G, 3, [77, 0, 130], [45, 19, 3], G * Hkv,
                        Hkv, 128, 16, kv_dtype=kv, q_dtype="f16" if kv == "f16" else "bf16")
    print(_run(wl, causal=True))


@pytest.mark.parametrize("B", [16, 32, 64])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("kv", ["fp8", "f16"])
def test_prefill_block_and_head_dim(B, D, kv):
    wl = W.make_prefill("prefill B=%d D=%d %s" % (B, D, kv), 40 + B + D, 2, [93, 200], [61, 128],
                        8, 2, D, B, kv_dtype=kv, q_dtype="f16" if kv == "f16" else "bf16")
    print(_run(wl, causal=True))


@pytest.mark.parametrize("short", [4, 2, 1, 3])
@pytest.mark.parametrize("G", [4, 2])
def test_prefill_rows_past_the_context_are_zero(short, G):
    # context_lens shorter than the chunk: rows at negative positions see no key.  A row
    # tile holds 16/G tokens; a shortfall that is not a multiple of it puts rows that see
    # nothing and rows that do in one tile (the first keys must not rescale the others)
    wl = W.make_prefill("prefill short ctx", 50, 2, [0, 40], [24, 10], 2 * G, 2, 128, 16)
    wl.context_lens = wl.context_lens.copy()
    wl.context_lens[0] = 24 - short  # chunk of 24 rows: rows 0 .. short-1 see nothing
    print(_run(wl, causal=True))


@pytest.mark.parametrize("factor", [1, 4, 8])
def test_fp8_prefill_full_sampled(factor):
    # the full chunked-prefill workload in its bench launch configuration; rows sampled
    # at the chunk edges (first, last) and inside, for every sequence; q x 4 and x 8
    # (exact) sharpen the softmax so that the relative tolerance decides
    wl = W.fp8_chunked_prefill()
    if factor != 1:
        wl = peaked(wl, factor)
    cu = wl.cu_seqlens_q
    rng = np.random.default_rng(7)
    rows = []
    for s in range(wl.num_seqs):
        a, b = int(cu[s]), int(cu[s + 1])
        rows += [a, a + 1, b - 1, b - 2] + list(rng.integers(a, b, 4))
    rows = np.array(sorted(set(rows)), np.int64)
    print(_run(wl, causal=True, rows=rows))


@pytest.mark.parametrize("kv,D", [("fp8", 128), ("bf16", 128), ("f16", 64), ("fp8", 64)])
def test_prefill_sharp_softmax(kv, D):
    # q x 32 (exact): scores spread over ~45 log2 units, so later chunks often pass a
    # row's reference by far more than the first softmax pass allows (a chunk sum above
    # 2^15), and the tile takes its scores again and the maxima path; several chunks
    # per sequence, rows that start inside a tile
    wl = W.make_prefill("prefill sharp %s D=%d" % (kv, D), 60 + D, 3, [300, 90, 0],
                        [77, 130, 64], 8, 2, D, 16, kv_dtype=kv,
                        q_dtype="f16" if kv == "f16" else "bf16")
    print(_run(peaked(wl, 32), causal=True))
