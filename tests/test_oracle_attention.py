"""Pins of the oracle's attention against what the pages and the mathematics fix.

- "Paging does not change the attention result; the output equals contiguous
  storage" ("What is the principle of PagedAttention?" §5; "03 | ..." §4): the
  oracle's paged decode equals dense attention over the contiguous static cache
  layout [batch][seq][kv_heads][head_dim] ("vLLM notes ...", static cache),
  computed by a library routine (torch scaled_dot_product_attention, fp64, CPU,
  with its own GQA grouping).
- Closed forms: ctx = 1 gives v_0 exactly; q = 0 gives the mean of V.
- Relabelling physical block ids leaves the output bitwise unchanged.
- Online-softmax merge ("03 | ..." §4): splitting the context into any partitions
  and merging the (max, exp_sum, weighted_value) states gives the one-shot result.
- Prefill: one new token equals decode; no cached context equals textbook causal
  attention (library routine, is_causal).
- Uninitialised slots are never read ("KV Cache: ...", lifecycle invariant 6):
  NaN in spare blocks and tail slots leaves the output finite and unchanged.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import NAN_BITS, to_storage


def _values(bits, dtype, scale=None):
    """Exact float64 values of storage bits via torch's own dtypes (independent decoder)."""
    t = {"f32": None, "f16": torch.float16, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn,
         "int8": None}[dtype]
    if dtype == "f32":
        return torch.from_numpy(np.asarray(bits, np.float32)).double()
    if dtype == "int8":
        return torch.from_numpy(np.asarray(bits, np.int8).astype(np.float64))
    raw = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16 if dtype != "fp8" else np.uint8))
    return raw.view(t).double()


QUANT = ("fp8", "int8")


def _paged_case(rng, ctxs, Hq, Hkv, D, B, kv_dtype, q_dtype=None, spare=3, fill_nan=True,
                scale_mode="block"):
    """Random contiguous K/V per sequence, scattered through shuffled tables by the oracle."""
    q_dtype = q_dtype or ("bf16" if kv_dtype in QUANT else kv_dtype)
    S = len(ctxs)
    nblk_seq = [math.ceil(c / B) for c in ctxs]
    NB = sum(nblk_seq) + spare + 1
    perm = rng.permutation(NB).astype(np.int32)
    W = max(1, max(nblk_seq))
    table = np.full((S, W), perm[-1], np.int32)
    o = 0
    for s, n in enumerate(nblk_seq):
        table[s, :n] = perm[o:o + n]
        o += n
    src_dtype = "bf16" if kv_dtype in QUANT else kv_dtype
    fill = NAN_BITS[kv_dtype] if (fill_nan and kv_dtype in NAN_BITS) else None
    pool = oracle.Pool(NB, B, Hkv, D, kv_dtype, fill_bits=fill, scale_mode=scale_mode)
    if kv_dtype in QUANT:
        lo, hi = (0.002, 0.02) if kv_dtype == "fp8" else (0.01, 0.04)
        pool.k_scale = rng.uniform(lo, hi, size=pool.scale_shape()).astype(np.float32)
        pool.v_scale = rng.uniform(lo, hi, size=pool.scale_shape()).astype(np.float32)
    ks, vs = [], []
    for s, c in enumerate(ctxs):
        k = to_storage(rng.standard_normal((c, Hkv, D), dtype=np.float32), src_dtype)
        v = to_storage(rng.standard_normal((c, Hkv, D), dtype=np.float32), src_dtype)
        slots = oracle.slot_mapping(table, np.full(c, s, np.int32), np.arange(c, dtype=np.int32), B)
        oracle.kv_cache_write(pool, slots, k, v, src_dtype)
        ks.append(k)
        vs.append(v)
    q = to_storage(rng.standard_normal((S, Hq, D), dtype=np.float32), q_dtype)
    return dict(pool=pool, table=table, ctx=np.array(ctxs, np.int32), q=q, q_dtype=q_dtype,
                ks=ks, vs=vs, NB=NB)


def _contiguous_values(case, s, which):
    """float64 [ctx][Hkv][D] values a dense reference sees for sequence s: the stored
    codes (dequantised by torch's own fp8 type for fp8) read back by logical position."""
    pool, B = case["pool"], case["pool"].block_size
    c = int(case["ctx"][s])
    pos = np.arange(c)
    blk = case["table"][s, pos // B]
    arr = pool.k if which == "k" else pool.v
    bits = arr[blk, :, pos % B, :]  # [ctx][Hkv][D]
    vals = _values(bits, pool.kv_dtype)
    if pool.kv_dtype in QUANT:
        sc = pool.k_scale if which == "k" else pool.v_scale
        if pool.scale_mode == "tensor":
            per = np.broadcast_to(sc[0], (c, pool.num_kv_heads))
        elif pool.scale_mode == "token":
            per = sc[blk, :, pos % B]                            # [ctx][Hkv]
        else:
            per = sc[blk]                                        # [ctx][Hkv]
        vals = vals * torch.from_numpy(np.ascontiguousarray(per, np.float64))[:, :, None]
    return vals


def _sdpa_decode(case, scale):
    outs = []
    for s in range(len(case["ctx"])):
        q = _values(case["q"][s], case["q_dtype"])  # [Hq][D]
        c = int(case["ctx"][s])
        if c == 0:
            outs.append(torch.zeros_like(q))
            continue
        K = _contiguous_values(case, s, "k").permute(1, 0, 2)[None]  # [1][Hkv][ctx][D]
        V = _contiguous_values(case, s, "v").permute(1, 0, 2)[None]
        o = F.scaled_dot_product_attention(q[None, :, None, :], K, V, scale=scale, enable_gqa=True)
        outs.append(o[0, :, 0, :])
    return torch.stack(outs).numpy()


@pytest.mark.parametrize("kv_dtype,Hq,Hkv,D,B", [
    ("f32", 4, 2, 64, 4), ("bf16", 8, 2, 128, 16), ("f16", 4, 4, 64, 32),
    ("fp8", 8, 1, 128, 16), ("bf16", 6, 3, 64, 8)])
def test_decode_equals_dense_contiguous_sdpa(kv_dtype, Hq, Hkv, D, B):
    rng = np.random.default_rng(100 + Hq + D + B)
    case = _paged_case(rng, [1, B - 1, B, B + 1, 2 * B, 3 * B + 5, 57], Hq, Hkv, D, B, kv_dtype)
    scale = 1.0 / math.sqrt(D)
    got = oracle.paged_decode(case["q"], case["q_dtype"], case["pool"], case["table"], case["ctx"], scale)
    ref = _sdpa_decode(case, scale)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kv_dtype,mode", [("fp8", "tensor"), ("fp8", "token"),
                                           ("int8", "token"), ("int8", "block"),
                                           ("int8", "tensor")])
def test_quantised_modes_equal_dense_sdpa(kv_dtype, mode):
    # [P1 §8.1] per-tensor and per-token-head scales: each stored code times the scale
    # its (block, head, token) owns, read back by logical position, must give the
    # oracle's paged result
    rng = np.random.default_rng(300 + len(mode) + len(kv_dtype))
    B = 16
    case = _paged_case(rng, [1, B - 1, B + 1, 3 * B + 5, 57], 8, 2, 128, B, kv_dtype,
                       scale_mode=mode)
    scale = 1.0 / math.sqrt(128)
    got = oracle.paged_decode(case["q"], case["q_dtype"], case["pool"], case["table"],
                              case["ctx"], scale)
    ref = _sdpa_decode(case, scale)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_scale_modes_reduce_to_per_block():
    # the same stored values under the three layouts of the scales: a tensor scale equal
    # to every block's, and token scales constant over each block, give identical output
    rng = np.random.default_rng(301)
    B, NB, H = 16, 9, 2
    case = _paged_case(rng, [20, 45], 4, H, 64, B, "int8", spare=NB - 5)
    blk_pool = case["pool"]
    outs = []
    for mode in ("block", "tensor", "token"):
        p = oracle.Pool(blk_pool.num_blocks, B, H, 64, "int8", scale_mode=mode)
        p.k, p.v = blk_pool.k, blk_pool.v
        if mode == "block":
            p.k_scale = np.full((p.num_blocks, H), 0.03, np.float32)
        elif mode == "tensor":
            p.k_scale = np.array([0.03], np.float32)
        else:
            p.k_scale = np.full((p.num_blocks, H, B), 0.03, np.float32)
        p.v_scale = p.k_scale * 2
        outs.append(oracle.paged_decode(case["q"], case["q_dtype"], p, case["table"],
                                        case["ctx"], 0.125))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_decode_closed_forms():
    rng = np.random.default_rng(5)
    case = _paged_case(rng, [1, 9, 33], 4, 2, 64, 4, "f32")
    scale = 0.125
    got = oracle.paged_decode(case["q"], "f32", case["pool"], case["table"], case["ctx"], scale)
    # ctx = 1: the only weight is 1, the output is v_0 exactly
    v0 = case["vs"][0][0].astype(np.float64)  # [Hkv][D]
    assert np.array_equal(got[0], np.repeat(v0, 2, axis=0))
    # q = 0: every score is 0, the output is the plain mean of V
    qz = np.zeros_like(case["q"])
    got0 = oracle.paged_decode(qz, "f32", case["pool"], case["table"], case["ctx"], scale)
    for s in range(3):
        mean = case["vs"][s].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(got0[s], np.repeat(mean, 2, axis=0), rtol=0, atol=1e-14)
    # ctx = 0: zeros, lse = -inf
    case["ctx"][1] = 0
    out, lse = oracle.paged_decode(case["q"], "f32", case["pool"], case["table"], case["ctx"],
                                   scale, return_lse=True)
    assert np.array_equal(out[1], np.zeros_like(out[1])) and np.all(lse[1] == -np.inf)


def test_decode_invariant_under_block_relabelling():
    rng = np.random.default_rng(8)
    case = _paged_case(rng, [13, 40, 7, 64], 8, 2, 64, 8, "bf16")
    scale = 0.125
    a = oracle.paged_decode(case["q"], "bf16", case["pool"], case["table"], case["ctx"], scale)
    NB = case["NB"]
    pi = rng.permutation(NB)
    pool2 = oracle.Pool(NB, 8, 2, 64, "bf16")
    pool2.k[pi] = case["pool"].k
    pool2.v[pi] = case["pool"].v
    table2 = pi[case["table"]].astype(np.int32)
    b = oracle.paged_decode(case["q"], "bf16", pool2, table2, case["ctx"], scale)
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


def test_uninitialised_slots_never_read():
    ctxs = [3, 17, 30]
    c1 = _paged_case(np.random.default_rng(9), ctxs, 4, 2, 64, 8, "f16", fill_nan=True)
    c2 = _paged_case(np.random.default_rng(9), ctxs, 4, 2, 64, 8, "f16", fill_nan=False)
    a = oracle.paged_decode(c1["q"], "f16", c1["pool"], c1["table"], c1["ctx"], 0.125)
    b = oracle.paged_decode(c2["q"], "f16", c2["pool"], c2["table"], c2["ctx"], 0.125)
    assert np.isfinite(a).all()
    assert np.array_equal(a, b)


@pytest.mark.parametrize("P", [1, 3, 7, 16, 64, 1000])
def test_split_partitions_merge_to_one_shot(P):
    rng = np.random.default_rng(10 + P)
    case = _paged_case(rng, [0, 1, 15, 16, 17, 100, 333], 4, 2, 64, 16, "bf16")
    scale = 1.0 / 8
    one = oracle.paged_decode(case["q"], "bf16", case["pool"], case["table"], case["ctx"], scale)
    maxp = math.ceil(333 / P)
    po, pm, ps = oracle.decode_partials(case["q"], "bf16", case["pool"], case["table"],
                                        case["ctx"], scale, P, maxp)
    red = oracle.split_reduce(po, pm, ps, case["ctx"], P)
    np.testing.assert_allclose(red, one, rtol=1e-12, atol=1e-13)
    # single partition: identity
    if P >= 333:
        np.testing.assert_allclose(po[:, :, 0, :], one, rtol=0, atol=0)


def test_state_merge_properties():
    rng = np.random.default_rng(12)
    D = 5
    acc = lambda: rng.standard_normal(D)
    a = (1.5, 2.0, acc())
    b = (-0.25, 3.0, acc())
    empty = (-np.inf, 0.0, np.zeros(D))
    for x in (a, b):
        m, l, ac = oracle.state_merge(x, empty)
        assert (m, l) == (x[0], x[1]) and np.array_equal(ac, x[2])
        m, l, ac = oracle.state_merge(empty, x)
        assert (m, l) == (x[0], x[1]) and np.array_equal(ac, x[2])
    m, l, ac = oracle.state_merge(empty, empty)
    assert m == -np.inf and l == 0 and not ac.any()
    m1, l1, a1 = oracle.state_merge(a, b)
    m2, l2, a2 = oracle.state_merge(b, a)
    assert m1 == m2 == 1.5
    np.testing.assert_allclose([l1], [l2], rtol=1e-15)
    np.testing.assert_allclose(a1, a2, rtol=1e-15)
    # value: l = l_a + l_b e^(m_b - m_a)
    np.testing.assert_allclose(l1, 2.0 + 3.0 * math.exp(-1.75), rtol=1e-15)


def test_prefill_single_token_equals_decode():
    rng = np.random.default_rng(13)
    case = _paged_case(rng, [1, 9, 40], 8, 2, 64, 8, "bf16")
    cu = np.arange(4, dtype=np.int32)
    dec = oracle.paged_decode(case["q"], "bf16", case["pool"], case["table"], case["ctx"], 0.125)
    pre = oracle.paged_prefill(case["q"], "bf16", cu, case["pool"], case["table"], case["ctx"],
                               0.125, causal=True)
    assert np.array_equal(dec, pre)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_prefill_no_cache_equals_causal_sdpa(kv_dtype):
    rng = np.random.default_rng(14)
    n = [5, 23, 1]
    case = _paged_case(rng, n, 8, 2, 64, 16, kv_dtype)
    qs = [to_storage(rng.standard_normal((c, 8, 64), dtype=np.float32), "bf16") for c in n]
    q = np.concatenate(qs)
    cu = np.r_[0, np.cumsum(n)].astype(np.int32)
    scale = 0.125
    got = oracle.paged_prefill(q, "bf16", cu, case["pool"], case["table"], case["ctx"], scale, True)
    for s, c in enumerate(n):
        Q = _values(qs[s], "bf16").permute(1, 0, 2)[None]  # [1][Hq][c][D]
        K = _contiguous_values(case, s, "k").permute(1, 0, 2)[None]
        V = _contiguous_values(case, s, "v").permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(Q, K, V, scale=scale, is_causal=True, enable_gqa=True)
        np.testing.assert_allclose(got[cu[s]:cu[s + 1]], ref[0].permute(1, 0, 2).numpy(),
                                   rtol=1e-12, atol=1e-12)
    # rows subset returns the same rows
    rows = np.array([0, 7, 28], np.int64)
    sub = oracle.paged_prefill(q, "bf16", cu, case["pool"], case["table"], case["ctx"], scale,
                               True, rows=rows)
    assert np.array_equal(sub, got[rows])


def test_prefill_with_cache_is_bottom_right_causal():
    """With ctx cached+new tokens, new row i sees exactly keys 0 .. ctx-new+i: compare with
    SDPA under an explicit bottom-right mask."""
    rng = np.random.default_rng(15)
    ctxs = [40, 19]
    new = [7, 19]
    case = _paged_case(rng, ctxs, 4, 4, 64, 8, "f16")
    qs = [to_storage(rng.standard_normal((c, 4, 64), dtype=np.float32), "f16") for c in new]
    q = np.concatenate(qs)
    cu = np.r_[0, np.cumsum(new)].astype(np.int32)
    got = oracle.paged_prefill(q, "f16", cu, case["pool"], case["table"], case["ctx"], 0.125, True)
    for s in range(2):
        Q = _values(qs[s], "f16").permute(1, 0, 2)[None]
        K = _contiguous_values(case, s, "k").permute(1, 0, 2)[None]
        V = _contiguous_values(case, s, "v").permute(1, 0, 2)[None]
        i = torch.arange(new[s])[:, None]
        t = torch.arange(ctxs[s])[None, :]
        mask = t <= (ctxs[s] - new[s] + i)
        ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=0.125)
        np.testing.assert_allclose(got[cu[s]:cu[s + 1]], ref[0].permute(1, 0, 2).numpy(),
                                   rtol=1e-12, atol=1e-12)
    nc = oracle.paged_prefill(q, "f16", cu, case["pool"], case["table"], case["ctx"], 0.125, False)
    dec_q = np.stack([qs[0][-1], qs[1][-1]])
    dec = oracle.paged_decode(dec_q, "f16", case["pool"], case["table"], case["ctx"], 0.125)
    assert np.array_equal(nc[[cu[1] - 1, cu[2] - 1]], dec)


# --------------------------------------------------------------------------------------
# Sliding window ("03 | PagedAttention and the KV-cache memory system" §1.1 table:
# sliding/local attention keeps and uses only the tokens inside the window; §7: at
# position p the window is [p - w + 1, p], and blocks before it may be released)
# --------------------------------------------------------------------------------------
@pytest.mark.parametrize("kv_dtype,Hq,Hkv,D,B,w", [
    ("bf16", 8, 2, 128, 16, 37), ("f32", 4, 2, 64, 4, 5), ("fp8", 8, 1, 128, 16, 100),
    ("f16", 4, 4, 64, 32, 64)])
def test_window_decode_equals_masked_sdpa(kv_dtype, Hq, Hkv, D, B, w):
    """Against the library routine on the keys of [ctx - w, ctx) only."""
    rng = np.random.default_rng(500 + w + B)
    ctxs = [1, w - 1, w, w + 1, 2 * w + 3, 5 * B + 7, 300]
    case = _paged_case(rng, ctxs, Hq, Hkv, D, B, kv_dtype)
    scale = 1.0 / math.sqrt(D)
    got = oracle.paged_decode(case["q"], case["q_dtype"], case["pool"], case["table"],
                              case["ctx"], scale, window=w)
    for s, c in enumerate(ctxs):
        q = _values(case["q"][s], case["q_dtype"])
        lo = max(0, c - w)
        K = _contiguous_values(case, s, "k")[lo:].permute(1, 0, 2)[None]
        V = _contiguous_values(case, s, "v")[lo:].permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(q[None, :, None, :], K, V, scale=scale,
                                             enable_gqa=True)[0, :, 0, :].numpy()
        np.testing.assert_allclose(got[s], ref, rtol=1e-12, atol=1e-12)


def test_window_of_one_is_the_newest_value_row():
    rng = np.random.default_rng(77)
    case = _paged_case(rng, [1, 9, 40], 4, 2, 64, 8, "bf16")
    got = oracle.paged_decode(case["q"], case["q_dtype"], case["pool"], case["table"],
                              case["ctx"], 0.125, window=1)
    for s, c in enumerate([1, 9, 40]):
        v_last = _contiguous_values(case, s, "v")[c - 1].numpy()  # [Hkv][D]
        np.testing.assert_array_equal(got[s], np.repeat(v_last, 2, axis=0))


def test_window_never_reads_keys_before_it():
    """NaN written into every K/V slot older than each sequence's window leaves the
    windowed output finite and unchanged, while the whole-context decode sees it."""
    rng = np.random.default_rng(78)
    ctxs = [70, 129, 16, 300]
    w = 48
    case = _paged_case(rng, ctxs, 8, 2, 64, 16, "bf16")
    pool, B = case["pool"], 16
    scale = 0.125
    before = oracle.paged_decode(case["q"], "bf16", pool, case["table"], case["ctx"], scale,
                                 window=w)
    full_before = oracle.paged_decode(case["q"], "bf16", pool, case["table"], case["ctx"], scale)
    for s, c in enumerate(ctxs):
        for t in range(max(0, c - w)):
            blk, off = case["table"][s, t // B], t % B
            pool.k[blk, :, off, :] = NAN_BITS["bf16"]
            pool.v[blk, :, off, :] = NAN_BITS["bf16"]
    after = oracle.paged_decode(case["q"], "bf16", pool, case["table"], case["ctx"], scale,
                                window=w)
    assert np.isfinite(after).all()
    np.testing.assert_array_equal(after, before)
    # the whole-context decode does read those slots (sequence 2 has none before its window)
    full = oracle.paged_decode(case["q"], "bf16", pool, case["table"], case["ctx"], scale)
    for s in (0, 1, 3):
        assert not np.array_equal(full[s], full_before[s])
    np.testing.assert_array_equal(full[2], full_before[2])
