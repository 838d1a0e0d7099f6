"""Pins of the oracle's addressing and write path against what the pages fix.

- physical_slot: the printed worked example and error rules
  ("KV Cache: capacity, layout, lifecycle", section "Page-table addressing").
- The mapping figures ("03 | PagedAttention and the KV-cache memory system" §3;
  "What is the principle of PagedAttention?" §2).
- Brute force over every small table: the slot lands in the block the table names,
  at the same offset, and distinct positions never share a slot.
- The write path ("03 | ..." §4.1): scatter then gather returns the inputs bit for
  bit; untouched slots keep their sentinel; padding entries are skipped.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_physical_slot_printed_example():
    g = _golden("slot_mapping_page_table_addressing.json")
    for case in g["cases"]:
        assert oracle.physical_slot(g["block_table"], g["block_size"], case["token_pos"]) == case["slot"]


def test_physical_slot_errors():
    table = [9, 2, 17]
    with pytest.raises(ValueError):
        oracle.physical_slot(table, 0, 3)  # block size must be positive
    with pytest.raises(ValueError):
        oracle.physical_slot(table, -4, 3)
    with pytest.raises(ValueError):
        oracle.physical_slot(table, 4, -1)  # negative position
    with pytest.raises(IndexError):
        oracle.physical_slot(table, 4, 12)  # logical block 3 is not allocated
    with pytest.raises(IndexError):
        oracle.physical_slot([], 4, 0)
    with pytest.raises(ValueError):
        oracle.physical_slot([9, -1, 17], 4, 5)  # negative physical id


def test_mapping_figures():
    g = _golden("block_table_figures.json")
    for case in g["cases"]:
        table = case["block_table"]
        sizes = [case["block_size"]] if case["block_size"] else [1, 2, 4, 16]
        for B in sizes:
            for pos in range(len(table) * B):
                slot = oracle.physical_slot(table, B, pos)
                assert slot // B == table[pos // B]
                assert slot % B == pos % B


def test_physical_slot_brute_force_small_tables():
    for L in range(0, 4):
        for table in itertools.product(range(6), repeat=L):
            for B in range(1, 5):
                seen = {}
                for pos in range(L * B + B):
                    if pos >= L * B:
                        with pytest.raises(IndexError):
                            oracle.physical_slot(list(table), B, pos)
                        continue
                    slot = oracle.physical_slot(list(table), B, pos)
                    assert slot // B == table[pos // B] and slot % B == pos % B
                    if len(set(table)) == len(table):
                        assert slot not in seen, "two positions share a slot"
                    seen[slot] = pos


def test_slot_mapping_matches_physical_slot_and_padding():
    rng = np.random.default_rng(7)
    S, W, B = 5, 6, 4
    bt = rng.permutation(40)[: S * W].reshape(S, W).astype(np.int32)
    bt[2, 4:] = -1  # unallocated tail of sequence 2
    seq = rng.integers(-1, S, size=200).astype(np.int32)
    pos = rng.integers(-2, W * B + 3, size=200).astype(np.int32)
    got = oracle.slot_mapping(bt, seq, pos, B)
    for i in range(200):
        try:
            if seq[i] < 0:
                raise ValueError
            want = oracle.physical_slot(list(bt[seq[i]]), B, int(pos[i]))
        except (ValueError, IndexError):
            want = -1
        assert got[i] == want


def _gather_logical(pool_arr, slots, B):
    blk, off = slots // B, slots % B
    return pool_arr[blk, :, off, :]


@pytest.mark.parametrize("dtype,np_t", [("f32", np.float32), ("f16", np.uint16), ("bf16", np.uint16)])
def test_write_then_gather_roundtrip(dtype, np_t):
    rng = np.random.default_rng(11)
    NB, B, H, D = 10, 4, 3, 8
    sentinel = np.array(0x7FC00000, np.uint32).view(np.float32) if dtype == "f32" else 0x7E00
    pool = oracle.Pool(NB, B, H, D, dtype, fill_bits=sentinel)
    T = 17
    slots = rng.permutation(NB * B)[:T].astype(np.int64)
    slots[3] = -1  # padding
    if dtype == "f32":
        k = rng.standard_normal((T, H, D)).astype(np.float32)
        v = rng.standard_normal((T, H, D)).astype(np.float32)
    else:
        k = rng.integers(0, 0x7C00, size=(T, H, D)).astype(np.uint16)
        v = rng.integers(0, 0x7C00, size=(T, H, D)).astype(np.uint16)
    oracle.kv_cache_write(pool, slots, k, v, dtype)
    live = slots >= 0
    gk = _gather_logical(pool.k, slots[live], B)
    gv = _gather_logical(pool.v, slots[live], B)
    assert np.array_equal(gk.view(np.uint8), k[live].view(np.uint8))
    assert np.array_equal(gv.view(np.uint8), v[live].view(np.uint8))
    # every other slot still holds the sentinel
    mask = np.ones(NB * B, bool)
    mask[slots[live]] = False
    rest = pool.k.transpose(0, 2, 1, 3).reshape(NB * B, H, D)[mask]
    if dtype == "f32":
        assert np.isnan(rest).all()
    else:
        assert (rest == sentinel).all()


def test_fp8_write_quantises_within_half_spacing():
    """e4m3(x/s)*s lies within half an e4m3 spacing of x (relative to s); values that
    are an exact e4m3 code times a power-of-two scale come back exactly."""
    import torch

    rng = np.random.default_rng(3)
    NB, B, H, D = 6, 4, 2, 16
    pool = oracle.Pool(NB, B, H, D, "fp8", fill_bits=0x7F)
    pool.k_scale = (2.0 ** rng.integers(-3, 4, size=(NB, H))).astype(np.float32)
    pool.v_scale = rng.uniform(0.01, 0.5, size=(NB, H)).astype(np.float32)
    T = NB * B
    slots = rng.permutation(T).astype(np.int64)
    codes = rng.integers(0, 0x7F, size=(T, H, D)).astype(np.uint8) | (
        rng.integers(0, 2, size=(T, H, D)).astype(np.uint8) << 7)
    exact = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    kx = (exact * pool.k_scale[slots // B][:, :, None]).astype(np.float32)
    kbits = torch.from_numpy(kx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(torch.from_numpy(kbits.view(np.int16)).view(torch.bfloat16).float().numpy(), kx)
    vx = rng.standard_normal((T, H, D)).astype(np.float32)
    vbits = torch.from_numpy(vx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    oracle.kv_cache_write(pool, slots, kbits, vbits, "bf16")
    got_k = pool.k[slots // B, :, slots % B, :]
    assert np.array_equal(got_k, codes), "exact codes times power-of-two scales must round-trip"
    vq = pool.v[slots // B, :, slots % B, :]
    vdec = torch.from_numpy(vq).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    vin = torch.from_numpy(vbits.view(np.int16)).view(torch.bfloat16).double().numpy()
    s = pool.v_scale[slots // B].astype(np.float64)[:, :, None]
    y = vin / s
    # spacing of e4m3 around |y|: 2^(e-3) for normal binades, 2^-9 below 2^-6
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
    half = 2.0 ** (e - 3) / 2
    inr = np.abs(y) <= 448
    # y is the fp32 quotient; allow its own rounding (2^-24 relative) on top
    assert np.all(np.abs(y - vdec)[inr] <= half[inr] + np.abs(y[inr]) * 2.0 ** -23)
    assert np.all(np.abs(vdec[~inr]) == 448)


@pytest.mark.parametrize("kv,mode", [("int8", "token"), ("int8", "tensor"), ("fp8", "token")])
def test_quantised_write_uses_each_tokens_scale(kv, mode):
    """[P1 §8.1] per-token-head and per-tensor scales: codes that are exact integers
    (int8) or exact e4m3 values (fp8) times the scale of their own (block, head, token)
    slot, read back by logical slot, come back exactly; any other value lands within
    half a code of x / scale."""
    import torch

    rng = np.random.default_rng(len(kv) * 10 + len(mode))
    NB, B, H, D = 6, 4, 2, 16
    pool = oracle.Pool(NB, B, H, D, kv, scale_mode=mode)
    pool.k_scale = (2.0 ** rng.integers(-3, 4, size=pool.scale_shape())).astype(np.float32)
    pool.v_scale = rng.uniform(0.01, 0.5, size=pool.scale_shape()).astype(np.float32)
    T = NB * B
    slots = rng.permutation(T).astype(np.int64)
    blk, off = slots // B, slots % B

    def per_slot(sc):  # [T][H] scale of each written row, by logical slot
        if mode == "tensor":
            return np.broadcast_to(sc[0], (T, H)).astype(np.float64)
        return sc[blk, :, off].astype(np.float64)

    if kv == "int8":
        codes = rng.integers(-127, 128, size=(T, H, D)).astype(np.int8)
        exact = codes.astype(np.float32)
    else:
        codes = rng.integers(0, 0x7F, size=(T, H, D)).astype(np.uint8) | (
            rng.integers(0, 2, size=(T, H, D)).astype(np.uint8) << 7)
        exact = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    kx = (exact * per_slot(pool.k_scale)[:, :, None]).astype(np.float32)
    kbits = torch.from_numpy(kx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    vx = rng.standard_normal((T, H, D)).astype(np.float32)
    vbits = torch.from_numpy(vx).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    oracle.kv_cache_write(pool, slots, kbits, vbits, "bf16")
    assert np.array_equal(pool.k[blk, :, off, :], codes)
    vin = torch.from_numpy(vbits.view(np.int16)).view(torch.bfloat16).double().numpy()
    y = vin / per_slot(pool.v_scale)[:, :, None]
    vq = pool.v[blk, :, off, :]
    if kv == "int8":
        assert (np.abs(vq.astype(np.float64) - np.clip(y, -127, 127)) <= 0.5 + 1e-9).all()
    else:
        dec = torch.from_numpy(vq).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        assert (np.abs(dec - np.clip(y, -448, 448)) <= 2.0 ** (np.floor(np.log2(
            np.maximum(np.abs(y), 2.0 ** -6))) - 3) / 2 + 1e-12).all()
