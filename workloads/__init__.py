"""Seeded synthetic workloads for paged decode / prefill.

This module builds INPUTS only: context lengths, block tables, query vectors and
the per-token K/V that the write path stores, each drawn from
``numpy.random.default_rng(seed)`` in a fixed order (context lengths, tail
lengths, block permutation, q, k, v), as fp32 N(0, 1) rounded to the storage type
(round to nearest even).  It holds none of the method's arithmetic: no slot
computation, no quantisation, no attention.  The tests feed the same arrays to
the HIP library and to the oracle; the benchmark feeds them to the library.

Block tables: every sequence owns ceil(ctx / B) distinct physical blocks drawn
from a shuffled pool (shared-prefix workloads share their first blocks).  One
extra block, never referenced by a live table entry, pads every table row past
its live length; the tests fill it (and all spare blocks) with NaN so that a read
of an uninitialised slot shows up in the output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8,
           "int8": np.int8}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "int8": 1}
QUANTISED = ("fp8", "int8")
# the largest magnitude of each quantised type (E4M3: 448; symmetric int8: 127)
QMAX = {"fp8": 448.0, "int8": 127.0}
NAN_BITS = {"f32": np.array(0x7FC00000, np.uint32).view(np.float32), "f16": 0x7E00,
            "bf16": 0x7FC0, "fp8": 0x7F}


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> storage bit patterns of `dtype` (round to nearest even)."""
    x = np.ascontiguousarray(x, np.float32)
    if dtype == "f32":
        return x
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def storage_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp32 values of f32/f16/bf16 storage bits (used only to derive fp8 scales)."""
    if dtype == "f32":
        return np.asarray(bits, np.float32)
    if dtype == "f16":
        return np.asarray(bits, np.uint16).view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


@dataclass
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    kv_dtype: str
    q_dtype: str
    num_blocks: int
    context_lens: np.ndarray          # int32 [S]
    block_table: np.ndarray           # int32 [S][W]
    q: np.ndarray                     # storage bits: decode [S][Hq][D], prefill [total_q][Hq][D]
    fill_seq: np.ndarray              # int32 [T]: owner sequence of each stored token
    fill_pos: np.ndarray              # int32 [T]: its position in that sequence
    k_src: np.ndarray                 # storage bits of src_dtype [T][Hkv][D]
    v_src: np.ndarray
    src_dtype: str
    scale: float                      # softmax scale (fp32 value of 1/sqrt(D))
    pad_block: int                    # block id used for table entries past the live length
    k_scale: Optional[np.ndarray] = None   # quantised pools: float32, shape per scale_mode
    v_scale: Optional[np.ndarray] = None
    scale_mode: str = "block"             # "block" [nb][Hkv], "tensor" [1], "token" [nb][Hkv][B]
    cu_seqlens_q: Optional[np.ndarray] = None  # prefill only: int32 [S+1]
    partition_size: int = 0
    shared_blocks: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def decode_new_token_rows(self) -> np.ndarray:
        """Index into fill_* of each sequence's newest token (position ctx-1), -1 if ctx=0."""
        idx = np.full(self.num_seqs, -1, np.int64)
        last = {(int(s), int(p)): i for i, (s, p) in enumerate(zip(self.fill_seq, self.fill_pos))}
        for s in range(self.num_seqs):
            c = int(self.context_lens[s])
            if c > 0:
                # a shared-prefix token is stored once, under the first sequence
                idx[s] = last.get((s, c - 1), last.get((0, c - 1), -1))
        return idx

    def kv_bytes(self) -> int:
        """Bytes of K and V that decode reads: sum(ctx) * 2 * Hkv * D * elem, plus the scales
        of a quantised pool (one per live block and head, one per token and head, or 2 x 4
        bytes for the whole pool)."""
        e = ELEM_BYTES[self.kv_dtype]
        ntok = int(self.context_lens.astype(np.int64).sum())
        tot = ntok * 2 * self.num_kv_heads * self.head_dim * e
        if self.kv_dtype in QUANTISED:
            if self.scale_mode == "block":
                nblk = sum(math.ceil(int(c) / self.block_size) for c in self.context_lens)
                tot += nblk * 2 * self.num_kv_heads * 4
            elif self.scale_mode == "token":
                tot += ntok * 2 * self.num_kv_heads * 4
            else:
                tot += 2 * 4
        return tot


def _assign_tables(rng, ctx, B, spare_frac, shared_prefix_blocks=0):
    """Shuffled physical ids: shared blocks first, then each sequence's private blocks."""
    S = len(ctx)
    need = [max(0, math.ceil(int(c) / B) - shared_prefix_blocks) for c in ctx]
    used = shared_prefix_blocks + sum(need)
    nblk_live = math.ceil(used * (1.0 + spare_frac)) if spare_frac > 0 else used
    num_blocks = nblk_live + 1  # + one padding block
    perm = rng.permutation(num_blocks).astype(np.int32)
    pad_block = int(perm[-1])
    W = max(1, max(math.ceil(int(c) / B) for c in ctx) if S else 1)
    table = np.full((S, W), pad_block, np.int32)
    shared = perm[:shared_prefix_blocks]
    nxt = shared_prefix_blocks
    for s in range(S):
        n_s = math.ceil(int(ctx[s]) / B)
        row = list(shared[: min(n_s, shared_prefix_blocks)])
        row += list(perm[nxt: nxt + need[s]])
        nxt += need[s]
        table[s, :len(row)] = row
    return table, num_blocks, pad_block


def _draw_kv(rng, T, Hkv, D, dtype, chunk=1 << 24):
    """k then v, each [T][Hkv][D] fp32 N(0,1) rounded to `dtype`, drawn in chunks."""
    out = []
    for _ in range(2):
        arr = np.empty((T, Hkv, D), STORAGE[dtype])
        flat = arr.reshape(-1)
        n = flat.size
        for o in range(0, n, chunk):
            m = min(chunk, n - o)
            flat[o:o + m] = to_storage(rng.standard_normal(m, dtype=np.float32), dtype)
        out.append(arr)
    return out


def make_decode(name, seed, ctx_lens=None, ctx_range=None, num_seqs=None, Hq=4, Hkv=2, D=64,
                B=4, kv_dtype="f32", q_dtype=None, spare_frac=0.0, shared_prefix=0,
                tail_range=None, partition_size=0, fp8_src_dtype="bf16", scale_mode="block"):
    """Generic decode workload.  ctx from an explicit list, from U[lo, hi] (inclusive), or
    as shared_prefix + U[tail_range] tails."""
    rng = np.random.default_rng(seed)
    q_dtype = q_dtype or ("bf16" if kv_dtype == "fp8" else kv_dtype)
    if ctx_lens is not None:
        ctx = np.asarray(ctx_lens, np.int32)
    elif ctx_range is not None:
        ctx = rng.integers(ctx_range[0], ctx_range[1] + 1, size=num_seqs).astype(np.int32)
    else:
        ctx = np.zeros(num_seqs, np.int32)
    if tail_range is not None:
        tails = rng.integers(tail_range[0], tail_range[1] + 1, size=num_seqs).astype(np.int32)
        ctx = (shared_prefix + tails).astype(np.int32)
    S = len(ctx)
    shared_blocks = shared_prefix // B
    table, num_blocks, pad = _assign_tables(rng, ctx, B, spare_frac, shared_blocks)
    q = to_storage(rng.standard_normal((S, Hq, D), dtype=np.float32), q_dtype)
    # stored tokens: the shared prefix once (under sequence 0), then each private part
    fs, fp = [], []
    if shared_prefix > 0 and S > 0:
        fs.append(np.zeros(shared_prefix, np.int32))
        fp.append(np.arange(shared_prefix, dtype=np.int32))
    for s in range(S):
        start = shared_prefix if shared_prefix > 0 else 0
        fs.append(np.full(int(ctx[s]) - start, s, np.int32))
        fp.append(np.arange(start, int(ctx[s]), dtype=np.int32))
    fill_seq = np.concatenate(fs) if fs else np.zeros(0, np.int32)
    fill_pos = np.concatenate(fp) if fp else np.zeros(0, np.int32)
    src_dtype = fp8_src_dtype if kv_dtype in QUANTISED else kv_dtype
    k_src, v_src = _draw_kv(rng, len(fill_seq), Hkv, D, src_dtype)
    wl = Workload(name, S, Hq, Hkv, D, B, kv_dtype, q_dtype, num_blocks, ctx, table, q,
                  fill_seq, fill_pos, k_src, v_src, src_dtype,
                  float(np.float32(1.0 / math.sqrt(D))), pad, scale_mode=scale_mode,
                  partition_size=partition_size, shared_blocks=shared_blocks)
    if kv_dtype in QUANTISED:
        wl.k_scale, wl.v_scale = amax_scales(wl)
    return wl


def make_prefill(name, seed, num_seqs, cached, new, Hq, Hkv, D, B, kv_dtype="fp8",
                 q_dtype="bf16", fp8_src_dtype="bf16"):
    """Chunked prefill: every sequence holds `cached` earlier tokens plus `new` query tokens
    (ctx = cached + new), all K/V of which are stored before attention reads them."""
    rng = np.random.default_rng(seed)
    cached = np.broadcast_to(np.asarray(cached, np.int32), (num_seqs,)).copy()
    new = np.broadcast_to(np.asarray(new, np.int32), (num_seqs,)).copy()
    ctx = (cached + new).astype(np.int32)
    table, num_blocks, pad = _assign_tables(rng, ctx, B, 0.0)
    total_q = int(new.sum())
    q = to_storage(rng.standard_normal((total_q, Hq, D), dtype=np.float32), q_dtype)
    fill_seq = np.concatenate([np.full(int(c), s, np.int32) for s, c in enumerate(ctx)])
    fill_pos = np.concatenate([np.arange(int(c), dtype=np.int32) for c in ctx])
    src_dtype = fp8_src_dtype if kv_dtype in QUANTISED else kv_dtype
    k_src, v_src = _draw_kv(rng, len(fill_seq), Hkv, D, src_dtype)
    cu = np.zeros(num_seqs + 1, np.int32)
    cu[1:] = np.cumsum(new)
    wl = Workload(name, num_seqs, Hq, Hkv, D, B, kv_dtype, q_dtype, num_blocks, ctx, table, q,
                  fill_seq, fill_pos, k_src, v_src, src_dtype,
                  float(np.float32(1.0 / math.sqrt(D))), pad, cu_seqlens_q=cu)
    if kv_dtype in QUANTISED:
        wl.k_scale, wl.v_scale = amax_scales(wl)
    return wl


def amax_scales(wl: Workload):
    """fp32 scales of a quantised pool, K and V separately: max(amax, 2^-20) / QMAX over the
    values that share the scale in the workload's scale_mode (a block and head, the whole
    pool, or one token and head).  Unused blocks get 1.0; in token mode a slot no token
    is written to gets NaN, so that a kernel that reads the scale of a key past the
    context shows it.  This is a property of the input, not of the method: any positive
    scale is valid."""
    qmax = np.float32(QMAX[wl.kv_dtype])
    floor = np.float32(2.0 ** -20)
    B, H = wl.block_size, wl.num_kv_heads
    phys = wl.block_table[wl.fill_seq, wl.fill_pos // B]
    off = wl.fill_pos % B
    scales = []
    for src in (wl.k_src, wl.v_src):
        vals = np.abs(storage_to_f32(src, wl.src_dtype)).max(axis=2)  # [T][Hkv]
        if wl.scale_mode == "tensor":
            amax = np.float32(vals.max()) if vals.size else np.float32(0)
            sc = np.array([np.maximum(amax, floor) / qmax], np.float32)
        elif wl.scale_mode == "token":
            sc = np.full((wl.num_blocks, H, B), np.nan, np.float32)
            sc[phys, :, off] = (np.maximum(vals, floor) / qmax).astype(np.float32)
        else:
            amax = np.zeros((wl.num_blocks, H), np.float32)
            np.maximum.at(amax, phys, vals)
            sc = (np.maximum(amax, floor) / qmax).astype(np.float32)
            used = np.zeros(wl.num_blocks, bool)
            used[phys] = True
            sc[~used] = 1.0
        scales.append(sc)
    return scales[0], scales[1]


# ----------------------------------------------------------------------------------------
# The five named workloads (full size) and reduced variants that the oracle finishes in
# seconds while still spanning several tiles, partitions and a ragged tail.
# ----------------------------------------------------------------------------------------
def tiny_decode(seed=1):
    """2 sequences (ctx 5 and 11), H_q 4, H_kv 2, D 64, B 4, fp32, 8 physical blocks,
    block ids a seeded permutation (3 blocks spare)."""
    rng_name = "tiny decode fp32 (S=2, ctx 5/11, Hq4 Hkv2 D64 B4)"
    rng = np.random.default_rng(seed)
    ctx = np.array([5, 11], np.int32)
    perm = rng.permutation(8).astype(np.int32)
    table = np.stack([np.r_[perm[0:2], perm[5]], perm[2:5]]).astype(np.int32)
    S, Hq, Hkv, D, B = 2, 4, 2, 64, 4
    q = rng.standard_normal((S, Hq, D), dtype=np.float32)
    fill_seq = np.r_[np.zeros(5, np.int32), np.ones(11, np.int32)]
    fill_pos = np.r_[np.arange(5), np.arange(11)].astype(np.int32)
    k_src, v_src = _draw_kv(rng, 16, Hkv, D, "f32")
    return Workload(rng_name, S, Hq, Hkv, D, B, "f32", "f32", 8, ctx, table, q, fill_seq,
                    fill_pos, k_src, v_src, "f32", float(np.float32(1.0 / 8.0)), int(perm[5]))


def llama3_8b_decode(seed=2, small=False, partition_size=512, kv_dtype="bf16",
                     scale_mode="block"):
    """64 sequences, ctx U[128, 4096], H_q 32, H_kv 8, D 128, B 16, bf16, pool = needed
    blocks + 20% spare, shuffled tables.  A quantised kv_dtype ("fp8", "int8") stores the
    same bf16 draws as codes with scales in `scale_mode`; q stays bf16."""
    kv = kv_dtype if kv_dtype == "bf16" else "%s, %s scales" % (kv_dtype, scale_mode)
    if small:
        return make_decode("llama3-8b-shaped decode (small: S=6, ctx U[1,1200], %s)" % kv, seed,
                           ctx_range=(1, 1200), num_seqs=6, Hq=32, Hkv=8, D=128, B=16,
                           kv_dtype=kv_dtype, q_dtype="bf16", spare_frac=0.2,
                           partition_size=partition_size, scale_mode=scale_mode)
    return make_decode("llama3-8b-shaped decode (S=64, ctx U[128,4096], Hq32 Hkv8 D128 B16 %s)"
                       % kv,
                       seed, ctx_range=(128, 4096), num_seqs=64, Hq=32, Hkv=8, D=128, B=16,
                       kv_dtype=kv_dtype, q_dtype="bf16", spare_frac=0.2,
                       partition_size=partition_size, scale_mode=scale_mode)


def long_context_decode(seed=3, small=False):
    """8 sequences, ctx U[32768, 131072], H_q 64, H_kv 8, D 128, B 16, bf16, 512-token
    partitions merged by log-sum-exp."""
    if small:
        return make_decode("long-context split-KV decode (small: S=3, ctx U[1500,4000])", seed,
                           ctx_range=(1500, 4000), num_seqs=3, Hq=64, Hkv=8, D=128, B=16,
                           kv_dtype="bf16", partition_size=512)
    return make_decode("long-context split-KV decode (S=8, ctx U[32768,131072], Hq64 Hkv8 D128 "
                       "B16 bf16, P=512)", seed, ctx_range=(32768, 131072), num_seqs=8, Hq=64,
                       Hkv=8, D=128, B=16, kv_dtype="bf16", partition_size=512)


def shared_prefix_decode(seed=4, small=False):
    """256 sequences sharing one 2048-token prefix (same physical blocks) plus private
    tails U[0, 512], H_q = H_kv = 32, D 128, B 32, fp16."""
    if small:
        return make_decode("MHA shared-prefix decode (small: S=8, prefix 256, tails U[0,100])",
                           seed, num_seqs=8, Hq=32, Hkv=32, D=128, B=32, kv_dtype="f16",
                           shared_prefix=256, tail_range=(0, 100))
    return make_decode("MHA shared-prefix decode (S=256, prefix 2048 + tails U[0,512], Hq=Hkv=32 "
                       "D128 B32 fp16)", seed, num_seqs=256, Hq=32, Hkv=32, D=128, B=32,
                       kv_dtype="f16", shared_prefix=2048, tail_range=(0, 512))


def fp8_chunked_prefill(seed=5, small=False):
    """16 sequences with 4096 cached tokens + 512 new query tokens each (causal inside the
    chunk), H_q 32, H_kv 8, D 128, B 16, e4m3 KV with per-block-per-head fp32 scales, bf16 q."""
    if small:
        return make_prefill("fp8 KV chunked prefill (small: S=3, cached 100..300, new 1..130)",
                             seed, 3, [300, 100, 0], [130, 1, 77], 32, 8, 128, 16)
    return make_prefill("fp8 KV chunked prefill (S=16, 4096 cached + 512 new, Hq32 Hkv8 D128 B16 "
                        "e4m3 + fp32 scales, bf16 q)", seed, 16, 4096, 512, 32, 8, 128, 16)


CONFIGS = {
    1: tiny_decode,
    2: llama3_8b_decode,
    3: long_context_decode,
    4: shared_prefix_decode,
    5: fp8_chunked_prefill,
}
