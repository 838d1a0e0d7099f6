"""GPU parity of paged decode attention against the oracle.

Method: "03 | PagedAttention and the KV-cache memory system" §4 (paged loop,
online-softmax merge, split-KV); the tolerance |gpu - oracle| <= 2e-3 + 1e-2|oracle|
per element, oracle in fp64 on the same stored values.  Every pool is first filled
with NaN (0xFF bytes) and then written through the library's own write path, whose
bytes are compared bit-exactly with the oracle's write; spare blocks, table padding
and tail slots stay NaN, so any read of an uninitialised slot fails the finiteness
check ("KV Cache: capacity, layout, lifecycle", lifecycle invariant 6).
"""
import math

import numpy as np
import pytest

import oracle
from helpers import GpuCase, assert_close, oracle_pool, peaked, plant_keys, to_f64, torch_bits
import workloads as W

pytestmark = pytest.mark.gpu


def _check_pools(case, opool):
    gk, gv = case.logical_pools()
    assert np.array_equal(gk.view(np.uint8), opool.k.view(np.uint8)), "K pool differs"
    assert np.array_equal(gv.view(np.uint8), opool.v.view(np.uint8)), "V pool differs"


def _run(wl, partitions, seqs=None, check_pools=True):
    case = GpuCase(wl)
    opool = oracle_pool(wl)
    if check_pools:
        _check_pools(case, opool)
    ref = oracle.paged_decode(wl.q, wl.q_dtype, opool, wl.block_table, wl.context_lens, wl.scale,
                              seqs=seqs)
    res = {}
    for P in partitions:
        out = to_f64(case.decode(partition_size=P), wl.q_dtype)
        if seqs is not None:
            out = out[seqs]
        res[P] = assert_close(out, ref, "%s P=%d" % (wl.name, P))
    return res


def test_tiny_decode_fp32():
    print(_run(W.tiny_decode(), [0, 64, -1]))


def test_llama3_8b_small():
    print(_run(W.llama3_8b_decode(small=True), [0, 64, 512, -1]))


def test_long_context_small():
    print(_run(W.long_context_decode(small=True), [512, 0, -1]))


def test_shared_prefix_small():
    print(_run(W.shared_prefix_decode(small=True), [0, 256, -1]))


@pytest.mark.parametrize("B", [1, 2, 4, 8, 16, 32, 64])
def test_edge_context_lengths(B):
    """ctx in {0, 1, B-1, B, B+1, 2B, 63, 64, 65, max}: block and chunk boundaries."""
    ctx = sorted({0, 1, max(B - 1, 0), B, B + 1, 2 * B, 63, 64, 65, 129, 300})
    wl = W.make_decode("edge B=%d" % B, 40 + B, ctx_lens=ctx, Hq=8, Hkv=2, D=128, B=B,
                       kv_dtype="bf16", spare_frac=0.1)
    print(_run(wl, [0, 64, 128, -1]))


@pytest.mark.parametrize("kv,Hq,Hkv,D", [
    ("f32", 4, 4, 64), ("f32", 16, 2, 128), ("f16", 6, 2, 64), ("f16", 12, 4, 128),
    ("bf16", 7, 1, 128), ("bf16", 16, 1, 64), ("bf16", 24, 2, 128), ("fp8", 8, 2, 128),
    ("fp8", 3, 3, 64)])
def test_dtype_head_grid(kv, Hq, Hkv, D):
    """Group sizes 1..16 including non-powers of two, MHA/GQA/MQA, D 64/128, all dtypes."""
    wl = W.make_decode("grid %s %d/%d D%d" % (kv, Hq, Hkv, D), 7 * Hq + D, ctx_range=(1, 700),
                       num_seqs=5, Hq=Hq, Hkv=Hkv, D=D, B=16, kv_dtype=kv, spare_frac=0.1)
    print(_run(wl, [0, 192, -1]))


def test_fp8_q_f16():
    wl = W.make_decode("fp8 kv, f16 q", 77, ctx_range=(50, 600), num_seqs=4, Hq=8, Hkv=2, D=128,
                       B=16, kv_dtype="fp8", q_dtype="f16", fp8_src_dtype="f16")
    print(_run(wl, [0, 128, -1]))


@pytest.mark.parametrize("kv,mode,B,Hq,Hkv,D,q_dtype", [
    ("int8", "block", 16, 8, 2, 128, "bf16"), ("int8", "token", 16, 8, 2, 128, "bf16"),
    ("int8", "tensor", 32, 16, 2, 64, "f16"), ("int8", "token", 4, 8, 2, 128, "bf16"),
    ("int8", "block", 1, 6, 2, 64, "bf16"), ("fp8", "token", 16, 8, 2, 128, "bf16"),
    ("fp8", "tensor", 16, 12, 4, 128, "bf16"), ("fp8", "token", 8, 3, 3, 64, "f16"),
    ("int8", "token", 64, 32, 8, 128, "f16")])
def test_quantised_scale_modes(kv, mode, B, Hq, Hkv, D, q_dtype):
    """fp8 and int8 pools with one scale per (block, head), per pool, or per (token, head).
    In token mode every scale slot that no token was written to holds NaN, so a kernel
    that lets the scale of a key past the context reach the output fails."""
    ctx = sorted({0, 1, max(B - 1, 1), B, B + 1, 63, 64, 65, 200, 517})
    wl = W.make_decode("quant %s/%s B%d" % (kv, mode, B), 13 * B + Hq + len(mode), ctx_lens=ctx,
                       Hq=Hq, Hkv=Hkv, D=D, B=B, kv_dtype=kv, q_dtype=q_dtype,
                       fp8_src_dtype=q_dtype, spare_frac=0.2, scale_mode=mode)
    if mode == "token":
        assert np.isnan(wl.v_scale).any()
    print(_run(wl, [0, 128, -1]))


def test_permutation_invariance_bitwise():
    """Relabelling physical ids (pool'[pi(b)] = pool[b], table' = pi(table)) leaves the GPU
    output bitwise unchanged (same partitioning)."""
    import torch
    wl = W.make_decode("perm", 91, ctx_range=(1, 900), num_seqs=6, Hq=16, Hkv=4, D=128, B=16,
                       kv_dtype="bf16", spare_frac=0.3)
    a = GpuCase(wl)
    rng = np.random.default_rng(5)
    pi = rng.permutation(wl.num_blocks).astype(np.int32)
    wl2 = W.Workload(**{**wl.__dict__})
    wl2.block_table = pi[wl.block_table]
    b = GpuCase(wl2)
    for P in (0, 64, -1):
        oa = a.decode(partition_size=P)
        ob = b.decode(partition_size=P)
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_split_reduce_standalone():
    """The LSE reduce on given partials (incl. empty contexts) against the oracle's merge."""
    import torch
    import paged_kv_cache_146_amd as pkv
    rng = np.random.default_rng(3)
    S, Hq, D, P = 5, 6, 128, 64
    ctx = np.array([0, 1, 64, 65, 1000], np.int32)
    maxp = math.ceil(ctx.max() / P)
    po = rng.standard_normal((S, Hq, maxp, D)).astype(np.float32)
    pm = (rng.standard_normal((S, Hq, maxp)) * 5).astype(np.float32)
    ps = rng.uniform(0.5, 40, size=(S, Hq, maxp)).astype(np.float32)
    ref = oracle.split_reduce(po, pm, ps, ctx, P)
    for dt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        out = pkv.pkv_split_kv_reduce(torch.from_numpy(po).cuda(), torch.from_numpy(pm).cuda(),
                                      torch.from_numpy(ps).cuda(), torch.from_numpy(ctx).cuda(),
                                      P, tdt)
        assert_close(to_f64(out, dt), ref, "reduce " + dt)


def _balanced_ws_bytes(wl, workers):
    """Workspace of the balanced mode that holds exactly `workers` workers: one 8-byte
    counter per (sequence, kv head), rounded to 256 bytes, then 2 * workers partial states
    of G x (D + 2) floats."""
    S, Hkv, D = wl.num_seqs, wl.num_kv_heads, wl.head_dim
    G = wl.num_q_heads // Hkv
    C = -(-S * Hkv * 8 // 256) * 256
    return C + 2 * workers * G * (D + 2) * 4


@pytest.mark.parametrize("workers", [1, 3, 8, 37])
def test_balanced_few_workers(workers):
    # Few workers give long shares that cut many pairs, and pairs that span several
    # shares, so most of the output comes from merged pieces.  The workspace starts as
    # 0xFF garbage and serves two calls in a row: the first call's counters must read
    # as stale in the second.
    import torch
    wl = W.llama3_8b_decode(small=True)
    case = GpuCase(wl)
    ref = oracle.paged_decode(wl.q, wl.q_dtype, oracle_pool(wl), wl.block_table,
                              wl.context_lens, wl.scale)
    ws = torch.full((_balanced_ws_bytes(wl, workers),), 0xFF, dtype=torch.uint8, device="cuda")
    for call in range(2):
        out = to_f64(case.decode(partition_size=-1, workspace=ws), wl.q_dtype)
        print(assert_close(out, ref, "%s workers=%d call %d" % (wl.name, workers, call)))


def test_balanced_graph_replay():
    # A captured call reuses its epoch on every replay: the counters it uses must be
    # back at rest when it ends.  An eager call between replays moves them to a newer
    # epoch, which the replay must read as stale.
    import torch
    wl = W.llama3_8b_decode(small=True)
    case = GpuCase(wl)
    ref = oracle.paged_decode(wl.q, wl.q_dtype, oracle_pool(wl), wl.block_table,
                              wl.context_lens, wl.scale)
    ws = torch.full((_balanced_ws_bytes(wl, 8),), 0xFF, dtype=torch.uint8, device="cuda")
    out = case.nan_out()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        case.decode(partition_size=-1, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        case.decode(partition_size=-1, workspace=ws, out=out)
    for r in range(3):
        out.view(torch.uint8).fill_(0xFF)
        graph.replay()
        torch.cuda.synchronize()
        print(assert_close(to_f64(out, wl.q_dtype), ref, "replay %d" % r))
        if r == 1:
            eager = case.decode(partition_size=-1, workspace=ws)
            print(assert_close(to_f64(eager, wl.q_dtype), ref, "eager between replays"))


# ---- full-size workloads: write path bit-exact, sampled sequences vs the oracle ----------
def test_llama3_8b_full_sampled():
    wl = W.llama3_8b_decode()
    seqs = np.array([0, 5, 17, 31, 42, 63], np.int32)
    print(_run(wl, [512, 256, 0, -1], seqs=seqs))


@pytest.fixture(scope="module")
def long_full():
    """The full long-context batch on the GPU (pool written by the library and checked
    bit for bit against the oracle's write) with the oracle's pool beside it."""
    wl = W.long_context_decode()
    case = GpuCase(wl)
    opool = oracle_pool(wl)
    _check_pools(case, opool)
    return wl, case, opool


def _compare(case, wl, opool, partitions, seqs, factor=1):
    """case's decode against the oracle's on the sampled sequences, with q scaled by
    `factor` (a power of two: exact) where factor != 1."""
    qw = wl if factor == 1 else peaked(wl, factor)
    q = None if factor == 1 else torch_bits(qw.q, qw.q_dtype)
    ref = oracle.paged_decode(qw.q, qw.q_dtype, opool, wl.block_table, wl.context_lens,
                              wl.scale, seqs=seqs)
    res = {}
    for P in partitions:
        out = to_f64(case.decode(partition_size=P, q=q), wl.q_dtype)[seqs]
        res[P] = assert_close(out, ref, "%s q x %g P=%d" % (wl.name, factor, P))
    return res


def test_long_context_full_sampled(long_full):
    """The configuration's 512-token partitions, the size pkv_decode_partition_size picks
    for this batch on this device (bench.py's launch), and the balanced mode; the
    longest and the shortest context and one more."""
    import paged_kv_cache_146_amd as pkv
    wl, case, opool = long_full
    auto = pkv.pkv_decode_partition_size(wl.context_lens, wl.num_kv_heads, wl.max_context_len)
    assert auto > 0
    seqs = np.array([int(np.argmax(wl.context_lens)), int(np.argmin(wl.context_lens)), 3],
                    np.int32)
    print("auto partition", auto, _compare(case, wl, opool, [512, auto, -1], seqs))


@pytest.mark.parametrize("factor", [4, 8])
def test_long_context_full_peaked(long_full, factor):
    import paged_kv_cache_146_amd as pkv
    wl, case, opool = long_full
    auto = pkv.pkv_decode_partition_size(wl.context_lens, wl.num_kv_heads, wl.max_context_len)
    seqs = np.array([int(np.argmax(wl.context_lens)), 6], np.int32)
    print(_compare(case, wl, opool, [auto, 512], seqs, factor))


@pytest.mark.parametrize("factor", [4, 8])
def test_llama3_8b_full_peaked(factor):
    wl = W.llama3_8b_decode()
    case = GpuCase(wl)
    opool = oracle_pool(wl)
    seqs = np.array([int(np.argmax(wl.context_lens)), int(np.argmin(wl.context_lens)), 9, 40],
                    np.int32)
    print(_compare(case, wl, opool, [0, -1, 512], seqs, factor))


@pytest.mark.parametrize("kv,mode", [("fp8", "block"), ("int8", "block"), ("fp8", "tensor"),
                                     ("int8", "token"), ("fp8", "token")])
def test_llama3_8b_full_quantised(kv, mode):
    """The full Llama-3-8B-shaped batch over 8-bit pools, in the unsplit launch (two
    chunks deep per wavefront, up to 16 chunks each), the balanced one and 192-token
    partitions:
    the write path bit for bit against the oracle's, sampled sequences within the
    tolerance (the longest and the shortest among them)."""
    wl = W.llama3_8b_decode(kv_dtype=kv, scale_mode=mode)
    seqs = np.array([int(np.argmax(wl.context_lens)), int(np.argmin(wl.context_lens)), 5],
                    np.int32)
    case = GpuCase(wl)
    # the oracle's fp8 encoder searches every code: fill its pool with the sampled
    # sequences' tokens only, and compare the pools on those sequences' blocks
    keep = np.isin(wl.fill_seq, seqs)
    opool = oracle.Pool(wl.num_blocks, wl.block_size, wl.num_kv_heads, wl.head_dim, wl.kv_dtype,
                        scale_mode=wl.scale_mode)
    opool.k.view(np.uint8)[...] = 0xFF
    opool.v.view(np.uint8)[...] = 0xFF
    opool.k_scale, opool.v_scale = wl.k_scale, wl.v_scale
    slots = oracle.slot_mapping(wl.block_table, wl.fill_seq[keep], wl.fill_pos[keep],
                                wl.block_size)
    oracle.kv_cache_write(opool, slots, wl.k_src[keep], wl.v_src[keep], wl.src_dtype)
    blocks = np.unique(np.concatenate([wl.block_table[s, :-(-int(wl.context_lens[s]) //
                                                             wl.block_size)] for s in seqs]))
    gk, gv = case.logical_pools()
    assert np.array_equal(gk[blocks].view(np.uint8), opool.k[blocks].view(np.uint8))
    assert np.array_equal(gv[blocks].view(np.uint8), opool.v[blocks].view(np.uint8))
    ref = oracle.paged_decode(wl.q, wl.q_dtype, opool, wl.block_table, wl.context_lens, wl.scale,
                              seqs=seqs)
    for P in (0, -1, 192):
        out = to_f64(case.decode(partition_size=P), wl.q_dtype)[seqs]
        print(assert_close(out, ref, "%s P=%d" % (wl.name, P)))


@pytest.mark.parametrize("which", ["llama3 small", "long small", "llama3 full", "edges B4",
                                   "edges B64"])
def test_planted_keys(which):
    """One written key per sequence, at a block edge deep in the context, with a large
    score and a distinctive V row: it must come through in every partition mode."""
    if which == "llama3 small":
        wl = W.llama3_8b_decode(small=True)
    elif which == "long small":
        wl = W.long_context_decode(small=True)
    elif which == "llama3 full":
        wl = W.llama3_8b_decode()
    else:
        B = 4 if which.endswith("B4") else 64
        wl = W.make_decode("planted " + which, 55 + B, ctx_range=(2, 1500), num_seqs=7, Hq=16,
                           Hkv=4, D=128, B=B, kv_dtype="f16", spare_frac=0.2)
    w2, pos = plant_keys(wl)
    assert (pos >= 0).sum() >= min(6, wl.num_seqs)
    seqs = None if wl.num_seqs <= 8 else np.array(
        [int(np.argmax(wl.context_lens)), int(np.argmin(wl.context_lens)), 7, 33], np.int32)
    print(_run(w2, [0, 64, 512, -1], seqs=seqs))


def test_shared_prefix_full_sampled():
    wl = W.shared_prefix_decode()
    seqs = np.array([0, 1, 100, 255] + [int(np.argmin(wl.context_lens))], np.int32)
    print(_run(wl, [0, 512, -1], seqs=seqs))


def test_8192_partitions():
    """64-token partitions with max_context_len = 8192 x 64, the most partitions the
    reduce takes: a grid of 8192 partition slices, nearly all empty; the plain decode
    and the fused step match the oracle."""
    import paged_kv_cache_146_amd as pkv
    from test_gpu_fused import _without_newest
    from helpers import torch_bits
    wl = W.make_decode("8192 partitions", 97, ctx_lens=[300, 5, 129, 0], Hq=4, Hkv=2, D=64,
                       B=16, kv_dtype="bf16")
    big = 8192 * 64
    case = GpuCase(wl)
    opool = oracle_pool(wl)
    ref = oracle.paged_decode(wl.q, wl.q_dtype, opool, wl.block_table, wl.context_lens, wl.scale)
    out = pkv.pkv_paged_attention_decode(case.q, case.desc, case.k_pool, case.v_pool,
                                         case.block_table, case.context_lens, big, wl.scale,
                                         partition_size=64, out=case.nan_out(),
                                         q_dtype=wl.q_dtype)
    print(assert_close(to_f64(out, wl.q_dtype), ref, "8192 partitions"))
    w2, rows = _without_newest(wl)
    c2 = GpuCase(w2)
    r = np.where(rows >= 0, rows, 0)
    out = pkv.pkv_decode_append(c2.q, c2.desc, c2.k_pool, c2.v_pool, c2.block_table,
                                c2.context_lens, big, torch_bits(wl.k_src[r], wl.src_dtype),
                                torch_bits(wl.v_src[r], wl.src_dtype), wl.scale,
                                partition_size=64, out=c2.nan_out())
    _check_pools(c2, opool)
    print(assert_close(to_f64(out, wl.q_dtype), ref, "8192 partitions, fused"))


def test_partition_size_from_the_device():
    """num_cus <= 0 asks the current device: the same choice as passing its CU count."""
    import torch
    import paged_kv_cache_146_amd as pkv
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ctx = np.random.default_rng(3).integers(32768, 131072 + 1, size=8)
    assert pkv.pkv_decode_partition_size(ctx, 8, 131072) == \
        pkv.pkv_decode_partition_size(ctx, 8, 131072, cus)


def test_sequence_order_invariance_bitwise():
    """Permuting the batch's sequences (q, table rows, lengths; the same slots) permutes
    the output bit for bit in the unsplit and fixed-partition modes: their workgroups take
    sequences by rank of context length, and each computes its (sequence, kv head,
    partition) the same way whatever the order (the balanced mode cuts the work by
    position in the batch, so only its values are order-free)."""
    import torch
    wl = W.make_decode("order", 92, ctx_range=(1, 900), num_seqs=9, Hq=16, Hkv=4, D=128, B=16,
                       kv_dtype="bf16", spare_frac=0.3)
    wl.context_lens = wl.context_lens.copy()
    wl.context_lens[[2, 5]] = wl.context_lens[7]  # ties in length
    a = GpuCase(wl)
    perm = np.random.default_rng(7).permutation(wl.num_seqs)
    inv = np.argsort(perm)
    wl2 = W.Workload(**{**wl.__dict__})
    wl2.q = wl.q[perm]
    wl2.block_table = np.ascontiguousarray(wl.block_table[perm])
    wl2.context_lens = np.ascontiguousarray(wl.context_lens[perm])
    wl2.fill_seq = inv[wl.fill_seq].astype(np.int32)
    b = GpuCase(wl2)
    for P in (0, 128):
        oa = a.decode(partition_size=P).cpu()
        ob = b.decode(partition_size=P).cpu()
        assert torch.equal(oa[torch.from_numpy(perm)].view(torch.int16), ob.view(torch.int16)), P
    ref = oracle.paged_decode(wl.q, wl.q_dtype, oracle_pool(wl), wl.block_table, wl.context_lens,
                              wl.scale)
    print(assert_close(to_f64(b.decode(partition_size=-1), wl.q_dtype), ref[perm], "balanced"))
