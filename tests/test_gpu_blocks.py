"""GPU side of block ownership: pkv_copy_blocks, and fork / copy on write end to end.

"KV Cache: capacity, layout, lifecycle", "Reference counting and tail-block COW":
the committed K/V and scales of a shared tail block are copied before the new table
is used; "Lifecycle and ownership": a block goes back to the free list only after
its last GPU access.  Block copies are compared bit for bit with numpy copies of the
same bytes; the forked sequences' attention is compared with the oracle run on each
sequence's own logical history, written into a pool of its own.
"""
import numpy as np
import pytest

import oracle
from helpers import assert_close, to_f64, torch_bits
from workloads import to_storage

pytestmark = pytest.mark.gpu


def _pkv():
    import paged_kv_cache_146_amd as pkv
    return pkv


@pytest.mark.parametrize("kv,mode", [("bf16", "block"), ("fp8", "block"), ("int8", "token"),
                                     ("fp8", "tensor")])
def test_copy_blocks_bit_exact(kv, mode):
    import torch
    pkv = _pkv()
    NB, B, H, D = 24, 16, 4, 128
    desc = pkv.pool_desc(NB, B, H, D, kv, mode)
    kp, vp = pkv.alloc_pool(desc)
    g = torch.Generator(device="cuda").manual_seed(5)
    kp.copy_(torch.randint(0, 256, kp.shape, dtype=torch.uint8, device="cuda", generator=g))
    vp.copy_(torch.randint(0, 256, vp.shape, dtype=torch.uint8, device="cuda", generator=g))
    shape = {"block": (NB, H), "tensor": (1,), "token": (NB, H, B)}[mode]
    quant = kv in ("fp8", "int8")
    ks = torch.rand(shape, device="cuda", generator=g) if quant else None
    vs = torch.rand(shape, device="cuda", generator=g) if quant else None
    pairs = [(3, 10), (5, 11), (7, 7), (-1, 2), (4, NB), (20, 0)]
    want_k = kp.cpu().numpy().reshape(NB, -1).copy()
    want_v = vp.cpu().numpy().reshape(NB, -1).copy()
    want_ks = ks.cpu().numpy().copy() if ks is not None else None
    want_vs = vs.cpu().numpy().copy() if vs is not None else None
    # one scale for the whole pool belongs to no block: it is left as it is
    per_block = quant and mode != "tensor"
    oracle.copy_blocks(want_k, want_v, want_ks if per_block else None,
                       want_vs if per_block else None, pairs)
    pkv.pkv_copy_blocks(torch.tensor(pairs, dtype=torch.int32, device="cuda"), desc, kp, vp,
                        ks, vs)
    assert np.array_equal(kp.cpu().numpy().reshape(NB, -1), want_k)
    assert np.array_equal(vp.cpu().numpy().reshape(NB, -1), want_v)
    if ks is not None:
        assert np.array_equal(ks.cpu().numpy(), want_ks)
        assert np.array_equal(vs.cpu().numpy(), want_vs)


def test_fork_copy_on_write_decode():
    # A parent of 37 tokens (tail block 5/16 full) is forked three times.  Two
    # children append their own tokens (the first append copies the shared tail);
    # the third never writes, so when the parent appends afterwards its tail is
    # still shared and the parent copies it.  Every sequence must then attend to
    # exactly its own history.
    import torch
    pkv = _pkv()
    rng = np.random.default_rng(11)
    NB, B, Hkv, G, D = 40, 16, 2, 4, 128
    Hq = Hkv * G
    desc = pkv.pool_desc(NB, B, Hkv, D, "bf16")
    kp, vp = pkv.alloc_pool(desc, fill_byte=0xFF)
    alloc = pkv.BlockAllocator(NB, B)
    hist = {}  # sequence -> list of (k, v) token rows (bf16 bits)

    def new_token():
        x = rng.standard_normal((2, 1, Hkv, D)).astype(np.float32)
        return to_storage(x[0], "bf16"), to_storage(x[1], "bf16")

    def append(seq, k, v):
        slot, src, dst = alloc.append(seq)
        if src >= 0:
            pkv.pkv_copy_blocks(torch.tensor([[src, dst]], dtype=torch.int32, device="cuda"),
                                desc, kp, vp)
        pkv.pkv_kv_cache_write(torch.tensor([slot], dtype=torch.int64, device="cuda"),
                               torch_bits(k, "bf16"), torch_bits(v, "bf16"), desc, kp, vp)
        hist.setdefault(seq, []).append((k, v))
        return src >= 0

    parent = alloc.add_seq()
    for _ in range(37):
        append(parent, *new_token())
    children = [alloc.fork(parent) for _ in range(3)]
    for c in children:
        hist[c] = list(hist[parent])
    copies = []
    for c, n in zip(children[:2], (12, 30)):
        copies.append([append(c, *new_token()) for _ in range(n)])
    copies.append([append(parent, *new_token()) for _ in range(2)])
    assert copies[0][0] and copies[1][0] and copies[2][0], "each first write copies the tail"
    assert not any(copies[0][1:]) and not any(copies[1][1:]) and not copies[2][1]
    seqs = [parent] + children
    tables = [alloc.table(s) for s in seqs]
    assert [t[1] for t in tables] == [len(hist[s]) for s in seqs] == [39, 49, 67, 37]
    assert alloc.refcount(tables[0][0][0]) == 4  # the full prefix blocks stay shared

    W = max(len(t[0]) for t in tables)
    bt = np.zeros((len(seqs), W), np.int32)
    for i, (t, _) in enumerate(tables):
        bt[i, :len(t)] = t
    ctx = np.array([t[1] for t in tables], np.int32)
    q = to_storage(rng.standard_normal((len(seqs), Hq, D)).astype(np.float32), "bf16")
    # the oracle: each sequence's history in a pool of its own, through a plain table
    nblk = [-(-len(hist[s]) // B) for s in seqs]
    opool = oracle.Pool(sum(nblk) + 1, B, Hkv, D, "bf16")
    obt = np.zeros((len(seqs), max(nblk)), np.int32)
    base = 0
    for i, s in enumerate(seqs):
        obt[i, :nblk[i]] = np.arange(base, base + nblk[i])
        rows = hist[s]
        k = np.concatenate([r[0] for r in rows])
        v = np.concatenate([r[1] for r in rows])
        oracle.kv_cache_write(opool, base * B + np.arange(len(rows)), k, v, "bf16")
        base += nblk[i]
    ref = oracle.paged_decode(q, "bf16", opool, obt, ctx, 1.0 / np.sqrt(D))
    qd = torch_bits(q, "bf16")
    for P in (0, -1):
        out = torch.empty_like(qd)
        out.view(torch.uint8).fill_(0xFF)
        pkv.pkv_paged_attention_decode(qd, desc, kp, vp, torch.from_numpy(bt).cuda(),
                                       torch.from_numpy(ctx).cuda(), int(ctx.max()),
                                       1.0 / np.sqrt(D), partition_size=P, out=out)
        print(assert_close(to_f64(out, "bf16"), ref, "fork/cow P=%d" % P))
    for s in seqs:
        alloc.free_seq(s)
    assert sorted(alloc.free_blocks()) == list(range(NB))


def test_deferred_release_waits_for_the_event():
    import torch
    pkv = _pkv()
    alloc = pkv.BlockAllocator(8, 4)
    s = alloc.add_seq()
    for _ in range(5):
        alloc.append(s)  # blocks 0 and 1
    torch.cuda.synchronize()
    torch.cuda._sleep(1 << 30)  # a bounded spin that keeps the stream busy for a while
    ev = torch.cuda.Event()
    ev.record()
    alloc.free_seq(s, ev)
    pending = alloc.free_blocks()
    torch.cuda.synchronize()
    done = alloc.free_blocks()
    assert 0 not in pending and 1 not in pending, "released before the GPU work finished"
    assert done[-2:] == [1, 0]  # reverse table order: block 0 is handed out next
