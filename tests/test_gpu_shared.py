"""GPU parity of the shared-prefix decode (pkv_paged_attention_decode_shared) against
the oracle's paged decode: the same function, computed with the shared blocks read
once per kv head.  The prefix runs on the matrix-core prefill kernel for bf16, f16
and fp8-block pools with G dividing 16 and blocks of 16 tokens or more, on the decode
tiles otherwise; the grid below covers both.

"03 | PagedAttention and the KV-cache memory system" §5 (requests that hit the same
prefix pages point their tables at the same physical blocks); "PagedAttention 的原理是
什么？它如何降低 KV Cache 的内存浪费？", section 4 (block-level sharing).  Tolerance
|gpu - oracle| <= 2e-3 + 1e-2 |oracle| per element; pools and outputs start as NaN
bytes, so a read of an unwritten slot or an output left unwritten fails.
"""
import numpy as np
import pytest

import oracle
from helpers import GpuCase, assert_close, oracle_pool, to_f64
import workloads as W

pytestmark = pytest.mark.gpu


def _pkv():
    import paged_kv_cache_146_amd as pkv
    return pkv


def _shared(case, shared_len, workspace=None):
    wl = case.wl
    return _pkv().pkv_paged_attention_decode_shared(
        case.q, case.desc, case.k_pool, case.v_pool, case.block_table, case.context_lens,
        wl.max_context_len, wl.scale, shared_len, k_scale=case.k_scale, v_scale=case.v_scale,
        out=case.nan_out(), q_dtype=wl.q_dtype, workspace=workspace)


def _check(wl, shared_lens, case=None):
    case = case or GpuCase(wl)
    ref = oracle.paged_decode(wl.q, wl.q_dtype, oracle_pool(wl), wl.block_table,
                              wl.context_lens, wl.scale)
    res = {}
    for sl in shared_lens:
        out = to_f64(_shared(case, sl), wl.q_dtype)
        res[sl] = assert_close(out, ref, "%s shared_len=%d" % (wl.name, sl))
    return res


def test_shared_prefix_config_small():
    """The MHA shared-prefix workload (fp16, B 32, H 32/32), reduced: the whole prefix,
    part of it, and none of it declared shared."""
    wl = W.shared_prefix_decode(small=True)
    print(_check(wl, [256, 64, 0]))


@pytest.mark.parametrize("kv,Hq,Hkv,D,B,prefix,S,mode", [
    ("bf16", 32, 8, 128, 16, 320, 37, "block"),   # G 4: 4 sequences per tile, ragged tiles
    ("f16", 6, 2, 64, 16, 192, 11, "block"),      # G 3: 5 sequences per tile, one dead column
    ("bf16", 16, 1, 128, 32, 1024, 6, "block"),   # G 16: one sequence per tile
    ("fp8", 16, 2, 128, 16, 512, 9, "token"),     # per-token scales, NaN in unwritten slots
    ("int8", 8, 8, 64, 64, 448, 20, "block"),     # MHA, int8, B 64
    ("bf16", 8, 2, 64, 4, 96, 5, "block"),        # B 4: tokens look up their own blocks
    ("f32", 4, 2, 64, 8, 40, 3, "block"),         # f32 pool, prefix of 40 tokens
    ("fp8", 16, 2, 128, 16, 512, 9, "block"),     # G 8, fp8 block scales
    ("f16", 8, 4, 64, 64, 640, 13, "block"),      # G 2, B 64, D 64
    ("f16", 4, 4, 128, 32, 384, 150, "block"),    # MHA, 150 sequences: two ragged row blocks
])
def test_shared_prefix_grid(kv, Hq, Hkv, D, B, prefix, S, mode):
    q_dtype = "bf16" if kv in ("fp8", "int8") else kv
    wl = W.make_decode("shared %s G%d B%d" % (kv, Hq // Hkv, B), 300 + Hq + B + S,
                       num_seqs=S, Hq=Hq, Hkv=Hkv, D=D, B=B, kv_dtype=kv, q_dtype=q_dtype,
                       shared_prefix=prefix, tail_range=(0, 200), spare_frac=0.1,
                       scale_mode=mode)
    print(_check(wl, [prefix, prefix - B if prefix > B else prefix]))


def test_contexts_shorter_than_the_prefix():
    """Sequences whose context ends inside the shared prefix (including 0 and exactly
    shared_len) see only their own first ctx tokens; the tails of the others still count."""
    wl = W.make_decode("short contexts", 91, num_seqs=12, Hq=16, Hkv=4, D=128, B=16,
                       kv_dtype="bf16", shared_prefix=256, tail_range=(1, 150))
    wl.context_lens = wl.context_lens.copy()
    wl.context_lens[[0, 3, 5, 7, 8]] = [1, 100, 0, 256, 255]
    case = GpuCase(wl)
    print(_check(wl, [256, 128], case=case))


def test_prefix_slots_past_every_context_unwritten():
    """Every context ends inside the shared prefix (the longest at 200 of 256 tokens), and
    only the prefix tokens below 200 were ever written: the slots from 200 on hold NaN
    bytes, which no sequence may read."""
    wl = W.make_decode("unwritten prefix tail", 97, num_seqs=40, Hq=16, Hkv=4, D=128, B=16,
                       kv_dtype="bf16", shared_prefix=256, tail_range=(0, 30))
    rng = np.random.default_rng(3)
    ctx = rng.integers(1, 201, size=wl.num_seqs).astype(np.int32)
    ctx[5] = 200
    keep = wl.fill_pos < 200  # the prefix is stored under sequence 0; every tail dropped
    wl.context_lens = ctx
    wl.fill_seq, wl.fill_pos = wl.fill_seq[keep], wl.fill_pos[keep]
    wl.k_src, wl.v_src = wl.k_src[keep], wl.v_src[keep]
    print(_check(wl, [256, 128]))


def test_contexts_inside_an_unaligned_prefix_tile():
    """B 4 and declared shared lengths that are not multiples of 16 (92, 84): contexts
    that end inside the last 16-token tile before the shared length (81, 85, 90) have
    an empty tail, as do 92 and 0."""
    wl = W.make_decode("unaligned shared length", 93, num_seqs=10, Hq=8, Hkv=2, D=64, B=4,
                       kv_dtype="bf16", shared_prefix=96, tail_range=(1, 80))
    wl.context_lens = wl.context_lens.copy()
    wl.context_lens[[0, 1, 2, 3, 4, 5]] = [81, 85, 90, 92, 84, 0]
    case = GpuCase(wl)
    print(_check(wl, [92, 84], case=case))


def test_long_prefix_many_slices_and_workspace_reuse():
    """A 4096-token prefix over 24 sequences (several prefix slices), twice in a row on a
    workspace filled with garbage, and against the plain balanced decode."""
    import torch
    pkv = _pkv()
    wl = W.make_decode("long prefix", 17, num_seqs=24, Hq=32, Hkv=8, D=128, B=16,
                       kv_dtype="bf16", shared_prefix=4096, tail_range=(0, 700))
    case = GpuCase(wl)
    ref = oracle.paged_decode(wl.q, wl.q_dtype, oracle_pool(wl), wl.block_table,
                              wl.context_lens, wl.scale)
    need = pkv.pkv_decode_shared_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads,
                                                 wl.head_dim, 4096)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for r in range(2):
        out = to_f64(_shared(case, 4096, workspace=ws), wl.q_dtype)
        print(assert_close(out, ref, "call %d" % r))
    plain = to_f64(case.decode(partition_size=-1), wl.q_dtype)
    print(assert_close(plain, ref, "plain balanced"))


def test_shared_argument_errors():
    import torch
    pkv = _pkv()
    wl = W.make_decode("errors", 5, num_seqs=2, Hq=4, Hkv=2, D=64, B=16, kv_dtype="bf16",
                       shared_prefix=32, tail_range=(0, 10))
    case = GpuCase(wl)
    for bad in (8, -16, 16 * (wl.max_blocks_per_seq + 1)):  # not a multiple of B, < 0, past the table
        with pytest.raises(pkv.PagedKVError) as e:
            _shared(case, bad)
        assert e.value.status == -1
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PagedKVError) as e:
        _shared(case, 32, workspace=small)
    assert e.value.status == -4


def test_shared_prefix_config_full():
    """The full shared-prefix configuration (256 sequences sharing a 2048-token prefix,
    private tails U[0, 512], MHA fp16, B 32) in bench.py's launch: the shared decode
    against the oracle's plain decode on sampled sequences (the longest and shortest
    tails among them), pool written bit for bit."""
    wl = W.shared_prefix_decode()
    case = GpuCase(wl)
    opool = oracle_pool(wl)
    gk, gv = case.logical_pools()
    assert np.array_equal(gk.view(np.uint8), opool.k.view(np.uint8)), "K pool differs"
    assert np.array_equal(gv.view(np.uint8), opool.v.view(np.uint8)), "V pool differs"
    seqs = np.array(sorted({0, 1, 100, 255, int(np.argmin(wl.context_lens)),
                            int(np.argmax(wl.context_lens))}), np.int32)
    ref = oracle.paged_decode(wl.q, wl.q_dtype, opool, wl.block_table, wl.context_lens,
                              wl.scale, seqs=seqs)
    shared_len = wl.shared_blocks * wl.block_size
    assert shared_len == 2048
    for call in range(2):  # the same workspace twice
        out = to_f64(_shared(case, shared_len), wl.q_dtype)[seqs]
        print(assert_close(out, ref, "%s shared decode, call %d" % (wl.name, call)))
