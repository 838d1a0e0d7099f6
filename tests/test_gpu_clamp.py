"""Contexts past what the call covers: context_lens above max_context_len, or above
the table's reach (max_blocks_per_seq * block_size).

The decode reads each sequence's first min(ctx, max_context_len, W * B) keys (the
clamp pagedkv.h documents), so the oracle is run on the clamped lengths.  The
fused step appends the newest token where the append would put it, at position
ctx - 1 of the UNclamped context ("03 | PagedAttention and the KV-cache memory
system" §4.1: the token's slot comes from the table; a position past the table
has no slot and is skipped), and must leave every other pool byte alone.  With
fixed partitions the split-KV workspace starts as NaN bytes, so a reduce that
merges a partition the decode never wrote fails the finiteness check.
"""
import numpy as np
import pytest

import oracle
from helpers import GpuCase, assert_close, oracle_pool, to_f64, torch_bits
import workloads as W

pytestmark = pytest.mark.gpu

CTX = [200, 50, 130, 0, 17, 64, 65, 255]


def _workload(W_cols):
    wl = W.make_decode("clamp", 321, ctx_lens=CTX, Hq=8, Hkv=2, D=128, B=16, kv_dtype="bf16",
                       spare_frac=0.2)
    if W_cols is not None:  # a table narrower than the contexts
        wl = W.Workload(**{**wl.__dict__})
        wl.block_table = np.ascontiguousarray(wl.block_table[:, :W_cols])
    return wl


def _nan_ws(nbytes):
    import torch
    return torch.full((max(16, nbytes),), 0xFF, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("W_cols,max_ctx", [(4, 256), (None, 100), (6, 90)])
@pytest.mark.parametrize("P", [64, 128, 0, -1])
def test_decode_clamped_contexts(W_cols, max_ctx, P):
    import paged_kv_cache_146_amd as pkv
    wl = _workload(W_cols)
    case = GpuCase(wl)  # tokens past the table get slot -1 and are not written
    cap = min(max_ctx, wl.max_blocks_per_seq * wl.block_size)
    clamped = np.minimum(wl.context_lens, cap).astype(np.int32)
    ref = oracle.paged_decode(wl.q, wl.q_dtype, oracle_pool(wl), wl.block_table, clamped,
                              wl.scale)
    ws = _nan_ws(pkv.pkv_decode_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads,
                                                wl.head_dim, max_ctx, P))
    for call in range(2):
        out = pkv.pkv_paged_attention_decode(case.q, case.desc, case.k_pool, case.v_pool,
                                             case.block_table, case.context_lens, max_ctx,
                                             wl.scale, partition_size=P, out=case.nan_out(),
                                             workspace=ws, q_dtype=wl.q_dtype)
        print(assert_close(to_f64(out, wl.q_dtype), ref, "W=%s max_ctx=%d P=%d call %d"
                           % (W_cols, max_ctx, P, call)))


@pytest.mark.parametrize("W_cols,max_ctx", [(4, 256), (None, 100), (6, 90), (None, 0)])
@pytest.mark.parametrize("P", [64, 128, 0, -1])
def test_fused_clamped_contexts(W_cols, max_ctx, P):
    """The fused step writes exactly the pool bytes of the append at ctx - 1 (nothing
    where the table has no entry) and decodes the clamped contexts."""
    import torch
    import paged_kv_cache_146_amd as pkv
    from test_gpu_fused import _without_newest
    wl = _workload(W_cols)
    w2, rows = _without_newest(wl)
    case = GpuCase(w2)
    r = np.where(rows >= 0, rows, 0)
    k_new = torch_bits(wl.k_src[r], wl.src_dtype)
    v_new = torch_bits(wl.v_src[r], wl.src_dtype)
    slots = torch.full((wl.num_seqs,), -7, dtype=torch.int64, device="cuda")
    ws = _nan_ws(pkv.pkv_decode_workspace_bytes(wl.num_seqs, wl.num_q_heads, wl.num_kv_heads,
                                                wl.head_dim, max_ctx, P))
    out = pkv.pkv_decode_append(case.q, case.desc, case.k_pool, case.v_pool, case.block_table,
                                case.context_lens, max_ctx, k_new, v_new, wl.scale,
                                partition_size=P, workspace=ws, out=case.nan_out(),
                                slot_mapping_out=slots)
    opool = oracle_pool(wl)  # the append of every token, the newest included
    gk, gv = case.logical_pools()
    assert np.array_equal(gk.view(np.uint8), opool.k.view(np.uint8)), "K pool differs"
    assert np.array_equal(gv.view(np.uint8), opool.v.view(np.uint8)), "V pool differs"
    want = oracle.slot_mapping(wl.block_table, np.arange(wl.num_seqs, dtype=np.int32),
                               wl.context_lens - 1, wl.block_size)
    got = slots.cpu().numpy()
    live = wl.context_lens > 0
    assert np.array_equal(got[live], want[live]), (got, want)
    assert np.all(got[~live] == -7)
    cap = min(max_ctx, wl.max_blocks_per_seq * wl.block_size)
    clamped = np.minimum(wl.context_lens, cap).astype(np.int32)
    ref = oracle.paged_decode(wl.q, wl.q_dtype, opool, wl.block_table, clamped, wl.scale)
    print(assert_close(to_f64(out, wl.q_dtype), ref, "fused W=%s max_ctx=%d P=%d"
                       % (W_cols, max_ctx, P)))
