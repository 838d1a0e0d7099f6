"""Pools with a block stride: one allocation holding every layer's K and V of a block
together ("03 | PagedAttention and the KV-cache memory system", §3.1: a cross-layer
block groups layer, K and V for transfer in larger units; all layers share the block
ids).  Layout [block][layer][K|V][kv head][page]; layer l's pools start at its K / V
pages of block 0 and the stride is the whole block.

Each layer is written through the library's write path with its own data; every
layer's bytes must then equal the oracle's write of that layer alone (bit-exact, so
no call touches another layer's bytes), and decode / prefill / block copies on one
layer must match the oracle for that layer.
"""
import numpy as np
import pytest

import oracle
from helpers import assert_close, logical_k, logical_v, oracle_pool, to_f64, torch_bits
import workloads as W

pytestmark = pytest.mark.gpu
L = 3


def _pkv():
    import paged_kv_cache_146_amd as pkv
    return pkv


class CrossLayer:
    """L layers of one workload shape in a single cross-layer allocation."""

    def __init__(self, wls):
        import torch
        pkv = _pkv()
        w = wls[0]
        self.wls = wls
        self.es = W.ELEM_BYTES[w.kv_dtype]
        self.dense = w.num_kv_heads * w.block_size * w.head_dim * self.es  # one pool's block
        self.stride = L * 2 * self.dense
        self.buf = torch.full((w.num_blocks * self.stride,), 0xFF, dtype=torch.uint8,
                              device="cuda")
        self.desc = pkv.pool_desc(w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim,
                                  w.kv_dtype, w.scale_mode, block_stride=self.stride)
        self.bt = torch.from_numpy(w.block_table).cuda()
        self.cl = torch.from_numpy(w.context_lens).cuda()
        self.scales = []
        for l, wl in enumerate(wls):
            k, v = self.pools(l)
            ks = torch.from_numpy(wl.k_scale).cuda() if wl.k_scale is not None else None
            vs = torch.from_numpy(wl.v_scale).cuda() if wl.v_scale is not None else None
            self.scales.append((ks, vs))
            seq = torch.from_numpy(wl.fill_seq).cuda()
            pos = torch.from_numpy(wl.fill_pos).cuda()
            slots = pkv.pkv_slot_mapping(self.bt, seq, pos, wl.block_size)
            pkv.pkv_kv_cache_write(slots, torch_bits(wl.k_src, wl.src_dtype),
                                   torch_bits(wl.v_src, wl.src_dtype), self.desc, k, v, ks, vs,
                                   src_dtype=wl.src_dtype)
        torch.cuda.synchronize()

    def pools(self, l):
        return self.buf[(2 * l) * self.dense:], self.buf[(2 * l + 1) * self.dense:]

    def logical(self, l):
        w = self.wls[0]
        raw = self.buf.cpu().numpy().reshape(w.num_blocks, L, 2, self.dense)
        args = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim, w.kv_dtype)
        return (logical_k(np.ascontiguousarray(raw[:, l, 0]), *args),
                logical_v(np.ascontiguousarray(raw[:, l, 1]), *args))


def _layers(kv, B, Hq, Hkv, D, mode="block", seed=900):
    base = W.make_decode("cross-layer %s B%d" % (kv, B), seed, ctx_range=(1, 700), num_seqs=6,
                         Hq=Hq, Hkv=Hkv, D=D, B=B, kv_dtype=kv, spare_frac=0.2, scale_mode=mode)
    wls = [base]
    rng = np.random.default_rng(seed + 1)
    for _ in range(1, L):  # same tables and queries, other K/V
        wl = W.Workload(**{**base.__dict__})
        wl.k_src, wl.v_src = W._draw_kv(rng, len(base.fill_seq), Hkv, D, base.src_dtype)
        if kv in W.QUANTISED:
            wl.k_scale, wl.v_scale = W.amax_scales(wl)
        wls.append(wl)
    return wls


@pytest.mark.parametrize("kv,B,Hq,Hkv,D,mode", [
    ("bf16", 16, 8, 2, 128, "block"), ("fp8", 32, 16, 4, 128, "token"), ("f16", 4, 4, 4, 64, "block")])
def test_cross_layer_write_and_decode(kv, B, Hq, Hkv, D, mode):
    pkv = _pkv()
    wls = _layers(kv, B, Hq, Hkv, D, mode)
    cl = CrossLayer(wls)
    opools = [oracle_pool(wl) for wl in wls]
    for l in range(L):
        gk, gv = cl.logical(l)
        assert np.array_equal(gk.view(np.uint8), opools[l].k.view(np.uint8)), "layer %d K" % l
        assert np.array_equal(gv.view(np.uint8), opools[l].v.view(np.uint8)), "layer %d V" % l
    l = 1
    wl = wls[l]
    ref = oracle.paged_decode(wl.q, wl.q_dtype, opools[l], wl.block_table, wl.context_lens,
                              wl.scale)
    k, v = cl.pools(l)
    ks, vs = cl.scales[l]
    q = torch_bits(wl.q, wl.q_dtype)
    for P in (0, 64, -1):
        out = pkv.pkv_paged_attention_decode(q, cl.desc, k, v, cl.bt, cl.cl, wl.max_context_len,
                                             wl.scale, partition_size=P, k_scale=ks, v_scale=vs,
                                             q_dtype=wl.q_dtype)
        print(assert_close(to_f64(out, wl.q_dtype), ref, "layer 1 P=%d" % P))
    wref = oracle.paged_decode(wl.q, wl.q_dtype, opools[l], wl.block_table, wl.context_lens,
                               wl.scale, window=100)
    out = pkv.pkv_paged_attention_decode_window(q, cl.desc, k, v, cl.bt, cl.cl,
                                                wl.max_context_len, wl.scale, 100,
                                                partition_size=-1, k_scale=ks, v_scale=vs,
                                                q_dtype=wl.q_dtype)
    print(assert_close(to_f64(out, wl.q_dtype), wref, "layer 1 window"))


def test_cross_layer_block_copy_touches_one_layer():
    import torch
    pkv = _pkv()
    wls = _layers("bf16", 16, 8, 2, 64)
    cl = CrossLayer(wls)
    nb = wls[0].num_blocks
    before = cl.buf.cpu().numpy().reshape(nb, L, 2, cl.dense).copy()
    pairs = [(3, 9), (0, 5), (7, 7), (-1, 2)]
    k, v = cl.pools(2)
    pkv.pkv_copy_blocks(torch.tensor(pairs, dtype=torch.int32, device="cuda"), cl.desc, k, v)
    after = cl.buf.cpu().numpy().reshape(nb, L, 2, cl.dense)
    want = before.copy()
    oracle.copy_blocks(want[:, 2, 0], want[:, 2, 1], None, None, pairs)
    assert np.array_equal(after, want)


def test_cross_layer_prefill():
    pkv = _pkv()
    base = W.fp8_chunked_prefill(small=True)
    wls = [base]
    rng = np.random.default_rng(5)
    for _ in range(1, L):
        wl = W.Workload(**{**base.__dict__})
        wl.k_src, wl.v_src = W._draw_kv(rng, len(base.fill_seq), base.num_kv_heads,
                                        base.head_dim, base.src_dtype)
        wl.k_scale, wl.v_scale = W.amax_scales(wl)
        wls.append(wl)
    cl = CrossLayer(wls)
    import torch
    wl = wls[2]
    ref = oracle.paged_prefill(wl.q, wl.q_dtype, wl.cu_seqlens_q, oracle_pool(wl), wl.block_table,
                               wl.context_lens, wl.scale)
    k, v = cl.pools(2)
    ks, vs = cl.scales[2]
    nq = np.diff(wl.cu_seqlens_q)
    out = pkv.pkv_paged_prefill(torch_bits(wl.q, wl.q_dtype), torch.from_numpy(wl.cu_seqlens_q).cuda(),
                                int(nq.max()), cl.desc, k, v, cl.bt, cl.cl, wl.max_context_len,
                                wl.scale, k_scale=ks, v_scale=vs, q_dtype=wl.q_dtype)
    print(assert_close(to_f64(out, wl.q_dtype), ref, "prefill layer 2"))
