"""Python face of the CPU oracle (``oracle.c``) — TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg import this package.  The product library never does, and this package never
imports the product: the two meet only in the tests, on inputs from the seeded
generators.

Arrays are numpy.  Storage types are passed as their bit patterns: ``float32``
for f32, ``uint16`` for f16 and bf16, ``uint8`` for fp8 (OCP E4M3).  Results are
``float64``.

Every function restates a passage of the pages (see ``oracle.h`` for the page
list); the pins that check each of them live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "fp8": 3, "int8": 4}
_NP_STORAGE = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8,
               "int8": np.int8}
# where a quantised element's scale lives: [block][head], one for the tensor, [block][head][token]
SCALE_MODES = {"block": 0, "tensor": 1, "token": 2}

ORC_OK, ORC_EVALUE, ORC_EINDEX = 0, 1, 2


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc (scalar C, OpenMP, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h"))
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Pool(ctypes.Structure):
    _fields_ = [
        ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p),
        ("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int64),
        ("num_kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int), ("scale_mode", ctypes.c_int),
    ]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            P, I64, I32, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
            sig = {
                "orc_physical_slot": (I32, [P, I64, I64, I64, P]),
                "orc_slot_mapping": (None, [P, I64, I64, P, P, I64, I64, P]),
                "orc_f16_decode": (D, [ctypes.c_uint16]),
                "orc_bf16_decode": (D, [ctypes.c_uint16]),
                "orc_e4m3_decode": (D, [ctypes.c_uint8]),
                "orc_e4m3_encode": (ctypes.c_uint8, [ctypes.c_float]),
                "orc_decode_n": (None, [P, I32, I64, P]),
                "orc_e4m3_encode_n": (None, [P, I64, P]),
                "orc_int8_encode_n": (None, [P, I64, P]),
                "orc_kv_cache_write": (I32, [P, I64, P, P, I32, I64, I64, I64, I64, I32, P, P, P, P,
                                              I32]),
                "orc_paged_decode": (I32, [P, I32, I64, I64, P, P, I64, P, D, I64, P, I64, P,
                                           P]),
                "orc_decode_partials": (I32, [P, I32, I64, I64, P, P, I64, P, D, I64, I64, P, P, P]),
                "orc_state_merge": (None, [D, D, P, D, D, P, I64, P, P, P]),
                "orc_split_reduce": (None, [P, P, P, P, I64, I64, I64, I64, I64, P]),
                "orc_paged_prefill": (I32, [P, I32, P, I64, I64, P, P, I64, P, D, I32, P, I64, P]),
                "orc_num_threads": (I32, []),
                "orc_set_num_threads": (None, [I32]),
            }
            for name, (res, args) in sig.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads of the oracle's OpenMP loops from now on (timing only)."""
    _load().orc_set_num_threads(int(n))


# --------------------------------------------------------------------------------------
# Addressing  [P2 "Page-table addressing"], [P1 §3, §4.1]
# --------------------------------------------------------------------------------------
def physical_slot(block_table, block_size: int, token_pos: int) -> int:
    """The page's ``physical_slot``: raises ValueError / IndexError as it does."""
    t = _c(block_table, np.int32)
    out = ctypes.c_int64(0)
    rc = _load().orc_physical_slot(_ptr(t), len(t), int(block_size), int(token_pos),
                                   ctypes.byref(out))
    if rc == ORC_EVALUE:
        raise ValueError("invalid block size, token position or physical block id")
    if rc == ORC_EINDEX:
        raise IndexError("logical block is not allocated")
    return int(out.value)


def slot_mapping(block_table, seq_idx, positions, block_size: int):
    bt = _c(block_table, np.int32)
    si, pos = _c(seq_idx, np.int32), _c(positions, np.int32)
    out = np.empty(len(si), np.int64)
    _load().orc_slot_mapping(_ptr(bt), bt.shape[0], bt.shape[1], _ptr(si), _ptr(pos), len(si),
                             int(block_size), _ptr(out))
    return out


# --------------------------------------------------------------------------------------
# Storage codecs
# --------------------------------------------------------------------------------------
def decode(bits, dtype: str):
    """Exact float64 values of storage bit patterns."""
    a = _c(bits, _NP_STORAGE[dtype])
    out = np.empty(a.size, np.float64)
    _load().orc_decode_n(_ptr(a), DTYPES[dtype], a.size, _ptr(out))
    return out.reshape(a.shape)


def e4m3_encode(x):
    a = _c(x, np.float32)
    out = np.empty(a.size, np.uint8)
    _load().orc_e4m3_encode_n(_ptr(a), a.size, _ptr(out))
    return out.reshape(a.shape)


def int8_encode(x):
    """symmetric int8 codes of float32 x (already divided by the scale)"""
    a = np.ascontiguousarray(x, np.float32)
    out = np.empty(a.shape, np.int8)
    _load().orc_int8_encode_n(_ptr(a), a.size, _ptr(out))
    return out


# --------------------------------------------------------------------------------------
# Pools
# --------------------------------------------------------------------------------------
class Pool:
    """Logical paged pool: K and V as [num_blocks][num_kv_heads][block_size][head_dim]."""

    def __init__(self, num_blocks, block_size, num_kv_heads, head_dim, kv_dtype, fill_bits=None,
                 scale_mode="block"):
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)
        self.num_kv_heads, self.head_dim = int(num_kv_heads), int(head_dim)
        self.kv_dtype = kv_dtype
        shape = (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)
        st = _NP_STORAGE[kv_dtype]
        if fill_bits is None:
            self.k = np.zeros(shape, st)
            self.v = np.zeros(shape, st)
        else:
            self.k = np.full(shape, fill_bits, st)
            self.v = np.full(shape, fill_bits, st)
        self.k_scale = None
        self.v_scale = None
        self.scale_mode = scale_mode

    def scale_shape(self):
        """shape of one scale array of a quantised pool in its scale mode"""
        return {"block": (self.num_blocks, self.num_kv_heads), "tensor": (1,),
                "token": (self.num_blocks, self.num_kv_heads, self.block_size)}[self.scale_mode]

    def _struct(self):
        s = _Pool()
        s.k_pool, s.v_pool = _ptr(self.k), _ptr(self.v)
        s.k_scale = _ptr(self.k_scale) if self.k_scale is not None else None
        s.v_scale = _ptr(self.v_scale) if self.v_scale is not None else None
        s.num_blocks, s.block_size = self.num_blocks, self.block_size
        s.num_kv_heads, s.head_dim = self.num_kv_heads, self.head_dim
        s.kv_dtype = DTYPES[self.kv_dtype]
        s.scale_mode = SCALE_MODES[self.scale_mode]
        return s


def kv_cache_write(pool: Pool, slots, k, v, src_dtype: str):
    """[P1 §4.1, §8.1] scatter k, v [T][H_kv][D] (storage bits of src_dtype) into pool."""
    sl = _c(slots, np.int64)
    k = _c(k, _NP_STORAGE[src_dtype])
    v = _c(v, _NP_STORAGE[src_dtype])
    ks = _c(pool.k_scale, np.float32) if pool.k_scale is not None else None
    vs = _c(pool.v_scale, np.float32) if pool.v_scale is not None else None
    rc = _load().orc_kv_cache_write(_ptr(sl), len(sl), _ptr(k), _ptr(v), DTYPES[src_dtype],
                                    pool.num_blocks, pool.block_size, pool.num_kv_heads,
                                    pool.head_dim, DTYPES[pool.kv_dtype], _ptr(pool.k),
                                    _ptr(pool.v), _ptr(ks), _ptr(vs),
                                    SCALE_MODES[pool.scale_mode])
    if rc != 0:
        raise ValueError("unsupported type combination for the cache write")


# --------------------------------------------------------------------------------------
# Attention  [P1 §4], [P3 §5]
# --------------------------------------------------------------------------------------
def paged_decode(q, q_dtype: str, pool: Pool, block_table, context_lens, scale: float,
                 seqs=None, return_lse: bool = False, window: int = 0):
    """window > 0: sliding-window decode ([P1 §1.1, §7]), keys [ctx - window, ctx) only."""
    q = _c(q, _NP_STORAGE[q_dtype])
    S, Hq, D = q.shape
    bt = _c(block_table, np.int32)
    cl = _c(context_lens, np.int32)
    sel = None if seqs is None else _c(seqs, np.int32)
    n = S if sel is None else len(sel)
    out = np.empty((n, Hq, D), np.float64)
    lse = np.empty((n, Hq), np.float64) if return_lse else None
    st = pool._struct()
    rc = _load().orc_paged_decode(_ptr(q), DTYPES[q_dtype], S, Hq, ctypes.byref(st), _ptr(bt),
                                  bt.shape[1], _ptr(cl), float(scale), int(window), _ptr(sel),
                                  n, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("invalid decode arguments")
    return (out, lse) if return_lse else out


def decode_partials(q, q_dtype: str, pool: Pool, block_table, context_lens, scale: float,
                    partition_size: int, max_partitions: int):
    q = _c(q, _NP_STORAGE[q_dtype])
    S, Hq, D = q.shape
    bt = _c(block_table, np.int32)
    cl = _c(context_lens, np.int32)
    po = np.empty((S, Hq, max_partitions, D), np.float64)
    pm = np.empty((S, Hq, max_partitions), np.float64)
    ps = np.empty((S, Hq, max_partitions), np.float64)
    st = pool._struct()
    rc = _load().orc_decode_partials(_ptr(q), DTYPES[q_dtype], S, Hq, ctypes.byref(st), _ptr(bt),
                                     bt.shape[1], _ptr(cl), float(scale), int(partition_size),
                                     int(max_partitions), _ptr(po), _ptr(pm), _ptr(ps))
    if rc != 0:
        raise ValueError("invalid partition arguments")
    return po, pm, ps


def state_merge(s1, s2):
    """Merge two states (m, l, acc) with acc the unnormalised weighted value sum."""
    m1, l1, a1 = s1
    m2, l2, a2 = s2
    a1, a2 = _c(a1, np.float64), _c(a2, np.float64)
    acc = np.empty_like(a1)
    m, l = ctypes.c_double(0), ctypes.c_double(0)
    _load().orc_state_merge(float(m1), float(l1), _ptr(a1), float(m2), float(l2), _ptr(a2),
                            a1.size, ctypes.byref(m), ctypes.byref(l), _ptr(acc))
    return m.value, l.value, acc


def split_reduce(part_out, part_max, part_sum, context_lens, partition_size: int):
    po = _c(part_out, np.float64)
    pm, ps = _c(part_max, np.float64), _c(part_sum, np.float64)
    cl = _c(context_lens, np.int32)
    S, Hq, P, D = po.shape
    out = np.empty((S, Hq, D), np.float64)
    _load().orc_split_reduce(_ptr(po), _ptr(pm), _ptr(ps), _ptr(cl), S, Hq, D,
                             int(partition_size), P, _ptr(out))
    return out


def paged_prefill(q, q_dtype: str, cu_seqlens_q, pool: Pool, block_table, context_lens,
                  scale: float, causal: bool = True, rows=None):
    q = _c(q, _NP_STORAGE[q_dtype])
    T, Hq, D = q.shape
    cu = _c(cu_seqlens_q, np.int32)
    bt = _c(block_table, np.int32)
    cl = _c(context_lens, np.int32)
    r = None if rows is None else _c(rows, np.int64)
    n = T if r is None else len(r)
    out = np.empty((n, Hq, D), np.float64)
    st = pool._struct()
    rc = _load().orc_paged_prefill(_ptr(q), DTYPES[q_dtype], _ptr(cu), len(cu) - 1, Hq,
                                   ctypes.byref(st), _ptr(bt), bt.shape[1], _ptr(cl),
                                   float(scale), int(bool(causal)), _ptr(r), n, _ptr(out))
    if rc != 0:
        raise ValueError("invalid prefill arguments")
    return out


def copy_blocks(k_pool, v_pool, k_scale, v_scale, pairs):
    """["KV Cache: capacity, layout, lifecycle", "Reference counting and tail-block COW"]
    copy on write copies the old tail block's committed K/V and its quantisation scales.
    Here every byte of block src goes to block dst, in place, pair by pair; pairs with
    an id outside the pool, or src == dst, are skipped.  k_pool, v_pool: numpy arrays
    whose first axis is the block; k_scale, v_scale: arrays whose first axis is the
    block ([num_blocks][H_kv] or [num_blocks][H_kv][B]), or None where no scale
    belongs to a block (unquantised pools, one scale for the whole pool)."""
    nb = k_pool.shape[0]
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        if not (0 <= src < nb and 0 <= dst < nb) or src == dst:
            continue
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]
        if k_scale is not None:
            k_scale[dst] = k_scale[src]
            v_scale[dst] = v_scale[src]
