"""paged_kv_cache_146_amd — paged KV-cache attention on AMD MI355X (gfx950).

Thin ctypes binding of ``libpagedkv.so`` (C ABI in ``include/pagedkv.h``): every
function here only checks and marshals arguments — pointers of torch tensors,
sizes, torch's current HIP stream — and calls the entry point of the same name.
All computation happens in the library's HIP kernels; if the library is not
built, every call raises instead of falling back to anything else.

Pools are raw byte tensors in the library's physical layout (see the header):
    K pool [num_blocks][num_kv_heads][head_dim/X][block_size][X]
    V pool [num_blocks][num_kv_heads][block_size/TG][head_dim][TG]
with X = 16 / element bytes and TG = min(X, block_size).  ``alloc_pool`` sizes them with ``pkv_pool_bytes``.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedkv.so")

PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3, PKV_INT8 = 0, 1, 2, 3, 4
DTYPE_NAMES = {"f32": PKV_F32, "f16": PKV_F16, "bf16": PKV_BF16, "fp8": PKV_FP8_E4M3,
               "int8": PKV_INT8}
ELEM_BYTES = {PKV_F32: 4, PKV_F16: 2, PKV_BF16: 2, PKV_FP8_E4M3: 1, PKV_INT8: 1}
QUANTISED = (PKV_FP8_E4M3, PKV_INT8)
# where a quantised pool keeps its fp32 scales: one per (block, kv head), one for
# the whole pool, or one per (block, kv head, token)
PKV_SCALE_BLOCK, PKV_SCALE_TENSOR, PKV_SCALE_TOKEN = 0, 1, 2
SCALE_MODES = {"block": PKV_SCALE_BLOCK, "tensor": PKV_SCALE_TENSOR, "token": PKV_SCALE_TOKEN}
STATUS = {0: "PKV_OK", -1: "PKV_EINVAL", -2: "PKV_ERANGE", -3: "PKV_EUNSUPPORTED",
          -4: "PKV_EWORKSPACE", -5: "PKV_EHIP", -6: "PKV_ENOBLOCKS"}
PKV_ENOBLOCKS = -6

EXPORTS = ["pkv_strerror", "pkv_version", "pkv_pool_bytes", "pkv_physical_slot",
           "pkv_validate_block_table", "pkv_slot_mapping", "pkv_kv_cache_write",
           "pkv_kv_cache_append", "pkv_decode_workspace_bytes", "pkv_decode_partition_size",
           "pkv_paged_attention_decode",
           "pkv_split_kv_reduce", "pkv_paged_prefill", "pkv_alloc_create", "pkv_alloc_destroy",
           "pkv_alloc_add_seq", "pkv_alloc_fork", "pkv_alloc_append", "pkv_alloc_free_seq",
           "pkv_alloc_block_table", "pkv_alloc_refcount", "pkv_alloc_free_blocks",
           "pkv_copy_blocks", "pkv_decode_shared_workspace_bytes",
           "pkv_paged_attention_decode_shared", "pkv_paged_attention_decode_window",
           "pkv_decode_append", "pkv_paged_attention_decode_noalloc"]


class PagedKVError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s failed: %s (%s)" % (where, STATUS.get(status, status), _strerror(status))
        super().__init__(msg)


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("scale_mode", ctypes.c_int32),
                ("block_stride", ctypes.c_int64)]

    def __repr__(self):
        return ("PoolDesc(num_blocks=%d, block_size=%d, num_kv_heads=%d, head_dim=%d, "
                "kv_dtype=%d, scale_mode=%d, block_stride=%d)"
                % (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim,
                   self.kv_dtype, self.scale_mode, self.block_stride))


_lock = threading.Lock()
_lib_handle = None


def lib():
    """The loaded libpagedkv.so (raises if it has not been built)."""
    global _lib_handle
    if _lib_handle is None:
        with _lock:
            if _lib_handle is None:
                if not os.path.exists(LIB_PATH):
                    raise RuntimeError(
                        "libpagedkv.so is not built (%s); run `python -m "
                        "paged_kv_cache_146_amd.build_lib`" % LIB_PATH)
                L = ctypes.CDLL(LIB_PATH)
                P, I32, I64, SZ, F = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                      ctypes.c_size_t, ctypes.c_float)
                sigs = {
                    "pkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
                    "pkv_version": (ctypes.c_int, []),
                    "pkv_pool_bytes": (ctypes.c_int, [P, P, P, P]),
                    "pkv_physical_slot": (ctypes.c_int, [P, I32, I32, I64, P]),
                    "pkv_validate_block_table": (ctypes.c_int, [P, I32, I32, P, I32, I32]),
                    "pkv_slot_mapping": (ctypes.c_int, [P, I32, I32, P, P, I32, I32, P, P]),
                    "pkv_kv_cache_write": (ctypes.c_int, [P, I32, P, P, I32, P, P, P, P, P, P]),
                    "pkv_kv_cache_append": (ctypes.c_int, [P, I32, I32, P, P, I32, P, P, I32, P,
                                                           P, P, P, P, P, P]),
                    "pkv_decode_workspace_bytes": (ctypes.c_int, [I32, I32, I32, I32, I32, I32, P]),
                    "pkv_decode_partition_size": (ctypes.c_int, [P, I32, I32, I32, I32, P]),
                    "pkv_paged_attention_decode": (ctypes.c_int, [P, I32, I32, I32, P, P, P, P, P,
                                                                  P, I32, P, I32, F, I32, P, SZ,
                                                                  P, P]),
                    "pkv_split_kv_reduce": (ctypes.c_int, [P, P, P, P, I32, I32, I32, I32, I32, P,
                                                           I32, P]),
                    "pkv_decode_shared_workspace_bytes": (ctypes.c_int, [I32, I32, I32, I32, I32,
                                                                         P]),
                    "pkv_decode_append": (ctypes.c_int, [P, I32, I32, I32, P, P, P, P, I32, P, I32,
                                                         P, P, F, I32, P, SZ, P, P, P]),
                    "pkv_paged_attention_decode_window": (ctypes.c_int, [P, I32, I32, I32, P, P, P,
                                                                         P, P, P, I32, P, I32,
                                                                         F, I32, I32, P, SZ, P,
                                                                         P]),
                    "pkv_paged_attention_decode_shared": (ctypes.c_int, [P, I32, I32, I32, P, P, P,
                                                                         P, P, P, I32, P, I32,
                                                                         I32, F, P, SZ, P, P]),
                    "pkv_paged_prefill": (ctypes.c_int, [P, I32, P, I32, I32, I32, I32, P, P, P,
                                                         P, P, P, I32, P, I32, F, I32, P, P]),
                    "pkv_alloc_create": (ctypes.c_int, [I32, I32, P, I32, P]),
                    "pkv_alloc_destroy": (None, [P]),
                    "pkv_alloc_add_seq": (ctypes.c_int, [P, P]),
                    "pkv_alloc_fork": (ctypes.c_int, [P, I32, P]),
                    "pkv_alloc_append": (ctypes.c_int, [P, I32, P, P, P]),
                    "pkv_alloc_free_seq": (ctypes.c_int, [P, I32, P]),
                    "pkv_alloc_block_table": (ctypes.c_int, [P, I32, P, I32, P, P]),
                    "pkv_alloc_refcount": (ctypes.c_int, [P, I32, P]),
                    "pkv_alloc_free_blocks": (ctypes.c_int, [P, P, I32, P]),
                    "pkv_copy_blocks": (ctypes.c_int, [P, I32, P, P, P, P, P, P]),
                    "pkv_paged_attention_decode_noalloc": (ctypes.c_int, [P, I32, I32, I32, P, P,
                                                                          P, P, P, P, I32, P,
                                                                          I32, F, I32, P, P]),
                }
                for name, (res, args) in sigs.items():
                    fn = getattr(L, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib_handle = L
    return _lib_handle


def _strerror(status: int) -> str:
    try:
        return lib().pkv_strerror(int(status)).decode()
    except Exception:  # pragma: no cover - only while reporting another failure
        return "?"


def _check(rc: int, where: str):
    if rc != 0:
        raise PagedKVError(rc, where)


# ---------------------------------------------------------------------------------------
# torch plumbing
# ---------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if isinstance(t, str):
        return DTYPE_NAMES[t]
    m = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
         torch.float8_e4m3fn: PKV_FP8_E4M3}
    if t not in m:
        raise ValueError("unsupported dtype %s" % (t,))
    return m[t]


def torch_dtype(code: int):
    torch = _torch()
    return {PKV_F32: torch.float32, PKV_F16: torch.float16, PKV_BF16: torch.bfloat16,
            PKV_FP8_E4M3: torch.uint8, PKV_INT8: torch.int8}[code]


def _ptr(t, name, device=True, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError("%s is required" % name)
    if device and not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------------------
# C-ABI calls (same names as include/pagedkv.h)
# ---------------------------------------------------------------------------------------
def pkv_version() -> int:
    return int(lib().pkv_version())


def pool_desc(num_blocks, block_size, num_kv_heads, head_dim, kv_dtype,
              scale_mode=PKV_SCALE_BLOCK, block_stride=0) -> PoolDesc:
    """block_stride: bytes from one block to the next in each pool (0 = dense)."""
    code = dtype_code(kv_dtype) if not isinstance(kv_dtype, int) else kv_dtype
    mode = SCALE_MODES[scale_mode] if isinstance(scale_mode, str) else int(scale_mode)
    return PoolDesc(int(num_blocks), int(block_size), int(num_kv_heads), int(head_dim), code,
                    mode, int(block_stride))


def pkv_pool_bytes(desc: PoolDesc):
    k, v, s = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().pkv_pool_bytes(ctypes.byref(desc), ctypes.byref(k), ctypes.byref(v),
                                ctypes.byref(s)), "pkv_pool_bytes")
    return k.value, v.value, s.value


def alloc_pool(desc: PoolDesc, device="cuda", fill_byte=None):
    """(k_pool, v_pool) as uint8 device tensors of pkv_pool_bytes(desc) bytes each."""
    torch = _torch()
    kb, vb, _ = pkv_pool_bytes(desc)
    k = torch.empty(kb, dtype=torch.uint8, device=device)
    v = torch.empty(vb, dtype=torch.uint8, device=device)
    if fill_byte is not None:
        k.fill_(fill_byte)
        v.fill_(fill_byte)
    return k, v


def pkv_physical_slot(table, block_size: int, token_pos: int) -> int:
    """Host-side slot of one position (the page's physical_slot); raises PagedKVError."""
    arr = (ctypes.c_int32 * len(table))(*[int(x) for x in table])
    out = ctypes.c_int64()
    _check(lib().pkv_physical_slot(arr, len(table), int(block_size), int(token_pos),
                                   ctypes.byref(out)), "pkv_physical_slot")
    return out.value


def pkv_validate_block_table(block_table, context_lens, block_size: int, num_blocks: int):
    """Host check of a [S][W] int32 table (numpy or CPU tensor); raises PagedKVError."""
    import numpy as np
    bt = np.ascontiguousarray(np.asarray(block_table), np.int32)
    cl = np.ascontiguousarray(np.asarray(context_lens), np.int32)
    S = bt.shape[0] if bt.ndim == 2 else 0
    W = bt.shape[1] if bt.ndim == 2 else 0
    _check(lib().pkv_validate_block_table(bt.ctypes.data, S, W, cl.ctypes.data, int(block_size),
                                          int(num_blocks)), "pkv_validate_block_table")


def pkv_slot_mapping(block_table, seq_idx, positions, block_size: int, out=None, stream=None):
    torch = _torch()
    T = int(seq_idx.numel())
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=seq_idx.device)
    S, W = (int(block_table.shape[0]), int(block_table.shape[1]))
    _check(lib().pkv_slot_mapping(_ptr(block_table, "block_table"), S, W,
                                  _ptr(seq_idx, "seq_idx"), _ptr(positions, "positions"), T,
                                  int(block_size), _ptr(out, "slot_mapping"), _stream(stream)),
           "pkv_slot_mapping")
    return out


def pkv_kv_cache_write(slot_mapping, k, v, desc: PoolDesc, k_pool, v_pool, k_scale=None,
                       v_scale=None, src_dtype=None, stream=None):
    T = int(slot_mapping.numel())
    sd = dtype_code(src_dtype if src_dtype is not None else k.dtype)
    _check(lib().pkv_kv_cache_write(_ptr(slot_mapping, "slot_mapping"), T, _ptr(k, "k"),
                                    _ptr(v, "v"), sd, ctypes.byref(desc), _ptr(k_pool, "k_pool"),
                                    _ptr(v_pool, "v_pool"),
                                    _ptr(k_scale, "k_scale", allow_none=True),
                                    _ptr(v_scale, "v_scale", allow_none=True), _stream(stream)),
           "pkv_kv_cache_write")


def pkv_kv_cache_append(block_table, seq_idx, positions, k, v, desc: PoolDesc, k_pool, v_pool,
                        k_scale=None, v_scale=None, src_dtype=None, slot_mapping_out=None,
                        stream=None):
    T = int(seq_idx.numel())
    S, W = (int(block_table.shape[0]), int(block_table.shape[1]))
    sd = dtype_code(src_dtype if src_dtype is not None else k.dtype)
    _check(lib().pkv_kv_cache_append(_ptr(block_table, "block_table"), S, W,
                                     _ptr(seq_idx, "seq_idx"), _ptr(positions, "positions"), T,
                                     _ptr(k, "k"), _ptr(v, "v"), sd, ctypes.byref(desc),
                                     _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"),
                                     _ptr(k_scale, "k_scale", allow_none=True),
                                     _ptr(v_scale, "v_scale", allow_none=True),
                                     _ptr(slot_mapping_out, "slot_mapping_out", allow_none=True),
                                     _stream(stream)),
           "pkv_kv_cache_append")
    return slot_mapping_out


class BlockAllocator:
    """Host block allocator (pkv_alloc_*): free stack, refcounts, fork, tail copy on
    write, deferred release.  Argument marshalling only; the logic is in the library."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self.block_size = int(block_size)
        h = ctypes.c_void_p()
        if free_order is None:
            _check(lib().pkv_alloc_create(int(num_blocks), int(block_size), None, 0,
                                          ctypes.byref(h)), "pkv_alloc_create")
        else:
            arr = (ctypes.c_int32 * len(free_order))(*[int(b) for b in free_order])
            _check(lib().pkv_alloc_create(int(num_blocks), int(block_size), arr, len(free_order),
                                          ctypes.byref(h)), "pkv_alloc_create")
        self._h = h

    def close(self):
        if self._h:
            lib().pkv_alloc_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass

    def add_seq(self) -> int:
        out = ctypes.c_int32()
        _check(lib().pkv_alloc_add_seq(self._h, ctypes.byref(out)), "pkv_alloc_add_seq")
        return out.value

    def fork(self, parent: int) -> int:
        out = ctypes.c_int32()
        _check(lib().pkv_alloc_fork(self._h, int(parent), ctypes.byref(out)), "pkv_alloc_fork")
        return out.value

    def append(self, seq: int):
        """(slot, cow_src, cow_dst) of the sequence's next token; cow_* are -1 without a copy."""
        slot, src, dst = ctypes.c_int64(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib().pkv_alloc_append(self._h, int(seq), ctypes.byref(slot), ctypes.byref(src),
                                      ctypes.byref(dst)), "pkv_alloc_append")
        return slot.value, src.value, dst.value

    def free_seq(self, seq: int, event=None):
        """event: a torch.cuda.Event recorded after the sequence's last GPU use, or None."""
        ev = ctypes.c_void_p(event.cuda_event) if event is not None else None
        _check(lib().pkv_alloc_free_seq(self._h, int(seq), ev), "pkv_alloc_free_seq")

    def table(self, seq: int):
        """(block table as a list, committed length)"""
        n, length = ctypes.c_int32(), ctypes.c_int64()
        _check(lib().pkv_alloc_block_table(self._h, int(seq), None, 0, ctypes.byref(n),
                                           ctypes.byref(length)), "pkv_alloc_block_table")
        arr = (ctypes.c_int32 * max(1, n.value))()
        _check(lib().pkv_alloc_block_table(self._h, int(seq), arr, n.value, ctypes.byref(n),
                                           ctypes.byref(length)), "pkv_alloc_block_table")
        return [arr[i] for i in range(n.value)], length.value

    def refcount(self, block: int) -> int:
        out = ctypes.c_int32()
        _check(lib().pkv_alloc_refcount(self._h, int(block), ctypes.byref(out)),
               "pkv_alloc_refcount")
        return out.value

    def free_blocks(self):
        """the free stack, bottom to top (the last entry is handed out next)"""
        n = ctypes.c_int32()
        _check(lib().pkv_alloc_free_blocks(self._h, None, 0, ctypes.byref(n)),
               "pkv_alloc_free_blocks")
        arr = (ctypes.c_int32 * max(1, n.value))()
        _check(lib().pkv_alloc_free_blocks(self._h, arr, n.value, ctypes.byref(n)),
               "pkv_alloc_free_blocks")
        return [arr[i] for i in range(n.value)]


def pkv_copy_blocks(pairs, desc: PoolDesc, k_pool, v_pool, k_scale=None, v_scale=None,
                    stream=None):
    """pairs: device int32 [n][2] of (src, dst) block ids"""
    n = int(pairs.shape[0]) if pairs.numel() else 0
    _check(lib().pkv_copy_blocks(_ptr(pairs, "pairs", allow_none=(n == 0)), n, ctypes.byref(desc),
                                 _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"),
                                 _ptr(k_scale, "k_scale", allow_none=True),
                                 _ptr(v_scale, "v_scale", allow_none=True), _stream(stream)),
           "pkv_copy_blocks")


PARTITION_BALANCED = -1
MAX_WORKERS = 4096


def pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                               partition_size) -> int:
    out = ctypes.c_size_t()
    _check(lib().pkv_decode_workspace_bytes(int(num_seqs), int(num_q_heads), int(num_kv_heads),
                                            int(head_dim), int(max_context_len),
                                            int(partition_size), ctypes.byref(out)),
           "pkv_decode_workspace_bytes")
    return out.value


def pkv_decode_partition_size(context_lens, num_kv_heads: int, max_context_len: int,
                              num_cus: int = 0) -> int:
    """The library's partition size for a decode step (0: unsplit), from HOST context
    lengths (a sequence of ints or an int32 numpy array); num_cus <= 0 asks the
    current device."""
    import numpy as np
    c = np.ascontiguousarray(np.asarray(context_lens, dtype=np.int32))
    out = ctypes.c_int32()
    _check(lib().pkv_decode_partition_size(c.ctypes.data if c.size else None, int(c.size),
                                           int(num_kv_heads), int(max_context_len),
                                           int(num_cus), ctypes.byref(out)),
           "pkv_decode_partition_size")
    return out.value


def pkv_paged_attention_decode(q, desc: PoolDesc, k_pool, v_pool, block_table, context_lens,
                               max_context_len: int, scale: float, partition_size: int = 0,
                               k_scale=None, v_scale=None, workspace=None, out=None,
                               q_dtype=None, stream=None):
    torch = _torch()
    S, Hq = int(q.shape[0]), int(q.shape[1])
    qd = dtype_code(q_dtype if q_dtype is not None else q.dtype)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    need = pkv_decode_workspace_bytes(S, Hq, desc.num_kv_heads, desc.head_dim, max_context_len,
                                      partition_size)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
    _check(lib().pkv_paged_attention_decode(
        _ptr(q, "q"), qd, S, Hq, ctypes.byref(desc), _ptr(k_pool, "k_pool"),
        _ptr(v_pool, "v_pool"), _ptr(k_scale, "k_scale", allow_none=True),
        _ptr(v_scale, "v_scale", allow_none=True), _ptr(block_table, "block_table"),
        int(block_table.shape[1]), _ptr(context_lens, "context_lens"), int(max_context_len),
        float(scale), int(partition_size), _ptr(workspace, "workspace", allow_none=True),
        ws_bytes, _ptr(out, "out"), _stream(stream)), "pkv_paged_attention_decode")
    return out


def pkv_paged_attention_decode_noalloc(q, desc: PoolDesc, k_pool, v_pool, block_table,
                                       context_lens, max_context_len: int, scale: float,
                                       partition_size: int = 0, k_scale=None, v_scale=None,
                                       out=None, q_dtype=None, stream=None):
    """pkv_paged_attention_decode with its split-KV scratch in the library's own device
    array (no workspace argument, nothing allocated by the call); `out` must be given
    by callers that cannot allocate."""
    torch = _torch()
    S, Hq = int(q.shape[0]), int(q.shape[1])
    qd = dtype_code(q_dtype if q_dtype is not None else q.dtype)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    _check(lib().pkv_paged_attention_decode_noalloc(
        _ptr(q, "q"), qd, S, Hq, ctypes.byref(desc), _ptr(k_pool, "k_pool"),
        _ptr(v_pool, "v_pool"), _ptr(k_scale, "k_scale", allow_none=True),
        _ptr(v_scale, "v_scale", allow_none=True), _ptr(block_table, "block_table"),
        int(block_table.shape[1]), _ptr(context_lens, "context_lens"), int(max_context_len),
        float(scale), int(partition_size), _ptr(out, "out"), _stream(stream)),
        "pkv_paged_attention_decode_noalloc")
    return out


def pkv_decode_shared_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                      shared_len) -> int:
    out = ctypes.c_size_t()
    _check(lib().pkv_decode_shared_workspace_bytes(int(num_seqs), int(num_q_heads),
                                                   int(num_kv_heads), int(head_dim),
                                                   int(shared_len), ctypes.byref(out)),
           "pkv_decode_shared_workspace_bytes")
    return out.value


def pkv_paged_attention_decode_shared(q, desc: PoolDesc, k_pool, v_pool, block_table,
                                      context_lens, max_context_len: int, scale: float,
                                      shared_len: int, k_scale=None, v_scale=None,
                                      workspace=None, out=None, q_dtype=None, stream=None):
    """Decode of a batch whose table rows share their first shared_len / block_size
    entries (the shared prefix is read once per kv head)."""
    torch = _torch()
    S, Hq = int(q.shape[0]), int(q.shape[1])
    qd = dtype_code(q_dtype if q_dtype is not None else q.dtype)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if workspace is None:
        need = pkv_decode_shared_workspace_bytes(S, Hq, desc.num_kv_heads, desc.head_dim,
                                                 shared_len)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = int(workspace.numel() * workspace.element_size())
    _check(lib().pkv_paged_attention_decode_shared(
        _ptr(q, "q"), qd, S, Hq, ctypes.byref(desc), _ptr(k_pool, "k_pool"),
        _ptr(v_pool, "v_pool"), _ptr(k_scale, "k_scale", allow_none=True),
        _ptr(v_scale, "v_scale", allow_none=True), _ptr(block_table, "block_table"),
        int(block_table.shape[1]), _ptr(context_lens, "context_lens"), int(max_context_len),
        int(shared_len), float(scale), _ptr(workspace, "workspace"), ws_bytes, _ptr(out, "out"),
        _stream(stream)), "pkv_paged_attention_decode_shared")
    return out


def pkv_paged_attention_decode_window(q, desc: PoolDesc, k_pool, v_pool, block_table,
                                      context_lens, max_context_len: int, scale: float,
                                      window: int, partition_size: int = 0, k_scale=None,
                                      v_scale=None, workspace=None, out=None, q_dtype=None,
                                      stream=None):
    """Sliding-window decode: sequence s sees the keys [max(0, ctx_s - window), ctx_s)."""
    torch = _torch()
    S, Hq = int(q.shape[0]), int(q.shape[1])
    qd = dtype_code(q_dtype if q_dtype is not None else q.dtype)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    need = pkv_decode_workspace_bytes(S, Hq, desc.num_kv_heads, desc.head_dim, max_context_len,
                                      partition_size)
    if need > 0 and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
    _check(lib().pkv_paged_attention_decode_window(
        _ptr(q, "q"), qd, S, Hq, ctypes.byref(desc), _ptr(k_pool, "k_pool"),
        _ptr(v_pool, "v_pool"), _ptr(k_scale, "k_scale", allow_none=True),
        _ptr(v_scale, "v_scale", allow_none=True), _ptr(block_table, "block_table"),
        int(block_table.shape[1]), _ptr(context_lens, "context_lens"), int(max_context_len),
        float(scale), int(window), int(partition_size),
        _ptr(workspace, "workspace", allow_none=True), ws_bytes, _ptr(out, "out"),
        _stream(stream)), "pkv_paged_attention_decode_window")
    return out


def pkv_decode_append(q, desc: PoolDesc, k_pool, v_pool, block_table, context_lens,
                      max_context_len: int, k_new, v_new, scale: float,
                      partition_size: int = -1, workspace=None, out=None,
                      slot_mapping_out=None, stream=None):
    """One decode step: stores each sequence's newest token (k_new / v_new
    [S][H_kv][D], position ctx - 1) in the decode's launch and returns the decode
    (balanced: -1, unsplit: 0, fixed partitions: a positive multiple of 64, which
    adds the reduce launch)."""
    torch = _torch()
    S, Hq = int(q.shape[0]), int(q.shape[1])
    qd = dtype_code(q.dtype)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    need = pkv_decode_workspace_bytes(S, Hq, desc.num_kv_heads, desc.head_dim,
                                      max_context_len, partition_size)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = int(workspace.numel() * workspace.element_size()) if workspace is not None else 0
    _check(lib().pkv_decode_append(
        _ptr(q, "q"), qd, S, Hq, ctypes.byref(desc), _ptr(k_pool, "k_pool"),
        _ptr(v_pool, "v_pool"), _ptr(block_table, "block_table"), int(block_table.shape[1]),
        _ptr(context_lens, "context_lens"), int(max_context_len), _ptr(k_new, "k_new"),
        _ptr(v_new, "v_new"), float(scale), int(partition_size),
        _ptr(workspace, "workspace", allow_none=True), ws_bytes,
        _ptr(out, "out"), _ptr(slot_mapping_out, "slot_mapping_out", allow_none=True),
        _stream(stream)), "pkv_decode_append")
    return out


def pkv_split_kv_reduce(part_out, part_max, part_sum, context_lens, partition_size: int,
                        out_dtype, out=None, stream=None):
    torch = _torch()
    S, Hq, P, D = (int(x) for x in part_out.shape)
    od = dtype_code(out_dtype)
    if out is None:
        out = torch.empty((S, Hq, D), dtype=torch_dtype(od), device=part_out.device)
    _check(lib().pkv_split_kv_reduce(_ptr(part_out, "part_out"), _ptr(part_max, "part_max"),
                                     _ptr(part_sum, "part_sum"), _ptr(context_lens, "context_lens"),
                                     S, Hq, D, int(partition_size), P, _ptr(out, "out"), od,
                                     _stream(stream)), "pkv_split_kv_reduce")
    return out


def pkv_paged_prefill(q, cu_seqlens_q, max_q_len: int, desc: PoolDesc, k_pool, v_pool,
                      block_table, context_lens, max_context_len: int, scale: float,
                      causal: bool = True, k_scale=None, v_scale=None, out=None, q_dtype=None,
                      stream=None):
    torch = _torch()
    T, Hq = int(q.shape[0]), int(q.shape[1])
    qd = dtype_code(q_dtype if q_dtype is not None else q.dtype)
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    S = int(cu_seqlens_q.numel()) - 1
    _check(lib().pkv_paged_prefill(
        _ptr(q, "q"), qd, _ptr(cu_seqlens_q, "cu_seqlens_q"), S, T, int(max_q_len), Hq,
        ctypes.byref(desc), _ptr(k_pool, "k_pool"), _ptr(v_pool, "v_pool"),
        _ptr(k_scale, "k_scale", allow_none=True), _ptr(v_scale, "v_scale", allow_none=True),
        _ptr(block_table, "block_table"), int(block_table.shape[1]),
        _ptr(context_lens, "context_lens"), int(max_context_len), float(scale), int(bool(causal)),
        _ptr(out, "out"), _stream(stream)), "pkv_paged_prefill")
    return out
