"""Python binding of libpkv.so: paged KV cache decode for AMD MI355X (gfx950).

Thin ctypes marshalling over the C ABI declared in include/pkv.h; every step of the
path runs in the library (host block pool in C++, kernels in HIP). PyTorch supplies
device memory and the current HIP stream only. The functions keep the C names:

  kv_pool_create(...)            -> KVPool (host block pool: allocate_slots, tables)
  kv_bytes_per_token(...)
  reshape_and_cache(...)         slot-mapped write of new tokens' K/V
  paged_attention_decode(...)    GQA decode attention through block tables
  paged_attention_decode_append(...)  the new token's cache write fused with the decode
  paged_attention_reduce(...)    merge of per-partition results
  paged_attention_decode_plan(...)  host-side order of a step's single-pass decodes
  reshape_and_cache_fp8, paged_attention_decode_fp8, paged_attention_decode_append_fp8:
                                 the same over an FP8 (e4m3) cache with per-tensor K/V scales

There is no fallback: if libpkv.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY selects another build of the same ABI (for example a debug build)
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(HERE, "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_ENOTSUP, PKV_ENOMEM, PKV_ENOENT, PKV_EHIP = 0, -1, -2, -3, -4, -5
PKV_F32, PKV_F16, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2, 3
PKV_PARTITION_AUTO = -1
BLOCK_SIZE = 16          # default tokens per block; 8 and 32 are the other sizes built
_CODE_NAMES = {PKV_EINVAL: "EINVAL", PKV_ENOTSUP: "ENOTSUP", PKV_ENOMEM: "ENOMEM",
               PKV_ENOENT: "ENOENT", PKV_EHIP: "EHIP"}

_lib = None


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODE_NAMES.get(code, code)}: {msg}")
        self.code = code
        self.name = _CODE_NAMES.get(code, str(code))


class _Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("total_blocks", "free_blocks", "used_blocks",
                                              "shared_blocks", "alloc_failures", "num_seqs",
                                              "cached_blocks", "prefix_hit_blocks")]


def lib():
    """Load libpkv.so (built in-tree by __graft_entry__.build()); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    U64 = ctypes.c_uint64
    PP = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "pkv_last_error": ([], ctypes.c_char_p),
        "pkv_version": ([], ctypes.c_char_p),
        "kv_bytes_per_token": ([I32, I32, I32, I32], I64),
        "kv_pool_create": ([I64, I32, I32, I32, I32, I32, P, PP], ctypes.c_int),
        "kv_pool_destroy": ([P], None),
        "kv_pool_bytes_per_token": ([P], I64),
        "kv_pool_cache_shape": ([P, P, P], ctypes.c_int),
        "kv_pool_add_seq": ([P, I64], ctypes.c_int),
        "kv_pool_share_prefix": ([P, I64, I64, I32], ctypes.c_int),
        "kv_pool_append": ([P, I64, I32, P], ctypes.c_int),
        "kv_pool_append_batch": ([P, P, I32, P], ctypes.c_int),
        "kv_pool_free_seq": ([P, I64], ctypes.c_int),
        "kv_pool_seq_len": ([P, I64, P], ctypes.c_int),
        "kv_pool_seq_blocks": ([P, I64, P, I32, P], ctypes.c_int),
        "kv_pool_free_queue": ([P, P, I64, P], ctypes.c_int),
        "kv_pool_refcount": ([P, I64, P], ctypes.c_int),
        "kv_pool_build_tables": ([P, P, I32, I32, P, P], ctypes.c_int),
        "kv_pool_stats": ([P, P], ctypes.c_int),
        "kv_pool_add_seq_prefix": ([P, I64, P, I32, U64, P], ctypes.c_int),
        "kv_pool_fork": ([P, I64, I64], ctypes.c_int),
        "kv_pool_append_tokens": ([P, I64, P, I32, P, P], ctypes.c_int),
        "kv_pool_append_batch_tokens": ([P, P, P, I32, P, P, P], ctypes.c_int),
        "copy_blocks": ([P, P, I32, P, I32, I64, I64, P], ctypes.c_int),
        "paged_attention_prefill": ([P, P, I64, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                     I64, F, I32, I32, P], ctypes.c_int),
        "reshape_and_cache": ([P, P, P, P, P, I32, I32, I32, I32, I64, I64, I64, I32, P],
                              ctypes.c_int),
        "paged_attention_decode": ([P, P, P, P, P, I64, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                    I64, F, I32, I32, I32, I32, P, P], ctypes.c_int),
        "paged_attention_decode_plan": ([P, I32, I32, P], ctypes.c_int),
        "paged_attention_reduce": ([P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, I32, I32,
                                    P],
                                   ctypes.c_int),
        "paged_attention_decode_append": ([P, P, P, P, P, I64, P, P, I64, I64, P, P, P, P, P,
                                           I32, I32, I32, I32, I32, I32, I64, F, I32, I32, I32,
                                           I32, P, P], ctypes.c_int),
        "reshape_and_cache_fp8": ([P, P, P, P, P, I32, I32, I32, I32, I64, I64, I64, I32, F, F,
                                   P], ctypes.c_int),
        "paged_attention_decode_fp8": ([P, P, P, P, P, I64, P, P, P, P, I32, I32, I32, I32, I32,
                                        I32, I64, F, F, F, I32, I32, I32, I32, P, P], ctypes.c_int),
        "paged_attention_decode_append_fp8": ([P, P, P, P, P, I64, P, P, I64, I64, P, P, P, P, P,
                                               I32, I32, I32, I32, I32, I32, I64, F, F, F, I32,
                                               I32, I32, I32, P, P], ctypes.c_int),
        "paged_attention_decode_noalloc": ([P, P, I64, P, P, P, P, I32, I32, I32, I32, I32, I32,
                                            I64, F, I32, I32, I32, P], ctypes.c_int),
        "paged_attention_decode_noalloc_workspace": ([], ctypes.c_size_t),
        "pkv_measure_read": ([P, I64, I32, I32, I32, P, I32, P], ctypes.c_int),
        "pkv_measure_gather": ([P, P, P, P, I32, I32, I32, I32, I32, I32, I64, P, I32, I32, P, I32,
                                P], ctypes.c_int),
        "pkv_measure_rate": ([I32, I32, I32, P, I32, P], ctypes.c_int),
        "pkv_timer_enable": ([I32], ctypes.c_int),
        "pkv_timer_read": ([I32, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        # A host-only build of the pool (PKV_LIBRARY, e.g. the sanitised one the CPU tests
        # build) has no kernel entry points: those stay unbound and fail when called.
        fn = getattr(L, name, None)
        if fn is None:
            continue
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


EXPORTED = ("pkv_last_error", "pkv_version", "kv_bytes_per_token", "kv_pool_create",
            "kv_pool_destroy", "kv_pool_bytes_per_token", "kv_pool_cache_shape",
            "kv_pool_add_seq", "kv_pool_share_prefix", "kv_pool_append", "kv_pool_append_batch",
            "kv_pool_free_seq", "kv_pool_seq_len", "kv_pool_seq_blocks", "kv_pool_free_queue",
            "kv_pool_refcount", "kv_pool_build_tables", "kv_pool_stats", "reshape_and_cache",
            "paged_attention_decode", "paged_attention_reduce", "paged_attention_decode_append",
            "reshape_and_cache_fp8", "paged_attention_decode_fp8",
            "paged_attention_decode_append_fp8", "pkv_timer_enable", "pkv_timer_read",
            "kv_pool_add_seq_prefix", "kv_pool_fork", "kv_pool_append_tokens",
            "kv_pool_append_batch_tokens", "copy_blocks", "paged_attention_prefill",
            "paged_attention_decode_plan", "paged_attention_decode_noalloc",
            "paged_attention_decode_noalloc_workspace", "pkv_measure_read", "pkv_measure_gather",
            "pkv_measure_rate")


def _check(rc: int):
    if rc != PKV_OK:
        raise PkvError(rc, lib().pkv_last_error().decode())


def version() -> str:
    return lib().pkv_version().decode()


# ------------------------------------------------------------------ dtypes / torch
def _torch():
    import torch
    return torch


def dtype_code(dt) -> int:
    """PKV_* code of a torch dtype or name; an FP8 cache is held in uint8 tensors."""
    torch = _torch()
    m = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16,
         torch.uint8: PKV_FP8_E4M3, "f32": PKV_F32, "f16": PKV_F16, "bf16": PKV_BF16,
         "fp8": PKV_FP8_E4M3}
    if dt not in m:
        raise ValueError(f"unsupported dtype {dt}")
    return m[dt]


def torch_dtype(code_or_name):
    torch = _torch()
    return {PKV_F32: torch.float32, PKV_F16: torch.float16, PKV_BF16: torch.bfloat16,
            PKV_FP8_E4M3: torch.uint8, "f32": torch.float32, "f16": torch.float16,
            "bf16": torch.bfloat16, "fp8": torch.uint8}[code_or_name]


def _stream(t, stream):
    if stream is not None:
        return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return ctypes.c_void_p(t.data_ptr())


# ------------------------------------------------------------ argument validation
# The C ABI sees raw pointers and sizes only, so a tensor of the wrong type or shape would
# be read with the wrong element size or extent. Every device wrapper below checks what it
# hands over (types, shapes, contiguity, one device) and raises ValueError before any call.
def _index(t, name, numel_min=None, shape=None):
    """An int32, contiguous index tensor (slots, lengths, tables, offsets)."""
    torch = _torch()
    if t is None:
        raise ValueError(f"{name} is required")
    if t.dtype != torch.int32:
        raise ValueError(f"{name} must be int32, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel_min is not None and t.numel() < numel_min:
        raise ValueError(f"{name} must hold at least {numel_min} entries, got {t.numel()}")


def _same_device(ref, named):
    for t, nm in named:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{nm} is on {t.device}, expected {ref.device} (where q is)")


def _float_type(t, name):
    torch = _torch()
    if t.dtype not in (torch.float32, torch.float16, torch.bfloat16):
        raise ValueError(f"{name} must be float32, float16 or bfloat16, got {t.dtype}")


def _caches(k_cache, v_cache, elem_dtype, hkv=None, head_dim=None):
    """k_cache [nb][Hkv][d/x][BS][x] and v_cache [nb][Hkv][d][BS] of elem_dtype, contiguous;
    returns (num_blocks, Hkv, head_dim, BS)."""
    torch = _torch()
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        if t.dtype != elem_dtype:
            raise ValueError(f"{nm} must be {elem_dtype}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if k_cache.dim() != 5 or v_cache.dim() != 4:
        raise ValueError("k_cache must be [nb][Hkv][d/x][BS][x] and v_cache [nb][Hkv][d][BS]")
    nb, h, d, bs = (int(x) for x in v_cache.shape)
    x = 16 // k_cache.element_size()
    if tuple(k_cache.shape) != (nb, h, d // x, bs, x) or d % x:
        raise ValueError(f"k_cache shape {tuple(k_cache.shape)} does not match v_cache "
                         f"{tuple(v_cache.shape)} in the documented layout (x = {x})")
    if hkv is not None and h != hkv:
        raise ValueError(f"the caches hold {h} KV heads, expected {hkv}")
    if head_dim is not None and d != head_dim:
        raise ValueError(f"the caches hold head_dim {d}, expected {head_dim}")
    return nb, h, d, bs


def _rows(t, name, B, H, d, dtype=None):
    """[B][H][d] with dense heads and dimensions (the first stride is free)."""
    if tuple(t.shape) != (B, H, d) or t.stride(2) != 1 or t.stride(1) != d:
        raise ValueError(f"{name} must be [{B}][{H}][{d}] with dense heads/dims, got "
                         f"{tuple(t.shape)} strides {tuple(t.stride())}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _partials(part_out, part_max, part_sum, B, Hq, d, partition_size, max_partitions):
    """The fp32 partial buffers of a partitioned decode: part_out [B][Hq][P][d],
    part_max / part_sum [B][Hq][P], contiguous. The reduce indexes them with
    P = part_out.shape[2], so max_partitions must be P (0: take it from part_out).
    Returns max_partitions."""
    torch = _torch()
    if partition_size == 0:
        return max_partitions
    if part_out is None or part_max is None or part_sum is None:
        raise ValueError("a partitioned decode needs part_out, part_max and part_sum")
    if part_out.dim() != 4 or tuple(part_out.shape[:2]) != (B, Hq) or part_out.shape[3] != d:
        raise ValueError(f"part_out must be [{B}][{Hq}][P][{d}], got {tuple(part_out.shape)}")
    P = int(part_out.shape[2])
    for t, nm in ((part_out, "part_out"), (part_max, "part_max"), (part_sum, "part_sum")):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{nm} must be a contiguous float32 tensor")
    for t, nm in ((part_max, "part_max"), (part_sum, "part_sum")):
        if tuple(t.shape) != (B, Hq, P):
            raise ValueError(f"{nm} must be [{B}][{Hq}][{P}], got {tuple(t.shape)}")
    if max_partitions == 0:
        return P
    if max_partitions != P:
        raise ValueError(f"max_partitions {max_partitions} differs from part_out's {P}")
    return P


def _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, partition_size, part_out,
                 part_max, part_sum, max_partitions, fp8, append=None):
    """Checks shared by the decode wrappers; returns (B, Hq, d, Hkv, BS, max_partitions)."""
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be [B][Hq][d]")
    B, Hq, d = (int(x) for x in q.shape)
    _float_type(q, "q")
    _rows(q, "q", B, Hq, d)
    if tuple(out.shape) != (B, Hq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B][Hq][d] tensor")
    _float_type(out, "out")
    _, hkv, _, bs = _caches(k_cache, v_cache, torch.uint8 if fp8 else q.dtype, head_dim=d)
    if Hq % hkv:
        raise ValueError(f"num_heads {Hq} is not a multiple of the caches' {hkv} KV heads")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError(f"block_tables must be [{B}][max_blocks], got {tuple(block_tables.shape)}")
    _index(block_tables, "block_tables")
    _index(seq_lens, "seq_lens", shape=(B,))
    maxp = _partials(part_out, part_max, part_sum, B, Hq, d, partition_size, max_partitions)
    named = [(out, "out"), (k_cache, "k_cache"), (v_cache, "v_cache"),
             (block_tables, "block_tables"), (seq_lens, "seq_lens"), (part_out, "part_out"),
             (part_max, "part_max"), (part_sum, "part_sum")]
    if append is not None:
        key, value, slot_mapping = append
        _rows(key, "key", B, hkv, d, q.dtype)
        _rows(value, "value", B, hkv, d, q.dtype)
        _index(slot_mapping, "slot_mapping", numel_min=B)
        named += [(key, "key"), (value, "value"), (slot_mapping, "slot_mapping")]
    _same_device(q, named)
    return B, Hq, d, hkv, bs, maxp


def kv_bytes_per_token(num_layers: int, num_kv_heads: int, head_dim: int, dtype) -> int:
    v = lib().kv_bytes_per_token(num_layers, num_kv_heads, head_dim, dtype_code(dtype))
    if v < 0:
        _check(PKV_EINVAL)
    return v


def cache_shapes(num_blocks: int, num_kv_heads: int, head_dim: int, dtype,
                 block_size: int = BLOCK_SIZE):
    """(k_shape, v_shape) of one layer's caches: [nb][Hkv][d/x][BS][x], [nb][Hkv][d][BS]."""
    x = 16 // {PKV_F32: 4, PKV_F16: 2, PKV_BF16: 2, PKV_FP8_E4M3: 1}[dtype_code(dtype)]
    return ((num_blocks, num_kv_heads, head_dim // x, block_size, x),
            (num_blocks, num_kv_heads, head_dim, block_size))


def block_size_of(v_cache) -> int:
    """Tokens per block of a cache pair, read from the V cache's shape [nb][Hkv][d][BS]."""
    if v_cache.dim() != 4:
        raise ValueError("v_cache must be [num_blocks][Hkv][d][block_size]")
    return int(v_cache.shape[3])


def alloc_caches(num_blocks: int, num_kv_heads: int, head_dim: int, dtype, device="cuda",
                 fill=None, block_size: int = BLOCK_SIZE):
    """Allocate one layer's (k_cache, v_cache) through PyTorch (uninitialised, or filled;
    an FP8 cache is uint8, fill being a code)."""
    torch = _torch()
    ks, vs = cache_shapes(num_blocks, num_kv_heads, head_dim, dtype, block_size)
    td = torch_dtype(dtype) if not isinstance(dtype, torch.dtype) else dtype
    kc = torch.empty(ks, dtype=td, device=device)
    vc = torch.empty(vs, dtype=td, device=device)
    if fill is not None:
        kc.fill_(fill)
        vc.fill_(fill)
    return kc, vc


# --------------------------------------------------------------------- block pool
class KVPool:
    """Host block pool (C++). seq ids are arbitrary 64-bit integers."""

    def __init__(self, num_blocks: int, num_layers: int, num_kv_heads: int, head_dim: int,
                 dtype, free_order=None, block_size: int = BLOCK_SIZE):
        import numpy as np
        self._np = np
        h = ctypes.c_void_p()
        fo = None
        if free_order is not None:
            self._order = np.ascontiguousarray(free_order, dtype=np.int32)
            if self._order.shape != (num_blocks,):
                raise ValueError("free_order must have num_blocks entries")
            fo = self._order.ctypes.data_as(ctypes.c_void_p)
        _check(lib().kv_pool_create(num_blocks, block_size, num_layers, num_kv_heads, head_dim,
                                    dtype_code(dtype), fo, ctypes.byref(h)))
        self._h = h
        self._destroy = lib().kv_pool_destroy   # kept: module globals may be gone at exit
        self.num_blocks = num_blocks
        self.num_layers, self.num_kv_heads, self.head_dim = num_layers, num_kv_heads, head_dim
        self.dtype = dtype

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            self._destroy(self._h)
            self._h = None

    __del__ = close

    def bytes_per_token(self) -> int:
        return lib().kv_pool_bytes_per_token(self._h)

    def cache_shape(self):
        ks = (ctypes.c_int64 * 5)()
        vs = (ctypes.c_int64 * 4)()
        _check(lib().kv_pool_cache_shape(self._h, ks, vs))
        return tuple(ks), tuple(vs)

    def add_seq(self, seq_id: int):
        _check(lib().kv_pool_add_seq(self._h, seq_id))

    def share_prefix(self, seq_id: int, src_seq_id: int, n_tokens: int):
        _check(lib().kv_pool_share_prefix(self._h, seq_id, src_seq_id, n_tokens))

    def append(self, seq_id: int, n_tokens: int, out=None):
        """allocate_slots for n_tokens new tokens; returns int32 slot ids (numpy)."""
        np = self._np
        slots = np.empty(max(n_tokens, 0), dtype=np.int32) if out is None else out
        _check(lib().kv_pool_append(self._h, seq_id, n_tokens,
                                    slots.ctypes.data_as(ctypes.c_void_p)))
        return slots

    def append_batch(self, seq_ids, out=None):
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        slots = np.empty(len(ids), dtype=np.int32) if out is None else out
        _check(lib().kv_pool_append_batch(self._h, ids.ctypes.data_as(ctypes.c_void_p),
                                          len(ids), slots.ctypes.data_as(ctypes.c_void_p)))
        return slots

    def add_seq_prefix(self, seq_id: int, prompt, salt: int = 0) -> int:
        """Register seq_id starting with the cached blocks of its prompt; returns the
        number of prompt tokens found (append the rest with append_tokens)."""
        np = self._np
        p = np.ascontiguousarray(prompt, dtype=np.int32)
        n = ctypes.c_int32()
        _check(lib().kv_pool_add_seq_prefix(self._h, seq_id, p.ctypes.data_as(ctypes.c_void_p),
                                            len(p), ctypes.c_uint64(salt & (2 ** 64 - 1)),
                                            ctypes.byref(n)))
        return n.value

    def fork(self, parent_id: int, child_id: int):
        _check(lib().kv_pool_fork(self._h, parent_id, child_id))

    def append_tokens(self, seq_id: int, tokens):
        """append for tokens with known ids: (int32 slots, (old, new) block copy or None)."""
        np = self._np
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        slots = np.empty(len(t), dtype=np.int32)
        cp = np.empty(2, dtype=np.int32)
        _check(lib().kv_pool_append_tokens(self._h, seq_id, t.ctypes.data_as(ctypes.c_void_p),
                                           len(t), slots.ctypes.data_as(ctypes.c_void_p),
                                           cp.ctypes.data_as(ctypes.c_void_p)))
        return slots, (None if cp[0] < 0 else (int(cp[0]), int(cp[1])))

    def append_batch_tokens(self, seq_ids, tokens, out=None):
        """Decode step with token ids: (int32 slots, int32 [k][2] block copies)."""
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        if t.shape != ids.shape:
            raise ValueError("one token per sequence")
        slots = np.empty(len(ids), dtype=np.int32) if out is None else out
        copies = np.empty((max(len(ids), 1), 2), dtype=np.int32)
        nc = ctypes.c_int32()
        _check(lib().kv_pool_append_batch_tokens(
            self._h, ids.ctypes.data_as(ctypes.c_void_p), t.ctypes.data_as(ctypes.c_void_p),
            len(ids), slots.ctypes.data_as(ctypes.c_void_p),
            copies.ctypes.data_as(ctypes.c_void_p), ctypes.byref(nc)))
        return slots, copies[:nc.value]

    def free_seq(self, seq_id: int):
        _check(lib().kv_pool_free_seq(self._h, seq_id))

    def seq_len(self, seq_id: int) -> int:
        v = ctypes.c_int64()
        _check(lib().kv_pool_seq_len(self._h, seq_id, ctypes.byref(v)))
        return v.value

    def seq_blocks(self, seq_id: int):
        np = self._np
        n = ctypes.c_int32()
        cap = self.num_blocks
        buf = np.empty(cap, dtype=np.int32)
        _check(lib().kv_pool_seq_blocks(self._h, seq_id, buf.ctypes.data_as(ctypes.c_void_p),
                                        cap, ctypes.byref(n)))
        return buf[:n.value].tolist()

    def free_queue(self):
        np = self._np
        n = ctypes.c_int64()
        buf = np.empty(self.num_blocks, dtype=np.int32)
        _check(lib().kv_pool_free_queue(self._h, buf.ctypes.data_as(ctypes.c_void_p),
                                        self.num_blocks, ctypes.byref(n)))
        return buf[:n.value].tolist()

    def refcount(self, blk: int) -> int:
        v = ctypes.c_int32()
        _check(lib().kv_pool_refcount(self._h, blk, ctypes.byref(v)))
        return v.value

    def build_tables(self, seq_ids, max_blocks: int, tables_out=None, lens_out=None):
        """Dense int32 [n][max_blocks] tables (-1 padded) and int32 lengths, on the host
        (pass pinned numpy/torch-backed buffers to fill them in place)."""
        np = self._np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        t = np.empty((len(ids), max_blocks), dtype=np.int32) if tables_out is None else tables_out
        l = np.empty(len(ids), dtype=np.int32) if lens_out is None else lens_out
        _check(lib().kv_pool_build_tables(self._h, ids.ctypes.data_as(ctypes.c_void_p), len(ids),
                                          max_blocks, t.ctypes.data_as(ctypes.c_void_p),
                                          l.ctypes.data_as(ctypes.c_void_p)))
        return t, l

    def stats(self) -> dict:
        s = _Stats()
        _check(lib().kv_pool_stats(self._h, ctypes.byref(s)))
        return {"total": s.total_blocks, "free": s.free_blocks, "used": s.used_blocks,
                "shared": s.shared_blocks, "alloc_failures": s.alloc_failures,
                "num_seqs": s.num_seqs, "cached": s.cached_blocks,
                "prefix_hits": s.prefix_hit_blocks}


def kv_pool_create(num_blocks, num_layers, num_kv_heads, head_dim, dtype, free_order=None,
                   block_size=BLOCK_SIZE) -> KVPool:
    return KVPool(num_blocks, num_layers, num_kv_heads, head_dim, dtype, free_order, block_size)


# ------------------------------------------------------------------------ kernels
def _order(seq_order, B: int):
    """seq_order (None or a host sequence of B ints) as (pointer, keep-alive array)."""
    if seq_order is None:
        return None, None
    import numpy as np
    a = np.ascontiguousarray(seq_order, dtype=np.int32)
    if a.shape != (B,):
        raise ValueError("seq_order must hold one entry per sequence")
    return a.ctypes.data_as(ctypes.c_void_p), a


def paged_attention_decode_plan(seq_lens, num_kv_heads: int):
    """The single-pass decode order for a step (host int32 [B]) from a host copy of the
    lengths; pass it as seq_order to every layer's decode call of that step."""
    import numpy as np
    ln = np.ascontiguousarray(seq_lens, dtype=np.int32)
    order = np.empty(ln.shape[0], dtype=np.int32)
    _check(lib().paged_attention_decode_plan(ln.ctypes.data_as(ctypes.c_void_p), ln.shape[0],
                                             num_kv_heads, order.ctypes.data_as(ctypes.c_void_p)))
    return order


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """key/value: device [T][Hkv][d] (token stride free, head/dim dense); caches in the
    documented layout; slot_mapping: device int32 [T]."""
    if key.dim() != 3:
        raise ValueError("key must be [T][Hkv][d]")
    T, hkv, d = (int(x) for x in key.shape)
    _float_type(key, "key")
    _rows(key, "key", T, hkv, d)
    _rows(value, "value", T, hkv, d, key.dtype)
    _caches(k_cache, v_cache, key.dtype, hkv, d)
    _index(slot_mapping, "slot_mapping", numel_min=T)
    _same_device(key, [(value, "value"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                       (slot_mapping, "slot_mapping")])
    _check(lib().reshape_and_cache(
        _dev(key, "key"), _dev(value, "value"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping"), T, hkv, d, block_size_of(v_cache),
        k_cache.shape[0], key.stride(0), value.stride(0), dtype_code(key.dtype),
        _stream(key, stream)))


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                           partition_size: int = 0, part_out=None, part_max=None, part_sum=None,
                           max_partitions: int = 0, num_kv_heads: int | None = None,
                           stream=None, seq_order=None):
    """out/q: device [B][Hq][d] (q's sequence stride is free); block_tables int32
    [B][max_blocks]; seq_lens int32 [B]. partition_size: 0 (single pass), a multiple
    of 16 (fixed partitions) or PKV_PARTITION_AUTO (balanced split); the last two
    need fp32 partial buffers part_out [B][Hq][P][d], part_max/part_sum [B][Hq][P]
    and a paged_attention_reduce call with the same arguments. seq_order: the step's
    paged_attention_decode_plan (host), or None."""
    B, Hq, d, hkv, _, max_partitions = _decode_args(
        out, q, k_cache, v_cache, block_tables, seq_lens, partition_size, part_out, part_max,
        part_sum, max_partitions, fp8=False)
    if num_kv_heads is not None and num_kv_heads != hkv:
        raise ValueError(f"num_kv_heads {num_kv_heads} differs from the caches' {hkv}")
    op, _keep = _order(seq_order, B)
    _check(lib().paged_attention_decode(
        _dev(out, "out"), _dev(part_out, "part_out"), _dev(part_max, "part_max"),
        _dev(part_sum, "part_sum"), _dev(q, "q"), q.stride(0), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"),
        B, Hq, hkv, d, block_size_of(v_cache), block_tables.shape[1], k_cache.shape[0], float(scale),
        partition_size, max_partitions, dtype_code(q.dtype), dtype_code(out.dtype), op,
        _stream(q, stream)))


def paged_attention_decode_append(out, q, key, value, slot_mapping, k_cache, v_cache,
                                  block_tables, seq_lens, scale: float, partition_size: int = 0,
                                  part_out=None, part_max=None, part_sum=None,
                                  max_partitions: int = 0, stream=None, seq_order=None):
    """reshape_and_cache of one new token per sequence (key/value [B][Hkv][d], their
    slots in slot_mapping int32 [B]) fused with paged_attention_decode over seq_lens,
    which count the new token. Same outputs and follow-up reduce as
    paged_attention_decode."""
    B, Hq, d, hkv, _, max_partitions = _decode_args(
        out, q, k_cache, v_cache, block_tables, seq_lens, partition_size, part_out, part_max,
        part_sum, max_partitions, fp8=False, append=(key, value, slot_mapping))
    op, _keep = _order(seq_order, B)
    _check(lib().paged_attention_decode_append(
        _dev(out, "out"), _dev(part_out, "part_out"), _dev(part_max, "part_max"),
        _dev(part_sum, "part_sum"), _dev(q, "q"), q.stride(0), _dev(key, "key"),
        _dev(value, "value"), key.stride(0), value.stride(0), _dev(slot_mapping, "slot_mapping"),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
        _dev(seq_lens, "seq_lens"), B, Hq, hkv, d, block_size_of(v_cache), block_tables.shape[1],
        k_cache.shape[0], float(scale), partition_size, max_partitions, dtype_code(q.dtype),
        dtype_code(out.dtype), op, _stream(q, stream)))


def paged_attention_decode_noalloc(out, q, k_cache, v_cache, block_tables, seq_lens,
                                   scale: float, partition_size: int = PKV_PARTITION_AUTO,
                                   stream=None):
    """A partitioned decode and its reduce in one call with no device allocation: the
    partition records live in the library's static per-device workspace (calls that
    overlap on one device race on it). partition_size: a multiple of 16 or
    PKV_PARTITION_AUTO (0: the single pass)."""
    B, Hq, d, hkv, bs, _ = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, 0,
                                        None, None, None, 0, fp8=False)
    _check(lib().paged_attention_decode_noalloc(
        _dev(out, "out"), _dev(q, "q"), q.stride(0), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"),
        B, Hq, hkv, d, bs, block_tables.shape[1], k_cache.shape[0], float(scale), partition_size,
        dtype_code(q.dtype), dtype_code(out.dtype), _stream(q, stream)))


def noalloc_workspace_bytes() -> int:
    """Bytes of the static per-device workspace of paged_attention_decode_noalloc."""
    return int(lib().paged_attention_decode_noalloc_workspace())


# ------------------------------------------------------------------ FP8 cache
def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale: float,
                          v_scale: float, stream=None):
    """reshape_and_cache into an FP8 cache: the e4m3 codes of key / k_scale and
    value / v_scale (key/value fp16 or bf16 [T][Hkv][d])."""
    torch = _torch()
    if key.dim() != 3:
        raise ValueError("key must be [T][Hkv][d]")
    T, hkv, d = (int(x) for x in key.shape)
    _float_type(key, "key")
    _rows(key, "key", T, hkv, d)
    _rows(value, "value", T, hkv, d, key.dtype)
    _caches(k_cache, v_cache, torch.uint8, hkv, d)
    _index(slot_mapping, "slot_mapping", numel_min=T)
    _same_device(key, [(value, "value"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                       (slot_mapping, "slot_mapping")])
    _check(lib().reshape_and_cache_fp8(
        _dev(key, "key"), _dev(value, "value"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(slot_mapping, "slot_mapping"), T, hkv, d, block_size_of(v_cache),
        k_cache.shape[0], key.stride(0), value.stride(0), dtype_code(key.dtype), float(k_scale),
        float(v_scale), _stream(key, stream)))


def paged_attention_decode_fp8(out, q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                               k_scale: float, v_scale: float, partition_size: int = 0,
                               part_out=None, part_max=None, part_sum=None,
                               max_partitions: int = 0, stream=None, seq_order=None):
    """paged_attention_decode over an FP8 cache (codes times k_scale / v_scale)."""
    B, Hq, d, hkv, _, max_partitions = _decode_args(
        out, q, k_cache, v_cache, block_tables, seq_lens, partition_size, part_out, part_max,
        part_sum, max_partitions, fp8=True)
    op, _keep = _order(seq_order, B)
    _check(lib().paged_attention_decode_fp8(
        _dev(out, "out"), _dev(part_out, "part_out"), _dev(part_max, "part_max"),
        _dev(part_sum, "part_sum"), _dev(q, "q"), q.stride(0), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"),
        B, Hq, k_cache.shape[1], d, block_size_of(v_cache), block_tables.shape[1], k_cache.shape[0],
        float(scale), float(k_scale), float(v_scale), partition_size, max_partitions,
        dtype_code(q.dtype), dtype_code(out.dtype), op, _stream(q, stream)))


def paged_attention_decode_append_fp8(out, q, key, value, slot_mapping, k_cache, v_cache,
                                      block_tables, seq_lens, scale: float, k_scale: float,
                                      v_scale: float, partition_size: int = 0, part_out=None,
                                      part_max=None, part_sum=None, max_partitions: int = 0,
                                      stream=None, seq_order=None):
    """paged_attention_decode_append over an FP8 cache: the new rows are stored as
    codes and attended to as their stored values."""
    B, Hq, d, hkv, _, max_partitions = _decode_args(
        out, q, k_cache, v_cache, block_tables, seq_lens, partition_size, part_out, part_max,
        part_sum, max_partitions, fp8=True, append=(key, value, slot_mapping))
    op, _keep = _order(seq_order, B)
    _check(lib().paged_attention_decode_append_fp8(
        _dev(out, "out"), _dev(part_out, "part_out"), _dev(part_max, "part_max"),
        _dev(part_sum, "part_sum"), _dev(q, "q"), q.stride(0), _dev(key, "key"),
        _dev(value, "value"), key.stride(0), value.stride(0), _dev(slot_mapping, "slot_mapping"),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
        _dev(seq_lens, "seq_lens"), B, Hq, hkv, d, block_size_of(v_cache), block_tables.shape[1],
        k_cache.shape[0], float(scale), float(k_scale), float(v_scale), partition_size,
        max_partitions, dtype_code(q.dtype), dtype_code(out.dtype), op, _stream(q, stream)))


def paged_attention_prefill(out, q, q_start, k_cache, v_cache, block_tables, seq_lens,
                            scale: float, max_q_len: int, stream=None):
    """Causal multi-query attention (chunked prefill): q/out [T][Hq][d] hold every
    sequence's chunk back to back, sequence b in rows q_start[b] .. q_start[b+1]-1 (device
    int32 [B+1]); the chunk is the last positions of seq_lens[b] and its K/V is already in
    the cache. max_q_len bounds the chunk lengths (host value)."""
    if q.dim() != 3:
        raise ValueError("q must be [T][Hq][d]")
    T, Hq, d = (int(x) for x in q.shape)
    _float_type(q, "q")
    _rows(q, "q", T, Hq, d)
    if tuple(out.shape) != (T, Hq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [T][Hq][d] tensor")
    _float_type(out, "out")
    _, hkv, _, _ = _caches(k_cache, v_cache, q.dtype, head_dim=d)
    if Hq % hkv:
        raise ValueError(f"num_heads {Hq} is not a multiple of the caches' {hkv} KV heads")
    B = seq_lens.numel()
    _index(seq_lens, "seq_lens", shape=(B,))
    _index(q_start, "q_start", shape=(B + 1,))
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError(f"block_tables must be [{B}][max_blocks], got {tuple(block_tables.shape)}")
    _index(block_tables, "block_tables")
    _same_device(q, [(out, "out"), (q_start, "q_start"), (k_cache, "k_cache"),
                     (v_cache, "v_cache"), (block_tables, "block_tables"), (seq_lens, "seq_lens")])
    _check(lib().paged_attention_prefill(
        _dev(out, "out"), _dev(q, "q"), q.stride(0), _dev(q_start, "q_start"),
        _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
        _dev(seq_lens, "seq_lens"), B, int(max_q_len), Hq, k_cache.shape[1], d, block_size_of(v_cache),
        block_tables.shape[1], k_cache.shape[0], float(scale), dtype_code(q.dtype),
        dtype_code(out.dtype), _stream(q, stream)))


def copy_blocks(k_caches, v_caches, pairs, stream=None):
    """Copy-on-write on the device: for each (src, dst) row of pairs (device int32
    [n][2]), block src onto block dst in every layer's K and V cache (lists of tensors)."""
    L = len(k_caches)
    if L != len(v_caches) or L == 0:
        raise ValueError("one K and one V cache per layer")
    for t in list(k_caches) + list(v_caches):
        if not t.is_contiguous() or t.shape[0] != k_caches[0].shape[0]:
            raise ValueError("caches must be contiguous with the same number of blocks")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise ValueError("pairs must be a contiguous [n][2] int32 tensor")
    _index(pairs, "pairs")
    for group in (k_caches, v_caches):
        for t in group:
            if t.dtype != k_caches[0].dtype or tuple(t.shape) != tuple(group[0].shape):
                raise ValueError("every layer's caches must have the same type and shape")
    _same_device(pairs, [(t, "cache") for t in list(k_caches) + list(v_caches)])
    kp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in k_caches])
    vp = (ctypes.c_void_p * L)(*[t.data_ptr() for t in v_caches])
    block_bytes = k_caches[0][0].numel() * k_caches[0].element_size()
    _check(lib().copy_blocks(kp, vp, L, _dev(pairs, "pairs"), pairs.shape[0], block_bytes,
                             k_caches[0].shape[0], _stream(pairs, stream)))


def paged_attention_reduce(out, part_out, part_max, part_sum, seq_lens, partition_size: int,
                           num_kv_heads: int, max_blocks_per_seq: int,
                           block_size: int = BLOCK_SIZE, stream=None):
    if out.dim() != 3 or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B][Hq][d] tensor")
    B, Hq, d = (int(x) for x in out.shape)
    _float_type(out, "out")
    if partition_size == 0:
        raise ValueError("paged_attention_reduce follows a partitioned decode (partition_size != 0)")
    P = _partials(part_out, part_max, part_sum, B, Hq, d, partition_size, 0)
    _index(seq_lens, "seq_lens", shape=(B,))
    _same_device(out, [(part_out, "part_out"), (part_max, "part_max"), (part_sum, "part_sum"),
                       (seq_lens, "seq_lens")])
    _check(lib().paged_attention_reduce(
        _dev(out, "out"), _dev(part_out, "part_out"), _dev(part_max, "part_max"),
        _dev(part_sum, "part_sum"), _dev(seq_lens, "seq_lens"), B, Hq, num_kv_heads, d,
        block_size, max_blocks_per_seq, partition_size, P, dtype_code(out.dtype),
        _stream(out, stream)))


# ------------------------------------------------------------------ kernel timer
PKV_TIMER_DECODE, PKV_TIMER_REDUCE, PKV_TIMER_CACHE_WRITE, PKV_TIMER_COPY_BLOCKS = 0, 1, 2, 3
PKV_TIMER_PREFILL = 4
PKV_TIMER_MEASURE = 5


def measure_read(buf, sink, waves_per_cu: int = 8, loads_in_flight: int = 8,
                 nontemporal: bool = True, stream=None):
    """Streaming ceiling (a measuring aid): read every byte of the device tensor buf once,
    contiguously, with no arithmetic (timed under PKV_TIMER_MEASURE)."""
    _index(sink, "sink")
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    _check(lib().pkv_measure_read(_dev(buf, "buf"), buf.numel() * buf.element_size(),
                                  waves_per_cu, loads_in_flight, 1 if nontemporal else 0,
                                  _dev(sink, "sink"), sink.numel(),
                                  _stream(buf, stream)))


def measure_gather(k_cache, v_cache, block_tables, seq_lens, sink, seq_order=None,
                   balanced: bool = False, nontemporal: bool = True, stream=None):
    """Gather ceiling (a measuring aid): read the K/V tiles a decode of this batch reads,
    through the block tables, with no arithmetic (timed under PKV_TIMER_MEASURE)."""
    torch = _torch()
    nb, hkv, d, bs = _caches(k_cache, v_cache, k_cache.dtype)
    B = seq_lens.numel()
    _index(seq_lens, "seq_lens", shape=(B,))
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be [B][max_blocks]")
    _index(block_tables, "block_tables")
    _index(sink, "sink")
    _same_device(k_cache, [(v_cache, "v_cache"), (block_tables, "block_tables"),
                           (seq_lens, "seq_lens"), (sink, "sink")])
    op, _keep = _order(seq_order, B)
    code = PKV_FP8_E4M3 if k_cache.dtype == torch.uint8 else dtype_code(k_cache.dtype)
    _check(lib().pkv_measure_gather(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                    _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"),
                                    B, hkv, d, bs, code, block_tables.shape[1], nb, op,
                                    1 if balanced else 0, 1 if nontemporal else 0,
                                    _dev(sink, "sink"), sink.numel(),
                                    _stream(k_cache, stream)))


RATE_KINDS = ("lds_read", "exp", "fma", "mfma", "mfma_exp", "mfma_fma", "mfma_16x16x16")


def measure_rate(kind: str, waves_per_simd: int, iters: int, sink, stream=None):
    """Unit rates (a measuring aid): kind in RATE_KINDS, waves_per_simd waves on every SIMD,
    iters iterations each (timed under PKV_TIMER_MEASURE); see pkv_measure_rate."""
    _index(sink, "sink")
    _check(lib().pkv_measure_rate(RATE_KINDS.index(kind), int(waves_per_simd), int(iters),
                                  _dev(sink, "sink"), sink.numel(), _stream(sink, stream)))


def timer_enable(on: bool = True):
    """Bind HIP start/stop events to every later launch of the library's kernels."""
    _check(lib().pkv_timer_enable(1 if on else 0))


def timer_read(entry: int):
    """(summed kernel milliseconds, launches) of one entry since its last read."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib().pkv_timer_read(entry, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def max_partitions_for(max_blocks: int, partition_size: int, block_size: int = BLOCK_SIZE) -> int:
    """Partial slots per (b, h): ceil(max_blocks*BS / P) for fixed partitions; for the
    balanced split a bound that keeps every piece at least four 16-token tiles long."""
    if partition_size == PKV_PARTITION_AUTO:
        tiles = -(-max_blocks * block_size // 16)
        return max(2, -(-tiles // 4) + 1)
    return -(-max_blocks * block_size // partition_size)


def alloc_partials(B: int, Hq: int, d: int, max_partitions: int, device="cuda"):
    torch = _torch()
    return (torch.empty((B, Hq, max_partitions, d), dtype=torch.float32, device=device),
            torch.empty((B, Hq, max_partitions), dtype=torch.float32, device=device),
            torch.empty((B, Hq, max_partitions), dtype=torch.float32, device=device))


def decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale: float,
           partition_size: int = 0, partials=None, stream=None, append=None, kv_scales=None,
           seq_order=None):
    """Decode + (if partitioned or balanced) reduce: the launches of one layer's attention.
    append=(key, value, slot_mapping) writes one new token per sequence first, fused
    (paged_attention_decode_append). kv_scales=(k_scale, v_scale): the caches are FP8.
    seq_order: the step's paged_attention_decode_plan (host), or None."""
    po, pm, ps = partials if partition_size != 0 else (None, None, None)
    maxp = po.shape[2] if po is not None else 0
    if kv_scales is not None:
        ks, vs = kv_scales
        if append is not None:
            key, value, slots = append
            paged_attention_decode_append_fp8(out, q, key, value, slots, k_cache, v_cache,
                                              block_tables, seq_lens, scale, ks, vs,
                                              partition_size, po, pm, ps, maxp, stream=stream,
                                              seq_order=seq_order)
        else:
            paged_attention_decode_fp8(out, q, k_cache, v_cache, block_tables, seq_lens, scale,
                                       ks, vs, partition_size, po, pm, ps, maxp, stream=stream,
                                       seq_order=seq_order)
    elif append is not None:
        key, value, slots = append
        paged_attention_decode_append(out, q, key, value, slots, k_cache, v_cache, block_tables,
                                      seq_lens, scale, partition_size, po, pm, ps, maxp,
                                      stream=stream, seq_order=seq_order)
    else:
        paged_attention_decode(out, q, k_cache, v_cache, block_tables, seq_lens, scale,
                               partition_size, po, pm, ps, maxp, stream=stream,
                               seq_order=seq_order)
    if partition_size != 0:
        paged_attention_reduce(out, po, pm, ps, seq_lens, partition_size, k_cache.shape[1],
                               block_tables.shape[1], block_size_of(v_cache), stream=stream)
