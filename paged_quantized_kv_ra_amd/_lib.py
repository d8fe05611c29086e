"""ctypes binding of libra_kv.so (C ABI in include/ra_kv.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch provides device memory and the current stream.  torch is
imported before the library is loaded so that libra_kv.so binds to the HIP
runtime torch already mapped (one runtime per process).

KV caches are torch tensors of shape [num_pages, num_kv_heads, 16 * head_dim]
holding the library's paged layout: dtype float16 for FP16 caches, uint8 for
E4M3 and INT8 codes.
"""
import ctypes
import math
import os

import torch

# RA_KV_LIB selects another build of the library (same ABI); default: the in-tree one
LIB_PATH = os.environ.get("RA_KV_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libra_kv.so")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_MISALIGNED, RA_ERR_WORKSPACE, RA_ERR_HIP = range(6)
RA_F16, RA_BF16, RA_F32 = 1, 2, 3
RA_KV_F16, RA_KV_FP8_E4M3, RA_KV_INT8, RA_KV_INT8_TOKEN = 1, 2, 3, 4
KV_CODES = {"f16": RA_KV_F16, "e4m3": RA_KV_FP8_E4M3, "int8": RA_KV_INT8, "int8_tok": RA_KV_INT8_TOKEN}
PAGE = 16

_c = ctypes
_vp = _c.c_void_p


class AttnArgs(_c.Structure):
    """Mirror of ra_attn_args."""
    _fields_ = [
        ("struct_size", _c.c_uint32),
        ("q_dtype", _c.c_int32),
        ("q", _vp),
        ("out", _vp),
        ("lse", _vp),
        ("k_cache", _vp),
        ("v_cache", _vp),
        ("kv_dtype", _c.c_int32),
        ("k_scale", _c.c_float),
        ("v_scale", _c.c_float),
        ("block_tables", _vp),
        ("block_table_stride", _c.c_int32),
        ("context_lens", _vp),
        ("query_start_loc", _vp),
        ("batch", _c.c_int32),
        ("total_q", _c.c_int32),
        ("num_q_heads", _c.c_int32),
        ("num_kv_heads", _c.c_int32),
        ("head_dim", _c.c_int32),
        ("page_size", _c.c_int32),
        ("num_pages", _c.c_int64),
        ("max_q_len", _c.c_int32),
        ("min_q_len", _c.c_int32),
        ("max_context_len", _c.c_int32),
        ("softmax_scale", _c.c_float),
        ("window_left", _c.c_int32),
        ("num_sinks", _c.c_int32),
        ("num_splits", _c.c_int32),
        ("partial_out", _vp),
        ("partial_lse", _vp),
        ("partial_slots", _c.c_int32),
        ("k_scales", _vp),
        ("v_scales", _vp),
        ("kv_pos0", _vp),
        ("q_pos0", _vp),
        ("new_k", _vp),
        ("new_v", _vp),
        ("new_dtype", _c.c_int32),
        ("new_k_stride", _c.c_int64),
        ("new_v_stride", _c.c_int64),
        ("new_slots", _vp),
        ("q_token_stride", _c.c_int64),
        ("rope_table", _vp),
        ("rope_max_position", _c.c_int32),
        ("rotary_dim", _c.c_int32),
        ("positions", _vp),
    ]


class RopeArgs(_c.Structure):
    """Mirror of ra_qkv_rope_args."""
    _fields_ = [
        ("struct_size", _c.c_uint32),
        ("qkv", _vp),
        ("src_dtype", _c.c_int32),
        ("qkv_token_stride", _c.c_int64),
        ("num_tokens", _c.c_int64),
        ("positions", _vp),
        ("rope_table", _vp),
        ("max_position", _c.c_int32),
        ("rotary_dim", _c.c_int32),
        ("q_out", _vp),
        ("q_token_stride", _c.c_int64),
        ("slot_mapping", _vp),
        ("k_cache", _vp),
        ("v_cache", _vp),
        ("kv_dtype", _c.c_int32),
        ("k_scale", _c.c_float),
        ("v_scale", _c.c_float),
        ("k_scales", _vp),
        ("v_scales", _vp),
        ("num_pages", _c.c_int64),
        ("num_q_heads", _c.c_int32),
        ("num_kv_heads", _c.c_int32),
        ("head_dim", _c.c_int32),
        ("page_size", _c.c_int32),
    ]


EXPORTED = {
    "ra_kv_store": (_c.c_int32, [_vp, _vp, _c.c_int32, _c.c_int64, _c.c_int64, _vp, _c.c_int64, _vp, _vp,
                                 _c.c_int32, _c.c_int64, _c.c_int32, _c.c_int32, _c.c_int32, _c.c_float,
                                 _c.c_float, _vp]),
    "ra_kv_store_int8_token": (_c.c_int32, [_vp, _vp, _c.c_int32, _c.c_int64, _c.c_int64, _vp, _c.c_int64, _vp,
                                            _vp, _vp, _vp, _c.c_int64, _c.c_int32, _c.c_int32, _c.c_int32, _vp]),
    "ra_paged_attn": (_c.c_int32, [_c.POINTER(AttnArgs), _vp]),
    "ra_paged_attn_noalloc": (_c.c_int32, [_c.POINTER(AttnArgs), _vp]),
    "ra_paged_attn_workspace": (_c.c_int32, [_c.POINTER(AttnArgs), _c.POINTER(_c.c_int32),
                                             _c.POINTER(_c.c_int64), _c.POINTER(_c.c_int64)]),
    "ra_lse_merge": (_c.c_int32, [_vp, _vp, _c.c_int32, _c.c_int64, _c.c_int32, _vp, _c.c_int32, _vp, _vp]),
    "ra_kv_gather_dequant": (_c.c_int32, [_vp, _c.c_int32, _c.c_int32, _c.c_float, _vp, _vp, _c.c_int32,
                                          _c.c_int64, _c.c_int32, _c.c_int32, _vp, _vp]),
    "ra_rope_table": (_c.c_int32, [_vp, _c.c_int32, _c.c_int32, _c.c_double, _c.c_double, _c.c_int32,
                                   _c.c_double, _c.c_double]),
    "ra_qkv_rope_store": (_c.c_int32, [_c.POINTER(RopeArgs), _vp]),
    "ra_last_error": (_c.c_char_p, []),
    "ra_abi_version": (_c.c_int32, []),
}

_LIB = None


class RaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


def load_library():
    """Load libra_kv.so (built in-tree); raise if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m paged_quantized_kv_ra_amd.build`")
        lib = _c.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTED.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = lib
    return _LIB


def _check(status):
    if status != RA_OK:
        raise RaError(status, load_library().ra_last_error().decode())


def _ptr(t):
    return None if t is None else _vp(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return _vp(stream.cuda_stream)


def abi_version():
    return load_library().ra_abi_version()


def _elem_bytes(kv_dtype):
    return 2 if kv_dtype == "f16" else 1


def new_cache(num_pages, num_kv_heads, head_dim, kv_dtype, device="cuda", fill=None):
    """Allocate one K or V cache tensor in the library's layout."""
    dt = torch.float16 if kv_dtype == "f16" else torch.uint8
    t = torch.empty((num_pages, num_kv_heads, PAGE * head_dim), dtype=dt, device=device)
    if fill is not None:
        if kv_dtype == "f16":
            t.view(torch.int16).fill_(fill if fill < 0x8000 else fill - 0x10000)
        else:
            t.fill_(fill)
    return t


def new_scale_plane(num_pages, num_kv_heads, device="cuda", fill=float("nan")):
    """Allocate one per-token INT8 scale plane [num_pages][num_kv_heads][16] fp32."""
    return torch.full((num_pages, num_kv_heads, PAGE), fill, dtype=torch.float32, device=device)


def _src_code(t):
    if t.dtype == torch.float16:
        return RA_F16
    if t.dtype == torch.bfloat16:
        return RA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def kv_store(k, v, slot_mapping, k_cache, v_cache, kv_dtype, k_scale=1.0, v_scale=1.0, stream=None,
             k_scales=None, v_scales=None):
    """Quantise k, v [T][Hkv][D] and scatter them into the caches at slot_mapping
    (per-token INT8: also their scales into the k_scales / v_scales planes)."""
    T, hkv, D = k.shape
    assert v.shape == k.shape and k.stride(2) == 1 and k.stride(1) == D and v.stride(2) == 1 and v.stride(1) == D
    assert slot_mapping.dtype == torch.int64 and slot_mapping.numel() == T
    num_pages = k_cache.shape[0]
    if kv_dtype == "int8_tok":
        _check(load_library().ra_kv_store_int8_token(
            _ptr(k), _ptr(v), _src_code(k), k.stride(0), v.stride(0), _ptr(slot_mapping), T,
            _ptr(k_cache), _ptr(v_cache), _ptr(k_scales), _ptr(v_scales), num_pages, hkv, D, PAGE,
            _stream(stream)))
        return
    _check(load_library().ra_kv_store(
        _ptr(k), _ptr(v), _src_code(k), k.stride(0), v.stride(0), _ptr(slot_mapping), T,
        _ptr(k_cache), _ptr(v_cache), KV_CODES[kv_dtype], num_pages, hkv, D, PAGE,
        float(k_scale), float(v_scale), _stream(stream)))


def _attn_args(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, kv_dtype, k_scale,
               v_scale, softmax_scale, max_q_len, min_q_len, max_context_len, window_left, num_sinks,
               num_splits, num_kv_heads, k_scales=None, v_scales=None, kv_pos0=None, q_pos0=None, new_k=None,
               new_v=None, new_slots=None, rope_table=None, positions=None, rotary_dim=None):
    T, hq, D = q.shape
    assert q.stride(2) == 1 and q.stride(1) == D, "query heads must be contiguous rows of head_dim"
    a = AttnArgs()
    a.struct_size = _c.sizeof(AttnArgs)
    a.q_dtype = _src_code(q)
    a.q = q.data_ptr()
    a.k_cache = k_cache.data_ptr()
    a.v_cache = v_cache.data_ptr()
    a.kv_dtype = KV_CODES[kv_dtype]
    a.k_scale = float(k_scale)
    a.v_scale = float(v_scale)
    a.block_tables = block_tables.data_ptr()
    a.block_table_stride = block_tables.shape[1]
    a.context_lens = context_lens.data_ptr()
    a.query_start_loc = query_start_loc.data_ptr()
    a.batch = context_lens.shape[0]
    a.total_q = T
    a.num_q_heads = hq
    a.num_kv_heads = num_kv_heads
    a.head_dim = D
    a.page_size = PAGE
    a.num_pages = k_cache.shape[0]
    a.max_q_len = int(max_q_len)
    a.min_q_len = int(min_q_len)
    a.max_context_len = int(max_context_len)
    a.softmax_scale = float(softmax_scale if softmax_scale is not None else 1.0 / math.sqrt(D))
    a.window_left = int(window_left)
    a.num_sinks = int(num_sinks)
    a.num_splits = int(num_splits)
    a.k_scales = None if k_scales is None else k_scales.data_ptr()
    a.v_scales = None if v_scales is None else v_scales.data_ptr()
    a.kv_pos0 = None if kv_pos0 is None else kv_pos0.data_ptr()
    a.q_pos0 = None if q_pos0 is None else q_pos0.data_ptr()
    if new_k is not None:            # fused store of the query tokens' K/V
        assert new_v is not None and new_slots is not None and new_slots.dtype == torch.int64
        assert new_k.stride(-1) == 1 and new_v.stride(-1) == 1 and new_k.dtype == new_v.dtype
        a.new_k = new_k.data_ptr()
        a.new_v = new_v.data_ptr()
        a.new_dtype = _src_code(new_k)
        a.new_k_stride = new_k.stride(0)
        a.new_v_stride = new_v.stride(0)
        a.new_slots = new_slots.data_ptr()
    a.q_token_stride = q.stride(0) if q.stride(0) != hq * D else 0
    if rope_table is not None:       # RoPE on the fused path
        assert rope_table.dtype == torch.float32 and rope_table.is_contiguous() and positions.dtype == torch.int64
        a.rope_table = rope_table.data_ptr()
        a.rope_max_position = rope_table.shape[0]
        a.rotary_dim = int(rotary_dim if rotary_dim is not None else rope_table.shape[2] * 2)
        a.positions = positions.data_ptr()
    return a


def paged_attn_workspace(args):
    slots = _c.c_int32()
    po = _c.c_int64()
    pl = _c.c_int64()
    _check(load_library().ra_paged_attn_workspace(_c.byref(args), _c.byref(slots), _c.byref(po), _c.byref(pl)))
    return slots.value, po.value, pl.value


def paged_attn(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, *, kv_dtype,
               max_q_len, max_context_len, k_scale=1.0, v_scale=1.0, softmax_scale=None, min_q_len=0,
               window_left=-1, num_sinks=0, num_splits=0, out=None, lse=None, partials_only=False,
               workspace=None, stream=None, k_scales=None, v_scales=None, kv_pos0=None, q_pos0=None,
               new_k=None, new_v=None, new_slots=None, rope_table=None, positions=None, rotary_dim=None,
               no_alloc=False):
    """Attention of the query blocks over the paged caches.

    q [total_q][Hq][D] fp16/bf16; block_tables int32 [B][stride];
    context_lens int32 [B]; query_start_loc int32 [B+1].  max_q_len and
    max_context_len are host upper bounds.  Returns (out, lse), or with
    partials_only=True (partial_out [S][total_q][Hq][D], partial_lse [S][total_q][Hq]).
    new_k, new_v [total_q][Hkv][D] and new_slots int64 [total_q]: the query
    tokens' own K/V, stored by the launch itself (decode and verify blocks).
    rope_table [P][2][R/2] fp32 and positions int64 [total_q] (with new_k):
    q and new_k are rotated by RoPE inside the launch.  q may be a view into
    packed QKV rows (its token stride is passed on).
    no_alloc=True calls ra_paged_attn_noalloc: the partials of a split call
    stay in the library's static scratch and no workspace is allocated (out
    and lse are still allocated here unless passed in).
    """
    T, hq, D = q.shape
    hkv = k_cache.shape[1]
    a = _attn_args(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, kv_dtype, k_scale,
                   v_scale, softmax_scale, max_q_len, min_q_len, max_context_len, window_left, num_sinks,
                   num_splits, hkv, k_scales, v_scales, kv_pos0, q_pos0, new_k, new_v, new_slots, rope_table,
                   positions, rotary_dim)
    if not partials_only:
        if out is None:
            out = torch.empty((T, hq, D), dtype=q.dtype, device=q.device)
        if lse is None:
            lse = torch.empty((T, hq), dtype=torch.float32, device=q.device)
        a.out = out.data_ptr()
        a.lse = lse.data_ptr()
    if no_alloc:
        if partials_only:
            raise ValueError("no_alloc keeps the partials in the library's scratch: partials_only is not available")
        _check(load_library().ra_paged_attn_noalloc(_c.byref(a), _stream(stream)))
        return out, lse
    slots, po_n, pl_n = paged_attn_workspace(a)
    po = pl = None
    if po_n > 0 or partials_only:
        if workspace is not None:
            po, pl = workspace
        else:
            po = torch.empty((slots, T, hq, D), dtype=torch.float32, device=q.device)
            pl = torch.empty((slots, T, hq), dtype=torch.float32, device=q.device)
        a.partial_out = po.data_ptr()
        a.partial_lse = pl.data_ptr()
        a.partial_slots = po.shape[0]
    _check(load_library().ra_paged_attn(_c.byref(a), _stream(stream)))
    if partials_only:
        return po, pl
    return out, lse


def lse_merge(partial_out, partial_lse, out_dtype=torch.float32, out=None, lse=None, stream=None):
    """Merge partials [S][rows...][D] / [S][rows...] into (out [rows...][D], lse [rows...])."""
    S = partial_out.shape[0]
    D = partial_out.shape[-1]
    rows = partial_lse[0].numel()
    code = {torch.float16: RA_F16, torch.bfloat16: RA_BF16, torch.float32: RA_F32}[out_dtype]
    if out is None:
        out = torch.empty(partial_out.shape[1:], dtype=out_dtype, device=partial_out.device)
    if lse is None:
        lse = torch.empty(partial_lse.shape[1:], dtype=torch.float32, device=partial_out.device)
    _check(load_library().ra_lse_merge(_ptr(partial_out), _ptr(partial_lse), S, rows, D, _ptr(out), code,
                                       _ptr(lse), _stream(stream)))
    return out, lse


def kv_gather_dequant(cache, which, kv_dtype, scale, block_table_row, ctx, head_dim, stream=None, scales=None):
    """Exact dequantised [ctx][Hkv][D] fp32 read-back of one sequence's K (which=0) or V (1)."""
    hkv = cache.shape[1]
    out = torch.empty((ctx, hkv, head_dim), dtype=torch.float32, device=cache.device)
    _check(load_library().ra_kv_gather_dequant(_ptr(cache), which, KV_CODES[kv_dtype], float(scale), _ptr(scales),
                                               _ptr(block_table_row), ctx, cache.shape[0], hkv, head_dim,
                                               _ptr(out), _stream(stream)))
    return out


def rope_table(max_position, rotary_dim, base, factor=1.0, original_max_position=0, beta_fast=32.0,
               beta_slow=1.0, device="cuda"):
    """The library's RoPE / YaRN table [max_position][2][rotary_dim / 2] fp32,
    built on the host and copied to `device` (None: keep the host tensor)."""
    t = torch.empty((max_position, 2, rotary_dim // 2), dtype=torch.float32)
    _check(load_library().ra_rope_table(_vp(t.data_ptr()), max_position, rotary_dim, float(base), float(factor),
                                        int(original_max_position), float(beta_fast), float(beta_slow)))
    return t if device is None else t.to(device)


def _rope_args(qkv, positions, table, rotary_dim, num_q_heads, num_kv_heads, head_dim, q_out, slot_mapping,
               k_cache, v_cache, kv_dtype, k_scale, v_scale, k_scales, v_scales):
    a = RopeArgs()
    a.struct_size = _c.sizeof(RopeArgs)
    a.qkv = qkv.data_ptr()
    a.src_dtype = _src_code(qkv)
    a.qkv_token_stride = qkv.stride(0)
    a.num_tokens = qkv.shape[0]
    a.positions = positions.data_ptr()
    a.rope_table = table.data_ptr()
    a.max_position = table.shape[0]
    a.rotary_dim = int(rotary_dim)
    a.q_out = q_out.data_ptr()
    a.q_token_stride = q_out.stride(0)
    a.slot_mapping = slot_mapping.data_ptr()
    a.k_cache = k_cache.data_ptr()
    a.v_cache = v_cache.data_ptr()
    a.kv_dtype = KV_CODES[kv_dtype]
    a.k_scale = float(k_scale)
    a.v_scale = float(v_scale)
    a.k_scales = None if k_scales is None else k_scales.data_ptr()
    a.v_scales = None if v_scales is None else v_scales.data_ptr()
    a.num_pages = k_cache.shape[0]
    a.num_q_heads = num_q_heads
    a.num_kv_heads = num_kv_heads
    a.head_dim = head_dim
    a.page_size = PAGE
    return a


def qkv_rope_store(qkv, positions, table, slot_mapping, k_cache, v_cache, kv_dtype, *, num_q_heads,
                   rotary_dim=None, k_scale=1.0, v_scale=1.0, k_scales=None, v_scales=None, q_out=None,
                   stream=None):
    """Packed QKV rows [T][(Hq + 2 Hkv) * D] -> rotated Q [T][Hq][D] (returned),
    rotated K and V stored into the caches at slot_mapping."""
    T = qkv.shape[0]
    hkv = k_cache.shape[1]
    D = k_cache.shape[2] // PAGE
    assert qkv.stride(-1) == 1 and qkv.shape[1] >= (num_q_heads + 2 * hkv) * D
    assert positions.dtype == torch.int64 and slot_mapping.dtype == torch.int64
    assert table.dtype == torch.float32 and table.is_contiguous()
    rot = table.shape[2] * 2 if rotary_dim is None else rotary_dim
    assert table.shape[1] == 2 and table.shape[2] * 2 == rot
    if q_out is None:
        q_out = torch.empty((T, num_q_heads, D), dtype=qkv.dtype, device=qkv.device)
    a = _rope_args(qkv, positions, table, rot, num_q_heads, hkv, D, q_out, slot_mapping, k_cache, v_cache,
                   kv_dtype, k_scale, v_scale, k_scales, v_scales)
    _check(load_library().ra_qkv_rope_store(_c.byref(a), _stream(stream)))
    return q_out
