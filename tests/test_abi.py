"""C ABI checks that run without a GPU.

* libra_kv.so loads and exports every function include/ra_kv.h declares;
* the ctypes mirror of ra_attn_args has the C layout (sizeof / offsetof from
  a C program compiled against the header with gcc);
* every host-side validation path returns its status and message before any
  HIP call (fake, never-dereferenced pointers are passed).
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "ra_kv.h")


def _lib():
    from paged_quantized_kv_ra_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libra_kv.so not built")
    return L


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = _lib()
    lib = L.load_library()
    names = declared_functions()
    assert len(names) >= 7
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.EXPORTED, f"{n} has no ctypes prototype"
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, re.M), n


def test_abi_version():
    L = _lib()
    assert L.abi_version() == 7001


@pytest.mark.parametrize("cname,pyname", [("ra_attn_args", "AttnArgs"), ("ra_qkv_rope_args", "RopeArgs")])
def test_struct_layout_matches_c(cname, pyname):
    L = _lib()
    S = getattr(L, pyname)
    fields = [f for f, _ in S._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "ra_kv.h"', 'int main(void) {',
           f'printf("size %zu\\n", sizeof({cname}));']
    src += [f'printf("{f} %zu\\n", offsetof({cname}, {f}));' for f in fields]
    src += ["return 0; }"]
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write("\n".join(src))
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), c, "-o", exe],
                       check=True)
        got = dict(l.split() for l in subprocess.run([exe], capture_output=True, text=True).stdout.splitlines())
    assert int(got["size"]) == ctypes.sizeof(S)
    for f in fields:
        assert int(got[f]) == getattr(S, f).offset, f


def test_header_compiles_as_c_and_cpp():
    with tempfile.TemporaryDirectory() as d:
        for comp, ext in (("gcc", "c"), ("g++", "cpp")):
            p = os.path.join(d, "h." + ext)
            open(p, "w").write("#include \"ra_kv.h\"\nint32_t (*f)(void) = ra_abi_version;\nint main(void){return f == 0;}\n")
            subprocess.run([comp, "-Wall", "-Werror", "-Wno-address", "-c", "-I", os.path.dirname(HEADER), p, "-o",
                            os.path.join(d, "h.o")], check=True)


def test_fused_store_targets_are_writable_fields():
    """The fused store writes the caches and scale planes it is handed, so
    the header declares those fields writable: a caller's mutable pointer goes
    in, and a writable pointer comes back out, with no cast, under -Werror in
    C and C++."""
    code = ('#include "ra_kv.h"\n'
            'int main(void) {\n'
            '  ra_attn_args a = {0};\n'
            '  static unsigned char kc[16], vc[16];\n'
            '  static float ks[16], vs[16];\n'
            '  a.k_cache = kc; a.v_cache = vc; a.k_scales = ks; a.v_scales = vs;\n'
            '  unsigned char* k = (unsigned char*)0; float* s = a.k_scales; void* v = a.v_cache;\n'
            '  k = (unsigned char*)a.k_cache;\n'
            '  return (k != kc) + (s != ks) + (v != vc) + (a.v_scales != vs);\n'
            '}\n')
    with tempfile.TemporaryDirectory() as d:
        for comp, ext in (("gcc", "c"), ("g++", "cpp")):
            p = os.path.join(d, "w." + ext)
            open(p, "w").write(code)
            exe = os.path.join(d, "w_" + ext)
            subprocess.run([comp, "-Wall", "-Werror", "-Wcast-qual", "-I", os.path.dirname(HEADER), p, "-o", exe],
                           check=True)
            assert subprocess.run([exe]).returncode == 0
    text = open(HEADER).read()
    body = text[text.index("typedef struct ra_attn_args"):text.index("} ra_attn_args;")]
    for f in ("k_cache", "v_cache", "k_scales", "v_scales"):
        decl = re.search(rf"^\s*([^;]*)\b{f};", body, re.M).group(1)
        assert "const" not in decl, f"{f} is declared read-only: {decl!r}"
    # the precondition on pages that take new tokens is stated with the fused store
    assert "must be read by no other sequence" in text


FAKE = 0x100000      # 16-byte aligned, never dereferenced by validation


def _good_args(L, **kw):
    a = L.AttnArgs()
    a.struct_size = ctypes.sizeof(L.AttnArgs)
    a.q_dtype = L.RA_F16
    a.q = FAKE
    a.out = FAKE
    a.lse = FAKE
    a.k_cache = FAKE
    a.v_cache = FAKE
    a.kv_dtype = L.RA_KV_FP8_E4M3
    a.k_scale = 0.01
    a.v_scale = 0.01
    a.block_tables = FAKE
    a.block_table_stride = 4
    a.context_lens = FAKE
    a.query_start_loc = FAKE
    a.batch = 2
    a.total_q = 10
    a.num_q_heads = 16
    a.num_kv_heads = 2
    a.head_dim = 128
    a.page_size = 16
    a.num_pages = 100
    a.max_q_len = 5
    a.min_q_len = 5
    a.max_context_len = 64
    a.softmax_scale = 0.088
    a.window_left = -1
    a.num_sinks = 0
    a.num_splits = 1
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def test_noalloc_validation():
    """ra_paged_attn_noalloc: host checks before anything is enqueued.  Partials
    beyond the static scratch (RA_KV_NOALLOC_SCRATCH_BYTES, 32 MiB) are refused
    with RA_ERR_WORKSPACE, also one row past the limit; out must be given; an
    empty batch is a no-op; the ordinary argument checks apply as well."""
    L = _lib()
    lib = L.load_library()
    header = open(HEADER).read()
    assert re.search(r"#define RA_KV_NOALLOC_SCRATCH_BYTES \(32u << 20\)", header)
    limit = 32 << 20
    # 64 slots x total_q x 16 heads x (128 + 1) x 4 bytes: 63 query tokens fit, 64 do not
    assert 64 * 63 * 16 * 129 * 4 <= limit < 64 * 64 * 16 * 129 * 4
    a = _good_args(L, num_splits=64, total_q=64, max_q_len=64, min_q_len=1, batch=1)
    assert lib.ra_paged_attn_noalloc(ctypes.byref(a), None) == 4
    assert b"static scratch" in lib.ra_last_error()
    a = _good_args(L, num_splits=4096, total_q=1000, max_q_len=1000, min_q_len=1, batch=1)
    assert lib.ra_paged_attn_noalloc(ctypes.byref(a), None) == 4
    a = _good_args(L, num_splits=8, out=None)
    assert lib.ra_paged_attn_noalloc(ctypes.byref(a), None) == 1
    assert b"out must be non-NULL" in lib.ra_last_error()
    a = _good_args(L, batch=0, total_q=0, q=None, out=None)
    assert lib.ra_paged_attn_noalloc(ctypes.byref(a), None) == 0
    for kw, status in ((dict(head_dim=96), 2), (dict(k_scale=0.0), 1), (dict(struct_size=8), 1)):
        assert lib.ra_paged_attn_noalloc(ctypes.byref(_good_args(L, **kw)), None) == status, kw


BAD_ATTN = [
    (dict(struct_size=8), 1, "struct_size"),
    (dict(batch=-1), 1, "batch"),
    (dict(q_dtype=3), 2, "q_dtype"),
    (dict(kv_dtype=9), 2, "kv_dtype"),
    (dict(head_dim=96), 2, "head_dim"),
    (dict(page_size=32), 2, "page_size"),
    (dict(num_q_heads=15), 1, "multiple"),
    (dict(num_kv_heads=0), 1, "multiple"),
    (dict(num_pages=0), 1, "num_pages"),
    (dict(block_table_stride=0), 1, "block_table_stride"),
    (dict(max_q_len=0), 1, "max_q_len"),
    (dict(min_q_len=6), 1, "min_q_len"),
    (dict(max_context_len=65), 1, "max_context_len"),
    (dict(softmax_scale=0.0), 1, "softmax_scale"),
    (dict(softmax_scale=float("nan")), 1, "softmax_scale"),
    (dict(k_scale=0.0), 1, "no fallback"),
    (dict(v_scale=float("inf")), 1, "no fallback"),
    (dict(k_scale=-1.0), 1, "no fallback"),
    (dict(kv_dtype=3, v_scale=float("nan")), 1, "INT8"),
    (dict(num_sinks=-1), 1, "num_sinks"),
    (dict(num_splits=-1), 1, "num_splits"),
    (dict(num_splits=5000), 1, "num_splits"),
    (dict(q=0), 1, "non-NULL"),
    (dict(block_tables=0), 1, "non-NULL"),
    (dict(q=FAKE + 8), 3, "aligned"),
    (dict(k_cache=FAKE + 4), 3, "aligned"),
    (dict(out=FAKE + 2), 3, "aligned"),
    (dict(num_splits=4), 4, "partial_out"),
    (dict(num_splits=4, partial_out=FAKE, partial_lse=FAKE, partial_slots=3), 4, "slots"),
    (dict(num_splits=4, partial_out=FAKE + 4, partial_lse=FAKE, partial_slots=4), 3, "partial_out"),
    (dict(out=0, num_splits=1), 4, "out is NULL"),
    # the merge launches one workgroup per query row: total_q * num_q_heads <= 2^31 - 16
    (dict(total_q=(0x7FFFFFF0 // 16) + 1, max_q_len=(0x7FFFFFF0 // 16) + 1), 1, "total_q * num_q_heads"),
]


@pytest.mark.parametrize("kw,status,msg", BAD_ATTN)
def test_attn_validation(kw, status, msg):
    L = _lib()
    lib = L.load_library()
    a = _good_args(L, **kw)
    st = lib.ra_paged_attn(ctypes.byref(a), None)
    assert st == status, (st, lib.ra_last_error())
    assert msg in lib.ra_last_error().decode()


def test_fp16_cache_ignores_scales_and_workspace_query():
    L = _lib()
    a = _good_args(L, kv_dtype=1, k_scale=0.0, v_scale=float("nan"), num_splits=0, max_context_len=64)
    slots, po, pl = L.paged_attn_workspace(a)
    assert slots == 1 and po == 0 and pl == 0
    a = _good_args(L, num_splits=0, max_context_len=64, block_table_stride=1000)
    a.max_context_len = 5000   # > 2048 tokens per matrix-core partition
    slots, po, pl = L.paged_attn_workspace(a)
    assert slots == 3 and po == 3 * 10 * 16 * 128 and pl == 3 * 10 * 16
    a = _good_args(L, num_splits=64, block_table_stride=1000, max_context_len=16000)
    assert L.paged_attn_workspace(a)[0] == 64
    # decode units (g * q_len < 16 rows): 512-token partitions up to 16K tokens,
    # at most 32 up to 64K, 2048-token partitions beyond
    for ctx, slots in [(5000, 10), (16384, 32), (40000, 32), (65536, 32), (100000, 49)]:
        a = _good_args(L, num_splits=0, max_q_len=1, min_q_len=1, block_table_stride=7000, max_context_len=ctx)
        assert L.paged_attn_workspace(a)[0] == slots, ctx
    # long query blocks (16 query heads over 2 KV heads, 48 rows per row group):
    # 2048-token partitions until the row groups alone give 2048 workgroups
    for ctx, ql, qmin, slots in [(32768, 5, 5, 16),        # verify: 1 row group -> 2048-token partitions
                                 (8192, 8192, 8192, 1),    # 2 x 1366 row groups >= 2048: one pass, direct
                                 (8192, 8192, 0, 16),      # min_q_len unknown: a decode sequence may take 16 x 512
                                 (131072, 4896, 4896, 2),  # 2 x 816 row groups: ceil(2048 / 1632) = 2
                                 (131072, 512, 6, 64)]:    # a 6-query block (1 row group) keeps 64 x 2048
        a = _good_args(L, num_splits=0, max_q_len=ql, min_q_len=qmin, total_q=ql, block_table_stride=8192,
                       max_context_len=ctx)
        assert L.paged_attn_workspace(a)[0] == slots, (ctx, ql, qmin)


def test_empty_batch_is_ok_without_pointers():
    L = _lib()
    lib = L.load_library()
    a = _good_args(L, batch=0, total_q=0, q=0, k_cache=0)
    assert lib.ra_paged_attn(ctypes.byref(a), None) == 0


def _store(lib, **kw):
    args = dict(k=FAKE, v=FAKE, src=1, ks=256, vs=256, slots=FAKE, n=4, kc=FAKE, vc=FAKE, kv=2, pages=10,
                hkv=2, d=128, page=16, ksc=0.1, vsc=0.1)
    args.update(kw)
    return lib.ra_kv_store(args["k"], args["v"], args["src"], args["ks"], args["vs"], args["slots"], args["n"],
                           args["kc"], args["vc"], args["kv"], args["pages"], args["hkv"], args["d"], args["page"],
                           args["ksc"], args["vsc"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(n=-1), 1, "num_tokens"),
    (dict(src=3), 2, "src_dtype"),
    (dict(kv=0), 2, "kv_dtype"),
    (dict(d=32), 2, "head_dim"),
    (dict(page=8), 2, "page_size"),
    (dict(hkv=0), 1, "num_kv_heads"),
    (dict(pages=0), 1, "num_pages"),
    (dict(ksc=0.0), 1, "no fallback"),
    (dict(vsc=float("nan")), 1, "no fallback"),
    (dict(ks=100), 1, "strides"),
    (dict(k=0), 1, "non-NULL"),
    (dict(kc=FAKE + 1), 3, "aligned"),
    (dict(ks=260), 3, "multiples of 8"),
    (dict(n=(1 << 30) // 32 + 1), 1, "store in chunks"),
])
def test_store_validation(kw, status, msg):
    L = _lib()
    lib = L.load_library()
    st = _store(lib, **kw)
    assert st == status, (st, lib.ra_last_error())
    assert msg in lib.ra_last_error().decode()


def test_store_zero_tokens_ok_and_fp16_ignores_scale():
    L = _lib()
    lib = L.load_library()
    assert _store(lib, n=0, k=0) == 0
    assert _store(lib, n=0, kv=1, ksc=0.0) == 0


@pytest.mark.parametrize("args,status,msg", [
    ((FAKE, FAKE, 0, 10, 128, FAKE, 1, FAKE), 1, "num_partitions"),
    ((FAKE, FAKE, 5000, 10, 128, FAKE, 1, FAKE), 1, "num_partitions"),
    ((FAKE, FAKE, 2, -1, 128, FAKE, 1, FAKE), 1, "rows"),
    ((FAKE, FAKE, 2, 0x7FFFFFF0 + 1, 128, FAKE, 1, FAKE), 1, "too many rows"),
    ((FAKE, FAKE, 2, 10, 80, FAKE, 1, FAKE), 2, "head_dim"),
    ((FAKE, FAKE, 2, 10, 128, FAKE, 7, FAKE), 2, "out_dtype"),
    ((0, FAKE, 2, 10, 128, FAKE, 1, FAKE), 1, "non-NULL"),
    ((FAKE + 4, FAKE, 2, 10, 128, FAKE, 1, FAKE), 3, "aligned"),
])
def test_merge_validation(args, status, msg):
    L = _lib()
    lib = L.load_library()
    st = lib.ra_lse_merge(*args, None)
    assert st == status and msg in lib.ra_last_error().decode()
    assert lib.ra_lse_merge(FAKE, FAKE, 2, 0, 128, FAKE, 1, None, None) == 0


@pytest.mark.parametrize("args,status,msg", [
    ((FAKE, 2, 2, 0.1, None, FAKE, 16, 4, 1, 128, FAKE), 1, "which"),
    ((FAKE, 0, 5, 0.1, None, FAKE, 16, 4, 1, 128, FAKE), 2, "kv_dtype"),
    ((FAKE, 0, 2, 0.1, None, FAKE, 16, 4, 1, 48, FAKE), 2, "head_dim"),
    ((FAKE, 0, 2, 0.0, None, FAKE, 16, 4, 1, 128, FAKE), 1, "scale"),
    ((FAKE, 0, 2, 0.1, None, FAKE, -1, 4, 1, 128, FAKE), 1, "ctx"),
    ((0, 0, 2, 0.1, None, FAKE, 16, 4, 1, 128, FAKE), 1, "non-NULL"),
    ((FAKE + 2, 0, 2, 0.1, None, FAKE, 16, 4, 1, 128, FAKE), 3, "aligned"),
    ((FAKE, 0, 4, 0.0, None, FAKE, 16, 4, 1, 128, FAKE), 1, "scale plane"),
])
def test_gather_validation(args, status, msg):
    L = _lib()
    lib = L.load_library()
    st = lib.ra_kv_gather_dequant(*args, None)
    assert st == status and msg in lib.ra_last_error().decode()


def _store_tok(lib, **kw):
    args = dict(k=FAKE, v=FAKE, src=1, ks=256, vs=256, slots=FAKE, n=4, kc=FAKE, vc=FAKE, kp=FAKE, vp=FAKE,
                pages=10, hkv=2, d=128, page=16)
    args.update(kw)
    return lib.ra_kv_store_int8_token(args["k"], args["v"], args["src"], args["ks"], args["vs"], args["slots"],
                                      args["n"], args["kc"], args["vc"], args["kp"], args["vp"], args["pages"],
                                      args["hkv"], args["d"], args["page"], None)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(kp=0), 1, "k_scales and v_scales"),
    (dict(vp=0), 1, "k_scales and v_scales"),
    (dict(kp=FAKE + 4), 3, "aligned"),
    (dict(d=96), 2, "head_dim"),
    (dict(n=-2), 1, "num_tokens"),
])
def test_store_int8_token_validation(kw, status, msg):
    L = _lib()
    lib = L.load_library()
    st = _store_tok(lib, **kw)
    assert st == status, (st, lib.ra_last_error())
    assert msg in lib.ra_last_error().decode()
    assert _store_tok(lib, n=0, kp=0) == 0


def test_plain_store_refuses_per_token_format():
    L = _lib()
    lib = L.load_library()
    assert _store(lib, kv=4) == 2
    assert "ra_kv_store_int8_token" in lib.ra_last_error().decode()


def test_attn_int8_token_needs_aligned_planes_and_ignores_layer_scales():
    L = _lib()
    lib = L.load_library()
    a = _good_args(L, kv_dtype=L.RA_KV_INT8_TOKEN, k_scale=0.0, v_scale=float("nan"))
    a.k_scales = None
    a.v_scales = FAKE
    assert lib.ra_paged_attn(ctypes.byref(a), None) == 1
    assert "k_scales and v_scales" in lib.ra_last_error().decode()
    a.k_scales = FAKE + 8
    assert lib.ra_paged_attn(ctypes.byref(a), None) == 3
    # the per-layer scales are not checked for this format: only the planes are
    slots = ctypes.c_int32()
    po = ctypes.c_int64()
    pl = ctypes.c_int64()
    a.k_scales = FAKE
    assert lib.ra_paged_attn_workspace(ctypes.byref(a), ctypes.byref(slots), ctypes.byref(po), ctypes.byref(pl)) == 0


def _rope_args(L, **kw):
    a = L.RopeArgs()
    a.struct_size = ctypes.sizeof(L.RopeArgs)
    a.qkv = FAKE
    a.src_dtype = L.RA_F16
    a.qkv_token_stride = (16 + 4) * 128
    a.num_tokens = 8
    a.positions = FAKE
    a.rope_table = FAKE
    a.max_position = 1024
    a.rotary_dim = 128
    a.q_out = FAKE
    a.q_token_stride = 16 * 128
    a.slot_mapping = FAKE
    a.k_cache = FAKE
    a.v_cache = FAKE
    a.kv_dtype = L.RA_KV_FP8_E4M3
    a.k_scale = 0.01
    a.v_scale = 0.01
    a.num_pages = 10
    a.num_q_heads = 16
    a.num_kv_heads = 2
    a.head_dim = 128
    a.page_size = 16
    for k, v in kw.items():
        setattr(a, k, v)
    return a


BAD_ROPE = [
    (dict(struct_size=8), 1, "struct_size"),
    (dict(num_tokens=-1), 1, "num_tokens"),
    (dict(src_dtype=3), 2, "src_dtype"),
    (dict(kv_dtype=7), 2, "kv_dtype"),
    (dict(head_dim=96), 2, "head_dim"),
    (dict(page_size=8), 2, "page_size"),
    (dict(num_kv_heads=0), 1, "num_kv_heads"),
    (dict(num_pages=0), 1, "num_pages"),
    (dict(rotary_dim=24), 1, "rotary_dim"),
    (dict(rotary_dim=256), 1, "rotary_dim"),
    (dict(max_position=0), 1, "max_position"),
    (dict(k_scale=0.0), 1, "no fallback"),
    (dict(v_scale=float("inf")), 1, "no fallback"),
    (dict(qkv_token_stride=16 * 128), 1, "qkv_token_stride"),
    (dict(q_token_stride=8), 1, "q_token_stride"),
    (dict(num_tokens=1 << 30), 1, "chunks"),
    (dict(positions=None), 1, "non-NULL"),
    (dict(rope_table=None), 1, "non-NULL"),
    (dict(kv_dtype=4), 1, "planes"),
    (dict(q_out=FAKE + 8), 3, "aligned"),
    (dict(qkv_token_stride=(16 + 4) * 128 + 4), 3, "aligned"),
]


@pytest.mark.parametrize("kw,status,msg", BAD_ROPE, ids=[f"{i}-{m}" for i, (_, _, m) in enumerate(BAD_ROPE)])
def test_qkv_rope_validation(kw, status, msg):
    L = _lib()
    lib = L.load_library()
    st = lib.ra_qkv_rope_store(ctypes.byref(_rope_args(L, **kw)), None)
    assert st == status, (st, lib.ra_last_error())
    assert msg in lib.ra_last_error().decode()


def test_qkv_rope_zero_tokens_and_fp16_ignores_scales():
    L = _lib()
    lib = L.load_library()
    assert lib.ra_qkv_rope_store(ctypes.byref(_rope_args(L, num_tokens=0, qkv=None, positions=None)), None) == 0
    a = _rope_args(L, num_tokens=0, kv_dtype=L.RA_KV_F16, k_scale=float("nan"), v_scale=-1.0)
    assert lib.ra_qkv_rope_store(ctypes.byref(a), None) == 0


@pytest.mark.parametrize("max_pos,rot,base,factor,orig", [
    (4096, 128, 10000.0, 1.0, 0),            # plain RoPE
    (4096, 128, 1e6, 2.0, 1024),             # YaRN over a ramp of dims
    (600, 64, 10000.0, 4.0, 256),
    (300, 16, 500.0, 2.0, 100),
])
def test_rope_table_matches_oracle(max_pos, rot, base, factor, orig):
    """The library's host table against the oracle's fp64 table rounded to
    fp32: equal up to one fp32 rounding step (the two round from separately
    computed fp64 values)."""
    import numpy as np
    from oracle import rope as R
    L = _lib()
    got = L.rope_table(max_pos, rot, base, factor, orig, device=None).numpy()
    want = R.rope_table(max_pos, rot, base, factor, original_max=orig or None)
    assert got.shape == want.shape
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got.astype(np.float64) - want) <= ulp + 1e-300)
    assert np.mean(got == want.astype(np.float32)) > 0.999


@pytest.mark.parametrize("rot,head_dim,base,orig,factor", [
    (128, 128, 1e6, 262144, 2.0),     # the pages' deployment: YaRN factor 2 over 262,144 positions
    (128, 128, 1e4, 4096, 2.0),
    (64, 64, 1e4, 2048, 4.0),
    (64, 128, 1e6, 32768, 2.0),       # partial rotary
    (16, 64, 500.0, 100, 2.0),
])
def test_rope_table_matches_the_runtime_yarn_routine(rot, head_dim, base, orig, factor):
    """The library's table pinned to a library routine, independently of the
    oracle: at position 1 each pair's angle is its frequency and its length the
    attention temperature; both must equal what the Hugging Face runtime's YaRN
    function gives for the same config entry, on every dim (ramp ends
    included)."""
    import numpy as np
    transformers = pytest.importorskip("transformers")
    from transformers.modeling_rope_utils import _compute_yarn_parameters
    cfg = transformers.PretrainedConfig()
    cfg.hidden_size, cfg.num_attention_heads, cfg.head_dim = head_dim * 4, 4, head_dim
    cfg.max_position_embeddings = int(orig * factor)
    cfg.rope_parameters = {"rope_type": "yarn", "rope_theta": base, "factor": factor,
                           "original_max_position_embeddings": orig, "partial_rotary_factor": rot / head_dim}
    inv, m = _compute_yarn_parameters(cfg, "cpu")
    inv = inv.double().numpy()
    L = _lib()
    t = L.rope_table(2, rot, base, factor, orig, device=None).numpy().astype(np.float64)
    freq = np.arctan2(t[1, 1], t[1, 0])
    np.testing.assert_allclose(freq, inv, rtol=3e-6, atol=0)
    np.testing.assert_allclose(np.hypot(t[1, 0], t[1, 1]), float(m), rtol=1e-6)
    np.testing.assert_allclose(t[0, 0], float(m), rtol=1e-7)
    assert np.all(t[0, 1] == 0.0)


def test_rope_table_validation():
    L = _lib()
    lib = L.load_library()
    buf = (ctypes.c_float * 64)()
    assert lib.ra_rope_table(buf, 4, 15, 10000.0, 1.0, 0, 32.0, 1.0) == 1
    assert lib.ra_rope_table(buf, 0, 16, 10000.0, 1.0, 0, 32.0, 1.0) == 1
    assert lib.ra_rope_table(buf, 4, 16, 1.0, 1.0, 0, 32.0, 1.0) == 1
    assert lib.ra_rope_table(buf, 4, 16, 10000.0, 2.0, 0, 32.0, 1.0) == 1
    assert lib.ra_rope_table(None, 4, 16, 10000.0, 1.0, 0, 32.0, 1.0) == 1
    assert lib.ra_rope_table(buf, 4, 16, 10000.0, 2.0, 64, 32.0, 1.0) == 0


BAD_FUSED = [
    (dict(max_q_len=7, min_q_len=1), 2, "fused store"),       # 8 * 7 = 56 rows > 48
    (dict(new_v=None), 1, "new_v and new_slots"),
    (dict(new_slots=None), 1, "new_v and new_slots"),
    (dict(new_dtype=3), 2, "new_dtype"),
    (dict(new_k_stride=128), 1, "new_k_stride"),
    (dict(new_v_stride=2 * 128 + 4), 3, "16-byte aligned"),
    (dict(new_k=FAKE + 8), 3, "16-byte aligned"),
]


@pytest.mark.parametrize("kw,status,msg", BAD_FUSED, ids=[f"{i}-{m}" for i, (_, _, m) in enumerate(BAD_FUSED)])
def test_fused_store_validation(kw, status, msg):
    L = _lib()
    lib = L.load_library()
    base = dict(new_k=FAKE, new_v=FAKE, new_dtype=L.RA_F16, new_k_stride=2 * 128, new_v_stride=2 * 128,
                new_slots=FAKE)
    base.update(kw)
    a = _good_args(L, **base)
    st = lib.ra_paged_attn(ctypes.byref(a), None)
    assert st == status, (st, lib.ra_last_error())
    assert msg in lib.ra_last_error().decode()


BAD_ROPE_ATTN = [
    (dict(new_k=None, new_v=None, new_slots=None), 1, "needs the fused store"),
    (dict(positions=None), 1, "needs positions"),
    (dict(rotary_dim=24), 1, "rotary_dim"),
    (dict(rotary_dim=256), 1, "rotary_dim"),
    (dict(rope_max_position=0), 1, "rope_max_position"),
    (dict(rope_table=FAKE + 4), 3, "rope_table must be 16-byte aligned"),
    (dict(q_token_stride=100), 1, "q_token_stride"),
    (dict(q_token_stride=20 * 128 + 4), 3, "q_token_stride"),
]


@pytest.mark.parametrize("kw,status,msg", BAD_ROPE_ATTN, ids=[f"{i}-{m}" for i, (_, _, m) in enumerate(BAD_ROPE_ATTN)])
def test_attention_rope_validation(kw, status, msg):
    L = _lib()
    lib = L.load_library()
    base = dict(new_k=FAKE, new_v=FAKE, new_dtype=L.RA_F16, new_k_stride=20 * 128, new_v_stride=20 * 128,
                new_slots=FAKE, rope_table=FAKE, rope_max_position=4096, rotary_dim=128, positions=FAKE)
    base.update(kw)
    a = _good_args(L, **base)
    st = lib.ra_paged_attn(ctypes.byref(a), None)
    assert st == status, (st, lib.ra_last_error())
    assert msg in lib.ra_last_error().decode()
