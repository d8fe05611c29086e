"""Oracle: the paged KV cache layout, scatter of new tokens and gather back.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Passages followed
-----------------
* "ReVolta 0.1.3" release notes, "Known issues": the INT8 path uses
  16-token kernel pages (so a page holds 16 token positions).
* ReVolta README, "Quick start" (prefix caching enabled) and intro list
  (a GPU KV pool shared by several long contexts): sequences address
  physical pages through a per-sequence block table, and several block
  tables may name the same physical page.

The pages never give a byte layout.  The layout below is the one the
library's C ABI declares (``include/ra_kv.h``), written out here from that
definition, element by element:

K and V are separate caches, each ``num_pages * Hkv`` blocks of
``16 * D * e`` bytes (e = 2 for FP16, 1 for E4M3 / INT8); block
``(page, head)`` starts at byte ``(page * Hkv + head) * 16 * D * e``.
Inside a block, with ``b`` the byte position computed below,
``offset = (b // 16) * 1024 + lane * 16 + b % 16``:

* K element (t, d):  lane = 16 * (d // (D/4)) + t,  b = (d % (D/4)) * e
* V element (t, d):  lane = 16 * (t // 4) + d // (D/16),
                     b = ((d % (D/16)) * 4 + t % 4) * e

INT8 with per-token scales ('int8_tok') stores its codes exactly like INT8
and, beside each cache, a plane of fp32 scales ``[num_pages][Hkv][16]``:
the scale of (slot, head) is float number ``(page * Hkv + head) * 16 + t``.

Scatter (the method's store step): for new token n with slot >= 0,
``cache[slot // 16][h][slot % 16][:] = code(n, h, :)``; bytes of tokens not
stored keep their previous content; slot < 0 means "skip".

Pins (tests/test_oracle_layout.py): offsets form a bijection onto each
block for every (D, e); hand-derived offsets of chosen elements; a scatter
of a full random permutation followed by a gather returns the input
bit for bit; bytes not addressed are untouched.
"""
import numpy as np

PAGE = 16


def k_offset(t, d, D, e):
    """Byte offset of K element (token-in-page t, dim d) inside its block."""
    q = D // 4
    lane = 16 * (d // q) + t
    b = (d % q) * e
    return (b // 16) * 1024 + lane * 16 + b % 16


def v_offset(t, d, D, e):
    """Byte offset of V element (token-in-page t, dim d) inside its block."""
    w = D // 16
    lane = 16 * (t // 4) + d // w
    b = ((d % w) * 4 + t % 4) * e
    return (b // 16) * 1024 + lane * 16 + b % 16


def block_bytes(D, e):
    return PAGE * D * e


def offset_table(which, D, e):
    """int64[16, D]: byte offset of every element of one block."""
    f = k_offset if which == "k" else v_offset
    out = np.empty((PAGE, D), dtype=np.int64)
    for t in range(PAGE):
        for d in range(D):
            out[t, d] = f(t, d, D, e)
    return out


def _element_byte_index(which, num_kv_heads, D, e, slots):
    """int64[n, Hkv, D]: absolute byte offset of the first byte of each element."""
    table = offset_table(which, D, e)                          # [16, D]
    slots = np.asarray(slots, dtype=np.int64)
    page = slots // PAGE
    t = slots % PAGE
    heads = np.arange(num_kv_heads, dtype=np.int64)
    base = (page[:, None] * num_kv_heads + heads[None, :]) * block_bytes(D, e)
    return base[:, :, None] + table[t][:, None, :]


def scatter(cache_bytes, codes, slots, which, num_kv_heads, D, kv_dtype):
    """Write codes [n][Hkv][D] into a cache given as a flat uint8 array.

    Returns a new array; ``slots`` int64[n], negative entries skipped.
    """
    e = 2 if kv_dtype == "f16" else 1
    cache = np.array(cache_bytes, dtype=np.uint8, copy=True).reshape(-1)
    codes = np.ascontiguousarray(codes)
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    raw = codes.view(np.uint8).reshape(codes.shape[0], num_kv_heads, D, e)
    idx = _element_byte_index(which, num_kv_heads, D, e, slots[keep])
    for j in range(e):
        cache[idx + j] = raw[keep][..., j]
    return cache


def gather(cache_bytes, slots, which, num_kv_heads, D, kv_dtype):
    """Read codes [n][Hkv][D] for the given slots back from a flat cache."""
    e = 2 if kv_dtype == "f16" else 1
    cache = np.asarray(cache_bytes, dtype=np.uint8).reshape(-1)
    idx = _element_byte_index(which, num_kv_heads, D, e, slots)
    raw = np.stack([cache[idx + j] for j in range(e)], axis=-1)
    raw = np.ascontiguousarray(raw)
    if kv_dtype == "f16":
        return raw.view(np.float16).reshape(raw.shape[:-1])
    if kv_dtype in ("int8", "int8_tok"):
        return raw.view(np.int8).reshape(raw.shape[:-1])
    return raw.reshape(raw.shape[:-1])


def scale_index(slots, num_kv_heads):
    """int64[n, Hkv]: float index of each (slot, head) scale in a scale plane."""
    slots = np.asarray(slots, dtype=np.int64)
    heads = np.arange(num_kv_heads, dtype=np.int64)
    return ((slots // PAGE)[:, None] * num_kv_heads + heads[None, :]) * PAGE + (slots % PAGE)[:, None]


def scatter_scales(plane, scales, slots, num_kv_heads):
    """Write scales [n][Hkv] into a flat fp32 scale plane; slot < 0 skipped."""
    out = np.array(plane, dtype=np.float32, copy=True).reshape(-1)
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    out[scale_index(slots[keep], num_kv_heads)] = np.asarray(scales, dtype=np.float32)[keep]
    return out


def gather_scales(plane, slots, num_kv_heads):
    """Read scales [n][Hkv] for the given slots back from a flat scale plane."""
    return np.asarray(plane, dtype=np.float32).reshape(-1)[scale_index(slots, num_kv_heads)]


def slots_for_sequence(block_table_row, ctx):
    """Slot of every logical position 0..ctx-1 of one sequence."""
    j = np.arange(ctx, dtype=np.int64)
    row = np.asarray(block_table_row, dtype=np.int64)
    return row[j // PAGE] * PAGE + j % PAGE
