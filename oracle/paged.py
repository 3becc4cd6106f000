"""Block-paged KV cache: layout, quantize-on-write and gather, in plain numpy.

Test infrastructure only (see ``oracle/__init__.py``).

Paging follows "SM70 release profile and acceleration status" (KV stored in
fixed-size token pages, 2048 tokens in the release profile, 16 as the
``--block-size 16`` alternative) and "1Cat-vLLM 1.5.0" RELEASE notes, section
"Reliability and correctness fixes" (block tables hold physical page units). The pages
do not fix a byte layout; the library's documented layout is restated here:

* key cache   ``[num_blocks, num_kv_heads, block_size, head_dim]``
  (token-major inside one page of one head),
* value cache ``[num_blocks, num_kv_heads, block_size // T, head_dim, T]``
  with ``T = min(block_size, 64)`` (dimension-major inside each group of T
  consecutive tokens of a page): the value of the token at page offset ``o``,
  dimension ``d`` is ``value_cache[page, h, o // T, d, o % T]``.

Token j of a sequence lives in physical page ``block_table[j // block_size]``
at offset ``j % block_size``. A write goes to ``slot = page * block_size +
offset``; a negative slot means "skip this token".

Cache element formats: ``"f16"`` (numpy float16 values), ``"e4m3"`` and
``"e5m2"`` (uint8 codes, see ``oracle.fp8``).
"""

import numpy as np

from . import fp8

F16 = "f16"
E4M3 = fp8.E4M3
E5M2 = fp8.E5M2


def value_group(block_size):
    """Tokens per dimension-major value group: T = min(block_size, 64)."""
    return min(int(block_size), 64)


def new_caches(num_blocks, num_kv_heads, block_size, head_dim, fmt, fill=0):
    dt = np.float16 if fmt == F16 else np.uint8
    T = value_group(block_size)
    kc = np.full((num_blocks, num_kv_heads, block_size, head_dim), fill, dtype=dt)
    vc = np.full((num_blocks, num_kv_heads, block_size // T, head_dim, T), fill, dtype=dt)
    return kc, vc


def quantize(x, fmt, scale=None):
    """Cache representation of values x: fp16 copy or FP8 codes."""
    if fmt == F16:
        return np.asarray(x).astype(np.float16)
    return fp8.encode(x, fmt, scale)


def write(k, v, slot_mapping, k_cache, v_cache, fmt, k_scale=None, v_scale=None):
    """Quantize-on-write. k, v: [T, Hkv, D]; k_scale, v_scale: [Hkv] float32
    (per KV head) or None. Writes in place, one token at a time."""
    ntok, Hkv, D = k.shape
    bs = k_cache.shape[2]
    T = value_group(bs)
    for t in range(ntok):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        page, off = slot // bs, slot % bs
        for h in range(Hkv):
            ks = None if k_scale is None else k_scale[h]
            vs = None if v_scale is None else v_scale[h]
            k_cache[page, h, off, :] = quantize(k[t, h, :], fmt, ks)
            v_cache[page, h, off // T, :, off % T] = quantize(v[t, h, :], fmt, vs)


def write_tokens(k, v, slot_mapping, k_cache, v_cache, fmt, k_scale=None, v_scale=None,
                 heads=None):
    """``write`` for many tokens at once: the same quantization to the same
    slots, vectorised over the tokens. k, v: [T, H, D]. Without ``heads``,
    H = Hkv and every KV head is written; with ``heads`` (a list of KV head
    indices) k[:, i] and v[:, i] hold head ``heads[i]`` and only those heads
    are written. Slots must be distinct (as for ``write``)."""
    bs = k_cache.shape[2]
    T = value_group(bs)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    keep = slots >= 0
    slots = slots[keep]
    page, off = slots // bs, slots % bs
    heads = list(range(k.shape[1])) if heads is None else [int(h) for h in heads]
    for i, h in enumerate(heads):
        ks = None if k_scale is None else k_scale[h]
        vs = None if v_scale is None else v_scale[h]
        k_cache[page, h, off, :] = quantize(k[keep, i, :], fmt, ks)
        v_cache[page, h, off // T, :, off % T] = quantize(v[keep, i, :], fmt, vs)


def dequant(codes, fmt, scale=None):
    """float64 values of cache elements."""
    if fmt == F16:
        return np.asarray(codes, dtype=np.float16).astype(np.float64)
    return fp8.dequant(codes, fmt, scale)


def gather(k_cache, v_cache, block_table, ctx, g, fmt, k_scale=None, v_scale=None):
    """Dequantized K and V ([ctx, D] float64 each) of KV head g for one
    sequence. Only the first ceil(ctx / block_size) block-table entries are
    read, so padding entries are never dereferenced."""
    bs = k_cache.shape[2]
    D = k_cache.shape[3]
    T = value_group(bs)
    if ctx == 0:
        return np.zeros((0, D)), np.zeros((0, D))
    j = np.arange(ctx)
    used = -(-ctx // bs)
    pages = np.asarray(block_table[:used], dtype=np.int64)[j // bs]
    off = j % bs
    k_raw = k_cache[pages, g, off, :]              # [ctx, D]
    v_raw = v_cache[pages, g, off // T, :, off % T]  # [ctx, D]
    ks = None if k_scale is None else k_scale[g]
    vs = None if v_scale is None else v_scale[g]
    return dequant(k_raw, fmt, ks), dequant(v_raw, fmt, vs)
