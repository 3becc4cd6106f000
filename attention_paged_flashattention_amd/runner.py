"""Drive a synthetic workload through the library on one GPU.

Uploads a ``synth.Case`` (queries, new K/V tokens, slots, block tables, context
lengths, scales), allocates its paged caches poisoned with NaN patterns, and
issues the ABI calls of each workload step. Holds no attention or FP8
arithmetic: every computation is a call into libpagedattn.so.
"""

import numpy as np
import torch

from . import pagedattn as pa
from . import synth


def upload16(arr, dtype, device):
    """16-bit host storage (np.float16 or bf16 bits) -> torch tensor."""
    if dtype == "f16":
        return torch.from_numpy(np.ascontiguousarray(arr)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(device)
    return t.view(torch.bfloat16)


def poison_cache(t, fmt):
    if fmt == "f16":
        t.view(torch.int16).fill_(synth.POISON["f16"])
    else:
        t.fill_(synth.POISON[fmt])


class DeviceCase:
    """A workload resident in HBM."""

    def __init__(self, case, device="cuda:0", upload_kv=True):
        self.case = case
        self.device = device
        c = case
        self.q = upload16(c.q, c.q_dtype, device)                       # [total_q, Hq, D]
        self.k = upload16(c.k, c.kv_dtype, device) if upload_kv else None
        self.v = upload16(c.v, c.kv_dtype, device) if upload_kv else None
        self.slots = torch.from_numpy(c.slot_mapping).to(device)
        self.block_tables = torch.from_numpy(c.block_tables).to(device)
        self.ctx_lens = torch.from_numpy(c.ctx_lens).to(device)
        self.k_scale = None if c.k_scale is None else torch.from_numpy(c.k_scale).to(device)
        self.v_scale = None if c.v_scale is None else torch.from_numpy(c.v_scale).to(device)
        cdt = torch.float16 if c.cache_fmt == "f16" else torch.uint8
        nb, hkv, bs, d = c.num_blocks, c.num_kv_heads, c.block_size, c.head_dim
        self.key_cache = torch.empty((nb, hkv, bs, d), dtype=cdt, device=device)
        vg = min(bs, 64)   # value groups: dimension-major inside 64-token groups
        self.value_cache = torch.empty((nb, hkv, bs // vg, d, vg), dtype=cdt, device=device)
        poison_cache(self.key_cache, c.cache_fmt)
        poison_cache(self.value_cache, c.cache_fmt)
        self.max_ctx = int(c.ctx_lens.max()) if len(c.ctx_lens) else 0

    # ---- quantize-on-write ----
    def write_tokens(self, start, stop, stream=None):
        """Write tokens [start, stop) of the concatenated K/V through their slots."""
        pa.kv_cache_write_fp8(self.k[start:stop], self.v[start:stop], self.slots[start:stop],
                              self.key_cache, self.value_cache, self.case.cache_fmt,
                              self.k_scale, self.v_scale, stream=stream)

    def write_all(self):
        self.write_tokens(0, self.k.shape[0])

    def last_token_rows(self, n):
        """Indices of the last n tokens of every sequence (the newest writes)."""
        c = self.case
        idx = []
        for b in range(c.batch):
            e = int(c.tok_start[b]) + int(c.ctx_lens[b])
            idx.extend(range(max(int(c.tok_start[b]), e - n), e))
        return torch.tensor(idx, dtype=torch.int64, device=self.device)

    # ---- attention ----
    def decode(self, q=None, ctx_lens=None, max_ctx=None, num_partitions=0, workspace=None,
               out=None, out_dtype=None, stream=None):
        c = self.case
        q = self.q if q is None else q
        return pa.attn_decode_paged(q, self.key_cache, self.value_cache, c.cache_fmt,
                                    self.block_tables, self.ctx_lens if ctx_lens is None else ctx_lens,
                                    self.max_ctx if max_ctx is None else max_ctx, c.softmax_scale,
                                    self.k_scale, self.v_scale, num_partitions=num_partitions,
                                    workspace=workspace, out=out, out_dtype=out_dtype, stream=stream)

    def verify(self, q_len, num_partitions=0, workspace=None, out=None, out_dtype=None,
               stream=None):
        c = self.case
        q = self.q.view(c.batch, q_len, c.num_q_heads, c.head_dim)
        return pa.attn_verify_paged(q, self.key_cache, self.value_cache, c.cache_fmt,
                                    self.block_tables, self.ctx_lens, self.max_ctx,
                                    c.softmax_scale, self.k_scale, self.v_scale,
                                    num_partitions=num_partitions, workspace=workspace, out=out,
                                    out_dtype=out_dtype, stream=stream)

    def window(self, q_len, window_left, num_partitions=0, workspace=None, out=None,
               out_dtype=None, stream=None):
        c = self.case
        q = self.q.view(c.batch, q_len, c.num_q_heads, c.head_dim)
        return pa.attn_window_paged(q, window_left, self.key_cache, self.value_cache, c.cache_fmt,
                                    self.block_tables, self.ctx_lens, self.max_ctx,
                                    c.softmax_scale, self.k_scale, self.v_scale,
                                    num_partitions=num_partitions, workspace=workspace, out=out,
                                    out_dtype=out_dtype, stream=stream)

    def prefill(self, q_rows, cu_seqlens, max_q_len, ctx_lens, max_ctx, out=None, out_dtype=None,
                stream=None):
        c = self.case
        return pa.attn_prefill_paged(q_rows, cu_seqlens, max_q_len, self.key_cache,
                                     self.value_cache, c.cache_fmt, self.block_tables, ctx_lens,
                                     max_ctx, c.softmax_scale, self.k_scale, self.v_scale, out=out,
                                     out_dtype=out_dtype, stream=stream)

    def prefill_chunk(self, start, stop, out=None, out_dtype=None, stream=None, write=True):
        """Single-sequence chunked prefill: write tokens [start, stop), then the
        queries of those positions attend to keys 0..pos (ctx = stop)."""
        assert self.case.batch == 1
        if write:
            self.write_tokens(start, stop, stream=stream)
        n = stop - start
        cu = torch.tensor([0, n], dtype=torch.int32, device=self.device)
        ctx = torch.tensor([stop], dtype=torch.int32, device=self.device)
        return self.prefill(self.q[start:stop], cu, n, ctx, stop, out=out, out_dtype=out_dtype,
                            stream=stream)
