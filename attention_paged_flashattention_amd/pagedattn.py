"""Python binding of libpagedattn.so (ctypes; argument marshalling only).

The functions carry the names of the C ABI in include/pagedattn.h and take
torch tensors for device memory; every step of the computation runs in the HIP
kernels of the library. Importing this module fails loudly when the library
has not been built -- there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpagedattn.so")

# pa_status
PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_HIP = 0, 1, 2, 3
# pa_dtype
PA_F16, PA_BF16, PA_F32, PA_FP8_E4M3, PA_FP8_E5M2 = 0, 1, 2, 3, 4
# pa_op
PA_OP_WRITE, PA_OP_PREFILL, PA_OP_DECODE, PA_OP_VERIFY, PA_OP_WINDOW = 0, 1, 2, 3, 4

CACHE_DTYPES = {"f16": PA_F16, "e4m3": PA_FP8_E4M3, "e5m2": PA_FP8_E5M2}
TORCH_DTYPES = {torch.float16: PA_F16, torch.bfloat16: PA_BF16, torch.float32: PA_F32}

EXPORTS = ["kv_cache_write_fp8", "attn_prefill_paged", "attn_decode_paged",
           "attn_verify_paged", "attn_verify_paged_noalloc", "attn_decode_append_paged",
           "attn_window_paged",
           "pa_window_workspace_bytes",
           "pa_decode_partitions", "pa_workspace_bytes",
           "pa_supports", "pa_last_error", "pa_version", "pa_validate_tables",
           "pa_profile_next_call"]


class PagedAttnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"[status {status}] {message}")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python -m attention_paged_flashattention_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_lib.kv_cache_write_fp8.argtypes = [_vp, _vp, _i32, _vp, _i64, _vp, _vp, _i32, _i64, _i32, _i32,
                                    _i32, _vp, _vp, _vp]
_lib.attn_prefill_paged.argtypes = [_vp, _i32, _vp, _i32, _i32, _i64, _vp, _vp, _i32, _i32, _i64,
                                    _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _f32, _vp,
                                    _i32, _vp]
_DECODE_TAIL = [_vp, _vp, _i32, _i32, _i64, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _vp, _vp,
                _f32, _i32, _vp, _sz, _vp, _i32, _vp]
_lib.attn_decode_paged.argtypes = [_vp, _i32, _i32] + _DECODE_TAIL
_lib.attn_verify_paged.argtypes = [_vp, _i32, _i32, _i32] + _DECODE_TAIL
_lib.attn_window_paged.argtypes = [_vp, _i32, _i32, _i32, _i32] + _DECODE_TAIL
# the same tail without (workspace, workspace_bytes)
_lib.attn_verify_paged_noalloc.argtypes = [_vp, _i32, _i32, _i32] + _DECODE_TAIL[:16] + \
    _DECODE_TAIL[18:]
_lib.attn_decode_append_paged.argtypes = [_vp, _i32, _i32, _i32, _vp, _vp] + _DECODE_TAIL
_lib.pa_window_workspace_bytes.argtypes = [_i32] * 8
_lib.pa_window_workspace_bytes.restype = _sz
_lib.pa_decode_partitions.argtypes = [_i32] * 6
_lib.pa_decode_partitions.restype = _i32
_lib.pa_workspace_bytes.argtypes = [_i32] * 8
_lib.pa_workspace_bytes.restype = _sz
_lib.pa_supports.argtypes = [_i32] * 8
_lib.pa_supports.restype = _i32
_lib.pa_last_error.restype = ctypes.c_char_p
_lib.pa_version.restype = ctypes.c_char_p
_lib.pa_validate_tables.argtypes = [_vp, _i32, _i32, _vp, _i32, _i32, _i64, _vp, _vp]
_lib.pa_profile_next_call.argtypes = [_vp, _vp]
_lib.pa_profile_next_call.restype = None
for _name in ("kv_cache_write_fp8", "attn_prefill_paged", "attn_decode_paged",
              "attn_verify_paged", "attn_verify_paged_noalloc", "attn_decode_append_paged",
              "attn_window_paged",
              "pa_validate_tables"):
    getattr(_lib, _name).restype = _i32


def lib():
    """The raw ctypes library (for callers that pass pointers themselves)."""
    return _lib


def pa_last_error():
    return _lib.pa_last_error().decode()


def pa_version():
    return _lib.pa_version().decode()


def _check(status):
    if status != PA_OK:
        raise PagedAttnError(status, pa_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _cache_dtype(cache_dtype):
    return CACHE_DTYPES[cache_dtype] if isinstance(cache_dtype, str) else int(cache_dtype)


def _need(t, name, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


class Bound:
    """An ABI call whose arguments were marshalled once; calling it issues the
    call again with the same pointers and sizes (the tensors must stay alive)."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = tuple(t(a) if not isinstance(a, (ctypes.c_void_p, type(None))) else a
                           for t, a in zip(fn.argtypes, args))
        self._keep = keep

    def __call__(self):
        _check(self._fn(*self._args))


def _write_args(key, value, slot_mapping, key_cache, value_cache, cache_dtype, k_scale, v_scale,
                stream):
    _need(key, "key", (torch.float16, torch.bfloat16), 3)
    _need(value, "value", key.dtype, 3)
    _need(slot_mapping, "slot_mapping", torch.int64, 1)
    _need(key_cache, "key_cache", ndim=4)
    _need(value_cache, "value_cache", ndim=5)
    nb, hkv, bs, d = key_cache.shape
    return [_ptr(key), _ptr(value), TORCH_DTYPES[key.dtype], _ptr(slot_mapping), key.shape[0],
            _ptr(key_cache), _ptr(value_cache), _cache_dtype(cache_dtype), nb, bs, hkv, d,
            _ptr(k_scale), _ptr(v_scale), _stream(key.device, stream)]


def kv_cache_write_fp8(key, value, slot_mapping, key_cache, value_cache, cache_dtype,
                       k_scale=None, v_scale=None, stream=None):
    """key/value [T, Hkv, D] fp16|bf16; slot_mapping [T] int64; caches
    [NB, Hkv, bs, D] / [NB, Hkv, bs/G, D, G] (G = min(bs, 64)), uint8 (FP8) or
    fp16."""
    _check(_lib.kv_cache_write_fp8(*_write_args(key, value, slot_mapping, key_cache, value_cache,
                                                cache_dtype, k_scale, v_scale, stream)))


def bind_kv_cache_write_fp8(key, value, slot_mapping, key_cache, value_cache, cache_dtype,
                            k_scale=None, v_scale=None, stream=None):
    args = _write_args(key, value, slot_mapping, key_cache, value_cache, cache_dtype, k_scale,
                       v_scale, stream)
    return Bound(_lib.kv_cache_write_fp8, args,
                 (key, value, slot_mapping, key_cache, value_cache, k_scale, v_scale))


def _out(q, out, out_dtype, shape):
    if out is None:
        out = torch.empty(shape, dtype=out_dtype or q.dtype, device=q.device)
    _need(out, "out", (torch.float32, torch.float16, torch.bfloat16))
    return out


def _prefill_args(q, cu_seqlens_q, max_q_len, key_cache, value_cache, cache_dtype, block_tables,
                  context_lens, max_context_len, softmax_scale, k_scale, v_scale, out, out_dtype,
                  stream):
    _need(q, "q", (torch.float16, torch.bfloat16), 3)
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    total_q, hq, d = q.shape
    nb, hkv, bs, _ = key_cache.shape
    out = _out(q, out, out_dtype, (total_q, hq, d))
    args = [_ptr(q), TORCH_DTYPES[q.dtype], _ptr(cu_seqlens_q), block_tables.shape[0],
            int(max_q_len), total_q, _ptr(key_cache), _ptr(value_cache), _cache_dtype(cache_dtype),
            bs, nb, _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
            int(max_context_len), hq, hkv, d, _ptr(k_scale), _ptr(v_scale), float(softmax_scale),
            _ptr(out), TORCH_DTYPES[out.dtype], _stream(q.device, stream)]
    return args, out


def attn_prefill_paged(q, cu_seqlens_q, max_q_len, key_cache, value_cache, cache_dtype,
                       block_tables, context_lens, max_context_len, softmax_scale,
                       k_scale=None, v_scale=None, out=None, out_dtype=None, stream=None):
    """q [total_q, Hq, D]; cu_seqlens_q [B+1] int32; block_tables [B, M] int32;
    context_lens [B] int32."""
    args, out = _prefill_args(q, cu_seqlens_q, max_q_len, key_cache, value_cache, cache_dtype,
                              block_tables, context_lens, max_context_len, softmax_scale,
                              k_scale, v_scale, out, out_dtype, stream)
    _check(_lib.attn_prefill_paged(*args))
    return out


def bind_attn_prefill_paged(q, cu_seqlens_q, max_q_len, key_cache, value_cache, cache_dtype,
                            block_tables, context_lens, max_context_len, softmax_scale,
                            k_scale=None, v_scale=None, out=None, out_dtype=None, stream=None):
    args, out = _prefill_args(q, cu_seqlens_q, max_q_len, key_cache, value_cache, cache_dtype,
                              block_tables, context_lens, max_context_len, softmax_scale,
                              k_scale, v_scale, out, out_dtype, stream)
    return Bound(_lib.attn_prefill_paged, args,
                 (q, cu_seqlens_q, key_cache, value_cache, block_tables, context_lens, k_scale,
                  v_scale, out)), out


def pa_workspace_bytes(op, batch, q_len, num_q_heads, num_kv_heads, head_dim, num_partitions,
                       max_context_len):
    return int(_lib.pa_workspace_bytes(op, batch, q_len, num_q_heads, num_kv_heads, head_dim,
                                       num_partitions, max_context_len))


def pa_window_workspace_bytes(batch, q_len, num_q_heads, num_kv_heads, head_dim, num_partitions,
                              max_context_len, window_left):
    return int(_lib.pa_window_workspace_bytes(batch, q_len, num_q_heads, num_kv_heads, head_dim,
                                              num_partitions, max_context_len, window_left))


def pa_decode_partitions(batch, q_len, num_q_heads, num_kv_heads, head_dim, max_context_len):
    return int(_lib.pa_decode_partitions(batch, q_len, num_q_heads, num_kv_heads, head_dim,
                                         max_context_len))


def pa_supports(op, q_dtype, cache_dtype, head_dim, num_q_heads, num_kv_heads, block_size, q_len):
    return bool(_lib.pa_supports(op, q_dtype, cache_dtype, head_dim, num_q_heads, num_kv_heads,
                                 block_size, q_len))


def _decode_like(fn, op, q, q_len, key_cache, value_cache, cache_dtype, block_tables, context_lens,
                 max_context_len, softmax_scale, k_scale, v_scale, num_partitions, workspace, out,
                 out_dtype, stream, bind=False, window=None, new_kv=None):
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    batch = q.shape[0]
    hq, d = q.shape[-2], q.shape[-1]
    nb, hkv, bs, _ = key_cache.shape
    if op == PA_OP_WINDOW:
        need = pa_window_workspace_bytes(batch, q_len, hq, hkv, d, num_partitions,
                                         max_context_len, window)
    else:
        need = pa_workspace_bytes(op, batch, q_len, hq, hkv, d, num_partitions, max_context_len)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    out = _out(q, out, out_dtype, tuple(q.shape))
    args = [_ptr(key_cache), _ptr(value_cache), _cache_dtype(cache_dtype), bs, nb, _ptr(block_tables),
            block_tables.shape[1], _ptr(context_lens), int(max_context_len), hq, hkv, d,
            _ptr(k_scale), _ptr(v_scale), float(softmax_scale), int(num_partitions),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out),
            TORCH_DTYPES[out.dtype], _stream(q.device, stream)]
    keep = ()
    if new_kv is not None:
        k_new, v_new = new_kv
        shape = (batch, q_len, hkv, d)
        for t, name in ((k_new, "key_new"), (v_new, "value_new")):
            _need(t, name, q.dtype)
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
        args = [_ptr(q), TORCH_DTYPES[q.dtype], batch, q_len, _ptr(k_new), _ptr(v_new)] + args
        keep = (k_new, v_new)
    elif op == PA_OP_DECODE:
        args = [_ptr(q), TORCH_DTYPES[q.dtype], batch] + args
    elif op == PA_OP_WINDOW:
        args = [_ptr(q), TORCH_DTYPES[q.dtype], batch, q_len, int(window)] + args
    else:
        args = [_ptr(q), TORCH_DTYPES[q.dtype], batch, q_len] + args
    if bind:
        return Bound(fn, args, (q, key_cache, value_cache, block_tables, context_lens, k_scale,
                                v_scale, workspace, out) + keep), out
    _check(fn(*args))
    return out


def attn_decode_paged(q, key_cache, value_cache, cache_dtype, block_tables, context_lens,
                      max_context_len, softmax_scale, k_scale=None, v_scale=None,
                      num_partitions=0, workspace=None, out=None, out_dtype=None, stream=None):
    """q [B, Hq, D] -> out [B, Hq, D]."""
    _need(q, "q", (torch.float16, torch.bfloat16), 3)
    return _decode_like(_lib.attn_decode_paged, PA_OP_DECODE, q, 1, key_cache, value_cache,
                        cache_dtype, block_tables, context_lens, max_context_len, softmax_scale,
                        k_scale, v_scale, num_partitions, workspace, out, out_dtype, stream)


def bind_attn_decode_paged(q, key_cache, value_cache, cache_dtype, block_tables, context_lens,
                           max_context_len, softmax_scale, k_scale=None, v_scale=None,
                           num_partitions=0, workspace=None, out=None, out_dtype=None,
                           stream=None):
    _need(q, "q", (torch.float16, torch.bfloat16), 3)
    return _decode_like(_lib.attn_decode_paged, PA_OP_DECODE, q, 1, key_cache, value_cache,
                        cache_dtype, block_tables, context_lens, max_context_len, softmax_scale,
                        k_scale, v_scale, num_partitions, workspace, out, out_dtype, stream,
                        bind=True)


def bind_attn_verify_paged(q, key_cache, value_cache, cache_dtype, block_tables, context_lens,
                           max_context_len, softmax_scale, k_scale=None, v_scale=None,
                           num_partitions=0, workspace=None, out=None, out_dtype=None,
                           stream=None):
    _need(q, "q", (torch.float16, torch.bfloat16), 4)
    return _decode_like(_lib.attn_verify_paged, PA_OP_VERIFY, q, q.shape[1], key_cache,
                        value_cache, cache_dtype, block_tables, context_lens, max_context_len,
                        softmax_scale, k_scale, v_scale, num_partitions, workspace, out,
                        out_dtype, stream, bind=True)


def attn_verify_paged(q, key_cache, value_cache, cache_dtype, block_tables, context_lens,
                      max_context_len, softmax_scale, k_scale=None, v_scale=None,
                      num_partitions=0, workspace=None, out=None, out_dtype=None, stream=None):
    """q [B, q_len, Hq, D] -> out [B, q_len, Hq, D]."""
    _need(q, "q", (torch.float16, torch.bfloat16), 4)
    return _decode_like(_lib.attn_verify_paged, PA_OP_VERIFY, q, q.shape[1], key_cache,
                        value_cache, cache_dtype, block_tables, context_lens, max_context_len,
                        softmax_scale, k_scale, v_scale, num_partitions, workspace, out,
                        out_dtype, stream)


NOALLOC_SCRATCH_BYTES = 16 << 20   # the static scratch of attn_verify_paged_noalloc


def attn_verify_paged_noalloc(q, key_cache, value_cache, cache_dtype, block_tables,
                              context_lens, max_context_len, softmax_scale, out, k_scale=None,
                              v_scale=None, num_partitions=0, stream=None):
    """attn_verify_paged with the partials in the library's static device
    scratch: q [B, q_len, Hq, D]; out [B, q_len, Hq, D] is caller-allocated
    (F32, F16 or BF16). No device memory is allocated by this call."""
    _need(q, "q", (torch.float16, torch.bfloat16), 4)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    _need(out, "out", (torch.float32, torch.float16, torch.bfloat16))
    batch, q_len, hq, d = q.shape
    nb, hkv, bs, _ = key_cache.shape
    _check(_lib.attn_verify_paged_noalloc(
        _ptr(q), TORCH_DTYPES[q.dtype], batch, q_len, _ptr(key_cache), _ptr(value_cache),
        _cache_dtype(cache_dtype), bs, nb, _ptr(block_tables), block_tables.shape[1],
        _ptr(context_lens), int(max_context_len), hq, hkv, d, _ptr(k_scale), _ptr(v_scale),
        float(softmax_scale), int(num_partitions), _ptr(out), TORCH_DTYPES[out.dtype],
        _stream(q.device, stream)))
    return out


def attn_decode_append_paged(q, key_new, value_new, key_cache, value_cache, cache_dtype,
                             block_tables, context_lens, max_context_len, softmax_scale,
                             k_scale=None, v_scale=None, num_partitions=0, workspace=None,
                             out=None, out_dtype=None, stream=None):
    """q [B, q_len, Hq, D]; key_new, value_new [B, q_len, Hkv, D] (q's dtype)
    -> out [B, q_len, Hq, D]. Writes the new tokens at positions
    ctx_b - q_len .. ctx_b - 1 of each sequence's pages, then attends (one
    kernel for both)."""
    _need(q, "q", (torch.float16, torch.bfloat16), 4)
    return _decode_like(_lib.attn_decode_append_paged, PA_OP_VERIFY, q, q.shape[1], key_cache,
                        value_cache, cache_dtype, block_tables, context_lens, max_context_len,
                        softmax_scale, k_scale, v_scale, num_partitions, workspace, out,
                        out_dtype, stream, new_kv=(key_new, value_new))


def bind_attn_decode_append_paged(q, key_new, value_new, key_cache, value_cache, cache_dtype,
                                  block_tables, context_lens, max_context_len, softmax_scale,
                                  k_scale=None, v_scale=None, num_partitions=0, workspace=None,
                                  out=None, out_dtype=None, stream=None):
    _need(q, "q", (torch.float16, torch.bfloat16), 4)
    return _decode_like(_lib.attn_decode_append_paged, PA_OP_VERIFY, q, q.shape[1], key_cache,
                        value_cache, cache_dtype, block_tables, context_lens, max_context_len,
                        softmax_scale, k_scale, v_scale, num_partitions, workspace, out,
                        out_dtype, stream, bind=True, new_kv=(key_new, value_new))


def attn_window_paged(q, window_left, key_cache, value_cache, cache_dtype, block_tables,
                      context_lens, max_context_len, softmax_scale, k_scale=None, v_scale=None,
                      num_partitions=0, workspace=None, out=None, out_dtype=None, stream=None):
    """q [B, q_len, Hq, D] -> out [B, q_len, Hq, D]; row i of sequence b sees
    keys pos - window_left .. ctx_b - 1 (pos = ctx_b - q_len + i)."""
    _need(q, "q", (torch.float16, torch.bfloat16), 4)
    return _decode_like(_lib.attn_window_paged, PA_OP_WINDOW, q, q.shape[1], key_cache,
                        value_cache, cache_dtype, block_tables, context_lens, max_context_len,
                        softmax_scale, k_scale, v_scale, num_partitions, workspace, out,
                        out_dtype, stream, window=window_left)


def bind_attn_window_paged(q, window_left, key_cache, value_cache, cache_dtype, block_tables,
                           context_lens, max_context_len, softmax_scale, k_scale=None,
                           v_scale=None, num_partitions=0, workspace=None, out=None,
                           out_dtype=None, stream=None):
    _need(q, "q", (torch.float16, torch.bfloat16), 4)
    return _decode_like(_lib.attn_window_paged, PA_OP_WINDOW, q, q.shape[1], key_cache,
                        value_cache, cache_dtype, block_tables, context_lens, max_context_len,
                        softmax_scale, k_scale, v_scale, num_partitions, workspace, out,
                        out_dtype, stream, bind=True, window=window_left)


def pa_profile_next_call(start_event, stop_event):
    """Attach the two hipEvent_t handles (ints) to the main kernel of the next
    call on this thread (they record its start and end); None clears."""
    _lib.pa_profile_next_call(ctypes.c_void_p(start_event), ctypes.c_void_p(stop_event))


def pa_validate_tables(block_tables, context_lens, max_context_len, block_size, num_blocks,
                       cu_seqlens_q=None, stream=None):
    cu = None if cu_seqlens_q is None else _ptr(cu_seqlens_q)
    st = _lib.pa_validate_tables(_ptr(block_tables), block_tables.shape[0], block_tables.shape[1],
                                 _ptr(context_lens), int(max_context_len), int(block_size),
                                 int(num_blocks), cu, _stream(block_tables.device, stream))
    _check(st)
