"""Python binding of libmla_paged.so: paged MLA decode on MI355X (gfx950).

Argument marshalling only.  Every step of the decode (split-KV schedule,
attention, combine) runs in the HIP kernels behind the C ABI declared in
``include/mla_paged.h``; torch only provides device memory and the stream.
If the shared library has not been built, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "MlaError",
    "HEAD_DIM",
    "V_DIM",
    "PAGE_SIZE",
    "META_INTS",
    "library_path",
    "load_library",
    "num_partitions",
    "metadata_ints",
    "workspace_bytes",
    "get_metadata",
    "decode_paged",
    "combine",
    "mla_decode",
    "NOPE_DIM",
    "ROPE_DIM",
    "absorb_query",
    "absorb_output",
    "kv_append",
    "schedules_in_decode",
    "prefers_in_decode",
    "kv_quantize_fp8",
    "decode_paged_fp8",
    "mla_decode_fp8",
    "FP8_TOKEN_BYTES",
    "set_debug_checks",
    "decode_step_noalloc",
    "prefill_expand_kv",
    "prefill_attention",
    "NOALLOC_SCRATCH_BYTES",
]

HEAD_DIM = 576
V_DIM = 512
PAGE_SIZE = 64
META_INTS = 8
MAX_FUSED_BATCH = 1024  # sequences for a decode that schedules itself
FP8_TOKEN_BYTES = 656  # one token of the FP8 latent cache
NOALLOC_SCRATCH_BYTES = 64 << 20  # static scratch of the no-allocation decode step, per GPU
NOPE_DIM = 128  # per-head query part before absorption; value head width
ROPE_DIM = 64

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libmla_paged.so"
_lib = None


class MlaError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG_DIR, _LIB_NAME)


def load_library() -> ctypes.CDLL:
    """Load the in-tree HIP library (built by ``python -m mla_paged_kv_06_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m mla_paged_kv_06_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    i32, sz, vp, f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float
    lib.mla_num_partitions.argtypes = [i32, i32, i32]
    lib.mla_num_partitions.restype = i32
    lib.mla_metadata_ints.argtypes = [i32, i32, i32]
    lib.mla_metadata_ints.restype = sz
    lib.mla_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.mla_workspace_bytes.restype = sz
    lib.mla_get_metadata.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
    lib.mla_get_metadata.restype = ctypes.c_int
    lib.mla_decode_paged.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32, vp, vp,
                                     i32, vp, sz, vp, vp, vp]
    lib.mla_decode_paged.restype = ctypes.c_int
    lib.mla_combine.argtypes = [vp, sz, vp, i32, i32, i32, i32, vp, vp, vp]
    lib.mla_combine.restype = ctypes.c_int
    lib.mla_absorb_query.argtypes = [vp, vp, vp, i32, i32, i32, vp, vp]
    lib.mla_absorb_query.restype = ctypes.c_int
    lib.mla_absorb_output.argtypes = [vp, vp, i32, i32, i32, vp, vp]
    lib.mla_absorb_output.restype = ctypes.c_int
    lib.mla_kv_append.argtypes = [vp, i32, vp, i32, vp, i32, vp, i32, vp, vp, vp, vp]
    lib.mla_kv_append.restype = ctypes.c_int
    lib.mla_kv_quantize_fp8.argtypes = [vp, i32, vp, vp]
    lib.mla_kv_quantize_fp8.restype = ctypes.c_int
    lib.mla_decode_paged_fp8.argtypes = list(lib.mla_decode_paged.argtypes)
    lib.mla_decode_paged_fp8.restype = ctypes.c_int
    lib.mla_probe_stream_read.argtypes = [vp, sz, vp, i32, vp]
    lib.mla_probe_stream_read.restype = ctypes.c_int
    lib.mla_probe_mfma.argtypes = [i32, i32, vp, vp, vp]
    lib.mla_probe_mfma.restype = ctypes.c_int
    lib.mla_probe_lds.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.mla_probe_lds.restype = ctypes.c_int
    lib.mla_probe_issue.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.mla_probe_issue.restype = ctypes.c_int
    lib.mla_probe_copy_ring.argtypes = [i32, vp, i32, i32, i32, vp, vp, vp]
    lib.mla_probe_copy_ring.restype = ctypes.c_int
    lib.mla_decode_step_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, f32, i32,
                                            vp, vp, vp]
    lib.mla_decode_step_noalloc.restype = ctypes.c_int
    lib.mla_prefill_expand_kv.argtypes = [vp, i32, i32, vp, vp, i32, vp, vp, vp]
    lib.mla_prefill_expand_kv.restype = ctypes.c_int
    lib.mla_prefill_attention.argtypes = [vp, vp, vp, i32, vp, vp, i32, i32, i32, f32, i32, vp,
                                          vp, vp]
    lib.mla_prefill_attention.restype = ctypes.c_int
    lib.mla_set_debug_checks.argtypes = [i32]
    lib.mla_set_debug_checks.restype = i32
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        text = load_library().mla_status_string(status).decode()
        raise MlaError(fn, status, text)


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t: Optional[torch.Tensor]) -> ctypes.c_void_p:
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, dims: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def set_debug_checks(on: Optional[bool] = None) -> bool:
    """Turn the device-content checks before every decode on or off (None
    leaves them as they are); returns the previous setting.  The default
    comes from MLA_DEBUG in the environment."""
    return bool(load_library().mla_set_debug_checks(-1 if on is None else int(bool(on))))


def num_partitions(s_q: int, h_q: int, num_cus: int = 0) -> int:
    return int(load_library().mla_num_partitions(s_q, h_q, num_cus))


def metadata_ints(s_q: int, h_q: int, num_cus: int = 0) -> int:
    return int(load_library().mla_metadata_ints(s_q, h_q, num_cus))


def workspace_bytes(batch: int, s_q: int, h_q: int, num_cus: int = 0) -> int:
    return int(load_library().mla_workspace_bytes(batch, s_q, h_q, num_cus))


def get_metadata(cache_seqlens: torch.Tensor, s_q: int, h_q: int, num_cus: int = 0,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split-KV schedule: returns ``(tile_metadata [parts, 8], num_splits [batch+1])``."""
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    batch = cache_seqlens.shape[0]
    parts = num_partitions(s_q, h_q, num_cus)
    if parts <= 0:
        raise MlaError("mla_num_partitions", 1, "invalid arguments")
    dev = cache_seqlens.device
    meta = torch.empty((parts, META_INTS), dtype=torch.int32, device=dev)
    splits = torch.empty((batch + 1,), dtype=torch.int32, device=dev)
    _check("mla_get_metadata", load_library().mla_get_metadata(
        _ptr(cache_seqlens), batch, s_q, h_q, num_cus, _ptr(meta), _ptr(splits), _stream(stream)))
    return meta, splits


def decode_paged(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                 cache_seqlens: torch.Tensor, softmax_scale: float, causal: bool,
                 tile_metadata: Optional[torch.Tensor], num_splits: torch.Tensor,
                 num_cus: int = 0, workspace: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 stream=None):
    """Decode (without the combine).  Returns ``(out, lse, workspace)``.  With
    ``tile_metadata=None`` (at most 1024 sequences) the decode schedules itself
    and writes ``num_splits``."""
    _need(q, "q", torch.bfloat16, 4)
    _need(kv_cache, "kv_cache", torch.bfloat16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    batch, s_q, h_q, d = q.shape
    if d != HEAD_DIM or kv_cache.shape[1] != PAGE_SIZE or kv_cache.shape[2] != HEAD_DIM:
        raise ValueError("q must be [b,s_q,h_q,576] and kv_cache [pages,64,576]")
    if block_table.shape[0] != batch or cache_seqlens.shape[0] != batch:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    dev = q.device
    if out is None:
        out = torch.empty((batch, s_q, h_q, V_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=dev)
    need = workspace_bytes(batch, s_q, h_q, num_cus)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _check("mla_decode_paged", load_library().mla_decode_paged(
        _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(cache_seqlens), batch, s_q, h_q,
        kv_cache.shape[0], block_table.shape[1], float(softmax_scale), int(bool(causal)),
        _ptr(tile_metadata), _ptr(num_splits), num_cus, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse, workspace


def kv_quantize_fp8(kv_cache: torch.Tensor, out: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """bf16 cache [pages, 64, 576] -> FP8 records [pages, 64, 656] (uint8):
    512 E4M3 latent codes, four float32 power-of-two block scales, the 64
    rotary values in bf16."""
    _need(kv_cache, "kv_cache", torch.bfloat16, 3)
    if kv_cache.shape[1] != PAGE_SIZE or kv_cache.shape[2] != HEAD_DIM:
        raise ValueError("kv_cache must be [pages,64,576]")
    P = kv_cache.shape[0]
    if out is None:
        out = torch.empty((P, PAGE_SIZE, FP8_TOKEN_BYTES), dtype=torch.uint8, device=kv_cache.device)
    if out.dtype != torch.uint8 or tuple(out.shape) != (P, PAGE_SIZE, FP8_TOKEN_BYTES) or \
            not out.is_contiguous():
        raise ValueError("out must be contiguous uint8 [pages,64,656]")
    _check("mla_kv_quantize_fp8", load_library().mla_kv_quantize_fp8(
        _ptr(kv_cache), P, _ptr(out), _stream(stream)))
    return out


def decode_paged_fp8(q: torch.Tensor, kv_fp8: torch.Tensor, block_table: torch.Tensor,
                     cache_seqlens: torch.Tensor, softmax_scale: float, causal: bool,
                     tile_metadata: torch.Tensor, num_splits: torch.Tensor, num_cus: int = 0,
                     workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     lse: Optional[torch.Tensor] = None, stream=None):
    """Decode over the FP8 cache (at most 16 rows per sequence; the schedule
    from get_metadata).  Returns ``(out, lse, workspace)``; combine as usual."""
    _need(q, "q", torch.bfloat16, 4)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    if kv_fp8.dtype != torch.uint8 or kv_fp8.dim() != 3 or not kv_fp8.is_contiguous() or \
            kv_fp8.shape[1] != PAGE_SIZE or kv_fp8.shape[2] != FP8_TOKEN_BYTES:
        raise ValueError("kv_fp8 must be contiguous uint8 [pages,64,656]")
    batch, s_q, h_q, d = q.shape
    if d != HEAD_DIM:
        raise ValueError("q must be [b,s_q,h_q,576]")
    if block_table.shape[0] != batch or cache_seqlens.shape[0] != batch:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    dev = q.device
    if out is None:
        out = torch.empty((batch, s_q, h_q, V_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((batch, s_q, h_q), dtype=torch.float32, device=dev)
    need = workspace_bytes(batch, s_q, h_q, num_cus)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev)
    _check("mla_decode_paged_fp8", load_library().mla_decode_paged_fp8(
        _ptr(q), _ptr(kv_fp8), _ptr(block_table), _ptr(cache_seqlens), batch, s_q, h_q,
        kv_fp8.shape[0], block_table.shape[1], float(softmax_scale), int(bool(causal)),
        _ptr(tile_metadata), _ptr(num_splits), num_cus, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse, workspace


def mla_decode_fp8(q, kv_fp8, block_table, cache_seqlens, softmax_scale, causal, num_cus: int = 0,
                   stream=None):
    """One full decode step over the FP8 cache: schedule, decode, combine."""
    batch, s_q, h_q, _ = q.shape
    meta, splits = get_metadata(cache_seqlens, s_q, h_q, num_cus, stream)
    out, lse, ws = decode_paged_fp8(q, kv_fp8, block_table, cache_seqlens, softmax_scale, causal,
                                    meta, splits, num_cus, stream=stream)
    combine(ws, splits, batch, s_q, h_q, out, lse, num_cus, stream)
    return out, lse


def combine(workspace: torch.Tensor, num_splits: torch.Tensor, batch: int, s_q: int, h_q: int,
            out: torch.Tensor, lse: torch.Tensor, num_cus: int = 0, stream=None) -> None:
    """Merge split partials into ``out`` / ``lse`` in place."""
    _check("mla_combine", load_library().mla_combine(
        _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(num_splits), batch,
        s_q, h_q, num_cus, _ptr(out), _ptr(lse), _stream(stream)))


def schedules_in_decode(batch: int, s_q: int, h_q: int, max_pages: int = 0) -> bool:
    """Whether the decode can compute the split-KV schedule in its own launch
    (at most 1024 sequences, and a block table small enough for its 32-bit
    unit arithmetic)."""
    return batch <= MAX_FUSED_BATCH and batch * (max_pages + 2) < (1 << 30)


def prefers_in_decode(batch: int, s_q: int, h_q: int, max_pages: int = 0) -> bool:
    """Whether the schedule inside the decode is the faster choice: wherever
    the decode can compute it (one schedule launch saved).  Measured faster
    or even at 16, 32, 64, 128 and 256 rows per sequence, and even with a
    single partition."""
    return schedules_in_decode(batch, s_q, h_q, max_pages)


def mla_decode(q, kv_cache, block_table, cache_seqlens, softmax_scale, causal, num_cus: int = 0,
               stream=None, schedule: str = "auto"):
    """One full decode step: schedule, decode, combine.  Returns ``(out, lse)``.

    ``schedule``: "separate" (mla_get_metadata, then the decode), "in_decode"
    (the decode schedules itself; at most 1024 sequences) or "auto" (in the
    decode when it can)."""
    batch, s_q, h_q, _ = q.shape
    if schedule not in ("auto", "separate", "in_decode"):
        raise ValueError(f"unknown schedule {schedule!r}")
    fused = schedule == "in_decode" or (
        schedule == "auto" and prefers_in_decode(batch, s_q, h_q, int(block_table.shape[1])))
    if fused:
        meta = None
        splits = torch.empty((batch + 1,), dtype=torch.int32, device=q.device)
    else:
        meta, splits = get_metadata(cache_seqlens, s_q, h_q, num_cus, stream)
    out, lse, ws = decode_paged(q, kv_cache, block_table, cache_seqlens, softmax_scale, causal,
                                meta, splits, num_cus, stream=stream)
    combine(ws, splits, batch, s_q, h_q, out, lse, num_cus, stream)
    return out, lse


def decode_step_noalloc(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                        cache_seqlens: torch.Tensor, softmax_scale: float, causal: bool,
                        out: torch.Tensor, lse: torch.Tensor, stream=None) -> None:
    """One whole decode step (schedule, decode, combine) into the given
    ``out`` / ``lse``, with the library's static per-GPU scratch instead of
    a workspace: nothing is allocated.  Calls that overlap on one GPU race."""
    _need(q, "q", torch.bfloat16, 4)
    _need(kv_cache, "kv_cache", torch.bfloat16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    _need(out, "out", torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    batch, s_q, h_q, d = q.shape
    if d != HEAD_DIM or kv_cache.shape[1] != PAGE_SIZE or kv_cache.shape[2] != HEAD_DIM:
        raise ValueError("q must be [b,s_q,h_q,576] and kv_cache [pages,64,576]")
    if block_table.shape[0] != batch or cache_seqlens.shape[0] != batch:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    if tuple(out.shape) != (batch, s_q, h_q, V_DIM) or tuple(lse.shape) != (batch, s_q, h_q):
        raise ValueError("out must be [b,s_q,h_q,512] and lse [b,s_q,h_q]")
    _check("mla_decode_step_noalloc", load_library().mla_decode_step_noalloc(
        _ptr(q), _ptr(kv_cache), _ptr(block_table), _ptr(cache_seqlens), batch, s_q, h_q,
        kv_cache.shape[0], block_table.shape[1], float(softmax_scale), int(bool(causal)),
        _ptr(out), _ptr(lse), _stream(stream)))


def prefill_expand_kv(latent: torch.Tensor, w_uk: torch.Tensor, w_uv: torch.Tensor,
                      k_nope: Optional[torch.Tensor] = None, v: Optional[torch.Tensor] = None,
                      stream=None):
    """Widen the latents per head for prefill: ``latent [T, >=512]`` (c_t =
    the first 512 values of row t), ``w_uk`` and ``w_uv [h, 128, 512]`` ->
    ``k_nope[t, h] = W_UK,h c_t`` and ``v[t, h] = W_UV,h c_t``, each
    ``[T, h, 128]``."""
    if latent.dim() != 2 or latent.dtype != torch.bfloat16 or latent.stride(1) != 1:
        raise ValueError("latent must be a bf16 [T, >=512] matrix with unit column stride")
    _need(w_uk, "w_uk", torch.bfloat16, 3)
    _need(w_uv, "w_uv", torch.bfloat16, 3)
    T = latent.shape[0]
    h_q = w_uk.shape[0]
    if tuple(w_uk.shape) != (h_q, NOPE_DIM, V_DIM) or tuple(w_uv.shape) != (h_q, NOPE_DIM, V_DIM):
        raise ValueError("w_uk and w_uv must be [h, 128, 512]")
    dev = latent.device
    if k_nope is None:
        k_nope = torch.empty((T, h_q, NOPE_DIM), dtype=torch.bfloat16, device=dev)
    if v is None:
        v = torch.empty((T, h_q, NOPE_DIM), dtype=torch.bfloat16, device=dev)
    _need(k_nope, "k_nope", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _check("mla_prefill_expand_kv", load_library().mla_prefill_expand_kv(
        _ptr(latent), latent.stride(0), T, _ptr(w_uk), _ptr(w_uv), h_q, _ptr(k_nope), _ptr(v),
        _stream(stream)))
    return k_nope, v


def prefill_attention(q: torch.Tensor, k_nope: torch.Tensor, k_rope: torch.Tensor,
                      v: torch.Tensor, cu_seqlens: torch.Tensor, max_seqlen: int,
                      softmax_scale: float, causal: bool = True,
                      o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                      stream=None):
    """Per-head attention over packed prompts: ``q [T, h, 192]``, ``k_nope``
    and ``v [T, h, 128]``, ``k_rope [T, 64]`` (any row stride, e.g. the last
    64 values of the cache entries), ``cu_seqlens [batch + 1]`` int32.
    Returns ``(o [T, h, 128], lse [T, h])``."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_nope, "k_nope", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    if k_rope.dim() != 2 or k_rope.dtype != torch.bfloat16 or k_rope.stride(1) != 1 or \
            k_rope.shape[1] != ROPE_DIM:
        raise ValueError("k_rope must be a bf16 [T, 64] matrix with unit column stride")
    T, h_q, d = q.shape
    if d != NOPE_DIM + ROPE_DIM or tuple(k_nope.shape) != (T, h_q, NOPE_DIM) or \
            tuple(v.shape) != (T, h_q, NOPE_DIM) or k_rope.shape[0] != T:
        raise ValueError("q [T,h,192], k_nope / v [T,h,128] and k_rope [T,64] must agree")
    dev = q.device
    if o is None:
        o = torch.empty((T, h_q, NOPE_DIM), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((T, h_q), dtype=torch.float32, device=dev)
    _check("mla_prefill_attention", load_library().mla_prefill_attention(
        _ptr(q), _ptr(k_nope), _ptr(k_rope), k_rope.stride(0), _ptr(v), _ptr(cu_seqlens),
        cu_seqlens.shape[0] - 1, h_q, int(max_seqlen), float(softmax_scale), int(bool(causal)),
        _ptr(o), _ptr(lse), _stream(stream)))
    return o, lse


def absorb_query(q_nope: torch.Tensor, q_rope: torch.Tensor, w_uk_t: torch.Tensor,
                 q_out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Absorbed query ``[W_UK,h^T q_nope ; q_rope]`` per head: ``q_nope [b,s_q,h,128]``,
    ``q_rope [b,s_q,h,64]``, ``w_uk_t [h,512,128]`` -> ``q_out [b,s_q,h,576]``."""
    _need(q_nope, "q_nope", torch.bfloat16, 4)
    _need(q_rope, "q_rope", torch.bfloat16, 4)
    _need(w_uk_t, "w_uk_t", torch.bfloat16, 3)
    batch, s_q, h_q, d = q_nope.shape
    if d != NOPE_DIM or tuple(q_rope.shape) != (batch, s_q, h_q, ROPE_DIM):
        raise ValueError("q_nope must be [b,s_q,h_q,128] and q_rope [b,s_q,h_q,64]")
    if tuple(w_uk_t.shape) != (h_q, V_DIM, NOPE_DIM):
        raise ValueError("w_uk_t must be [h_q,512,128]")
    if q_out is None:
        q_out = torch.empty((batch, s_q, h_q, HEAD_DIM), dtype=torch.bfloat16, device=q_nope.device)
    _need(q_out, "q_out", torch.bfloat16, 4)
    _check("mla_absorb_query", load_library().mla_absorb_query(
        _ptr(q_nope), _ptr(q_rope), _ptr(w_uk_t), batch, s_q, h_q, _ptr(q_out), _stream(stream)))
    return q_out


def absorb_output(out: torch.Tensor, w_uv: torch.Tensor, o: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """Per-head output ``W_UV,h out``: ``out [b,s_q,h,512]``, ``w_uv [h,128,512]`` ->
    ``o [b,s_q,h,128]``."""
    _need(out, "out", torch.bfloat16, 4)
    _need(w_uv, "w_uv", torch.bfloat16, 3)
    batch, s_q, h_q, d = out.shape
    if d != V_DIM or tuple(w_uv.shape) != (h_q, NOPE_DIM, V_DIM):
        raise ValueError("out must be [b,s_q,h_q,512] and w_uv [h_q,128,512]")
    if o is None:
        o = torch.empty((batch, s_q, h_q, NOPE_DIM), dtype=torch.bfloat16, device=out.device)
    _need(o, "o", torch.bfloat16, 4)
    _check("mla_absorb_output", load_library().mla_absorb_output(
        _ptr(out), _ptr(w_uv), batch, s_q, h_q, _ptr(o), _stream(stream)))
    return o


def kv_append(kv_cache: torch.Tensor, block_table: torch.Tensor, cache_seqlens: torch.Tensor,
              new_kv: torch.Tensor, free_pages: torch.Tensor, free_count: torch.Tensor,
              status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Append ``new_kv [b, n_new, 576]`` to each sequence's pages, taking new
    pages from the top of the ``free_pages`` stack (``free_count [1]`` entries
    valid); updates ``kv_cache``, ``block_table``, ``cache_seqlens`` and
    ``free_count`` in place.  Returns the device status word (0 = done, 1 =
    too few free pages or a table row too short: nothing written)."""
    _need(kv_cache, "kv_cache", torch.bfloat16, 3)
    _need(block_table, "block_table", torch.int32, 2)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    _need(new_kv, "new_kv", torch.bfloat16, 3)
    _need(free_pages, "free_pages", torch.int32, 1)
    _need(free_count, "free_count", torch.int32, 1)
    batch, n_new, d = new_kv.shape
    if d != HEAD_DIM or kv_cache.shape[1] != PAGE_SIZE or kv_cache.shape[2] != HEAD_DIM:
        raise ValueError("new_kv must be [b,n_new,576] and kv_cache [pages,64,576]")
    if block_table.shape[0] != batch or cache_seqlens.shape[0] != batch:
        raise ValueError("block_table / cache_seqlens batch mismatch")
    if status is None:
        status = torch.empty((1,), dtype=torch.int32, device=kv_cache.device)
    _check("mla_kv_append", load_library().mla_kv_append(
        _ptr(kv_cache), kv_cache.shape[0], _ptr(block_table), block_table.shape[1],
        _ptr(cache_seqlens), batch, _ptr(new_kv), n_new, _ptr(free_pages), _ptr(free_count),
        _ptr(status), _stream(stream)))
    return status
