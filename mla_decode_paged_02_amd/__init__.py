"""Python binding of libmla355 (MLA attention over a paged latent KV cache on MI355X).

Argument marshalling only: every step of the computation runs in the HIP kernels of
libmla355.so.  PyTorch supplies device memory and the current stream; the functions
build plain C descriptors (pointer, element type, shape, strides) from tensors without
copying them and call the C ABI declared in include/mla355.h.  If the shared library is
missing or fails to load, every call raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LIBRARY_PATH", "MlaError", "library", "decode_paged", "decode_paged_noalloc",
    "decode_noalloc_scratch_bytes", "decode_paged_sparse", "decode_paged_sparse_shared",
    "decode_paged_sparse_ext", "decode_paged_fp8", "indexer_paged_fp8", "prefill_paged", "decode_num_partitions",
    "decode_workspace_bytes", "indexer_workspace_bytes", "reserve_workspace", "check_device_errors", "shutdown",
    "version", "profile_enable", "profile_read", "profile_read_each", "MASKS", "STATUS",
]

LIBRARY_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla355.so")

MASKS = {"null": 0, "causal": 1, "sliding_window_causal": 2}
STATUS = {0: "MLA_OK", 1: "MLA_ERR_NULL_ARG", 2: "MLA_ERR_SHAPE", 3: "MLA_ERR_DTYPE",
          4: "MLA_ERR_ALIGNMENT", 5: "MLA_ERR_UNSUPPORTED", 6: "MLA_ERR_WORKSPACE",
          7: "MLA_ERR_HIP", 8: "MLA_ERR_VALUE"}
DT_BF16, DT_FP8, DT_F32, DT_I32, DT_U32 = 0, 1, 2, 3, 4


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class MlaTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


_LIB = None


def library() -> ctypes.CDLL:
    """Load libmla355.so from this package directory (raises if it is not built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIBRARY_PATH):
            raise MlaError(5, f"{LIBRARY_PATH} is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(LIBRARY_PATH)
        P = ctypes.POINTER(MlaTensor)
        i32, f32, vp = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p
        lib.mla_decode_paged.argtypes = [P, P, P, P, P, f32, i32, i32, i32, P, vp]
        lib.mla_decode_paged_noalloc.argtypes = [P, P, P, P, P, f32, i32, i32, i32, P, vp]
        lib.mla_decode_noalloc_scratch_bytes.argtypes = []
        lib.mla_decode_noalloc_scratch_bytes.restype = ctypes.c_size_t
        lib.mla_decode_paged_sparse.argtypes = [P, P, P, P, P, P, P, f32, i32, P, vp]
        lib.mla_decode_paged_sparse_shared.argtypes = [P, P, P, P, P, P, P, f32, i32, P, vp]
        lib.mla_decode_paged_sparse_ext.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, f32, i32, P, vp]
        lib.mla_decode_paged_fp8.argtypes = [P, P, P, P, P, P, P, f32, i32, i32, i32, P, vp]
        lib.mla_indexer_paged_fp8.argtypes = [P, P, P, P, P, P, P, i32, i32, P, vp]
        lib.mla_prefill_paged.argtypes = [P, P, P, P, P, P, P, P, P, f32, i32, P, vp]
        for fn in ("mla_decode_paged", "mla_decode_paged_noalloc", "mla_decode_paged_sparse", "mla_decode_paged_sparse_shared", "mla_decode_paged_sparse_ext", "mla_decode_paged_fp8", "mla_indexer_paged_fp8", "mla_prefill_paged",
                   "mla_reserve_workspace", "mla_check_device_errors"):
            getattr(lib, fn).restype = ctypes.c_int
        lib.mla_decode_workspace_bytes.argtypes = [ctypes.c_int64, i32, i32, i32]
        lib.mla_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.mla_indexer_workspace_bytes.argtypes = [ctypes.c_int64, i32, i32]
        lib.mla_indexer_workspace_bytes.restype = ctypes.c_size_t
        lib.mla_reserve_workspace.argtypes = [i32, vp, ctypes.c_size_t]
        lib.mla_check_device_errors.argtypes = [i32, vp, ctypes.POINTER(ctypes.c_uint32)]
        lib.mla_profile_enable.argtypes = [i32]
        lib.mla_profile_enable.restype = ctypes.c_int
        lib.mla_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
        lib.mla_profile_read.restype = ctypes.c_int
        lib.mla_profile_read_each.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_int64,
                                              ctypes.POINTER(ctypes.c_int64)]
        lib.mla_profile_read_each.restype = ctypes.c_int
        lib.mla_decode_num_partitions.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, i32]
        lib.mla_decode_num_partitions.restype = ctypes.c_int32
        lib.mla_shutdown.argtypes = []
        lib.mla_shutdown.restype = None
        lib.mla_status_string.argtypes = [ctypes.c_int]
        lib.mla_status_string.restype = ctypes.c_char_p
        lib.mla_last_error_message.argtypes = []
        lib.mla_last_error_message.restype = ctypes.c_char_p
        lib.mla_version.argtypes = []
        lib.mla_version.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def _check(status: int) -> None:
    if status != 0:
        msg = library().mla_last_error_message().decode()
        raise MlaError(status, msg)


def _dtype_code(t) -> int:
    import torch
    table = {torch.bfloat16: DT_BF16, torch.float8_e4m3fn: DT_FP8, torch.uint8: DT_FP8,
             torch.float32: DT_F32, torch.int32: DT_I32}
    if hasattr(torch, "uint32"):
        table[torch.uint32] = DT_U32
    if t.dtype not in table:
        raise MlaError(3, f"unsupported tensor dtype {t.dtype}")
    return table[t.dtype]


def _desc(t, as_dtype: int | None = None):
    """A descriptor of tensor ``t`` (None -> NULL).  ``as_dtype`` reinterprets the element
    type with the same width (int32 offsets passed as uint32)."""
    if t is None:
        return None
    if t.dim() > 4:
        raise MlaError(2, "at most 4 dimensions")
    d = MlaTensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _dtype_code(t) if as_dtype is None else as_dtype
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return ctypes.byref(d)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _on_gpu(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise MlaError(2, "tensors must be on the GPU")


def _offsets(t):
    import torch
    if t.dtype == torch.int32:
        return _desc(t, DT_U32)
    return _desc(t)


def decode_paged(q, input_row_offsets, page_table, cache_lens, latent_cache, scale,
                 mask="causal", local_window_size=-1, num_partitions=0, out=None, stream=None):
    """Dense MLA decode (mla_decode_paged).  q bf16 [T, H, 576]; latent_cache bf16
    [num_pages, PS, 576]; returns out bf16 [T, H, 512] (allocated if not given)."""
    import torch
    _on_gpu(q, input_row_offsets, page_table, cache_lens, latent_cache, out)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], 512), dtype=torch.bfloat16, device=q.device)
    _check(library().mla_decode_paged(
        _desc(q), _offsets(input_row_offsets), _desc(page_table), _desc(cache_lens),
        _desc(latent_cache), float(scale), MASKS[mask] if isinstance(mask, str) else int(mask),
        int(local_window_size), int(num_partitions), _desc(out), _stream(stream)))
    return out


def decode_paged_noalloc(q, input_row_offsets, page_table, cache_lens, latent_cache, scale,
                         mask="causal", local_window_size=-1, num_partitions=0, out=None, stream=None):
    """decode_paged through mla_decode_paged_noalloc (the library allocates nothing; its
    workspace is a fixed per-GPU array).  `out` should be given by callers that cannot
    allocate; without it one is allocated here, by torch."""
    import torch
    _on_gpu(q, input_row_offsets, page_table, cache_lens, latent_cache, out)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], 512), dtype=torch.bfloat16, device=q.device)
    _check(library().mla_decode_paged_noalloc(
        _desc(q), _offsets(input_row_offsets), _desc(page_table), _desc(cache_lens),
        _desc(latent_cache), float(scale), MASKS[mask] if isinstance(mask, str) else int(mask),
        int(local_window_size), int(num_partitions), _desc(out), _stream(stream)))
    return out


def decode_noalloc_scratch_bytes() -> int:
    return int(library().mla_decode_noalloc_scratch_bytes())


def decode_paged_sparse(q, q_scale, input_row_offsets, latent_cache, cache_scale, d_indices,
                        topk_lengths, scale, num_partitions=0, out=None, stream=None):
    """Sparse MLA decode (mla_decode_paged_sparse).  q / latent_cache fp8 e4m3 (torch
    float8_e4m3fn or uint8 codes) or bf16, or uint8 rows of 640 bytes in the rope-aware
    layout; returns out bf16 [T, H, 512]."""
    import torch
    _on_gpu(q, q_scale, input_row_offsets, latent_cache, cache_scale, d_indices, topk_lengths, out)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], 512), dtype=torch.bfloat16, device=q.device)
    _check(library().mla_decode_paged_sparse(
        _desc(q), _desc(q_scale), _offsets(input_row_offsets), _desc(latent_cache),
        _desc(cache_scale), _desc(d_indices), _desc(topk_lengths), float(scale),
        int(num_partitions), _desc(out), _stream(stream)))
    return out


def decode_paged_sparse_shared(q, q_scale, input_row_offsets, latent_cache, cache_scale, d_indices,
                               topk_lengths, scale, num_partitions=0, out=None, stream=None):
    """Sparse MLA decode where the query tokens of a sequence share its index list
    (mla_decode_paged_sparse_shared): d_indices i32 [B, stride] and topk_lengths i32 [B],
    one per sequence of input_row_offsets; otherwise as decode_paged_sparse."""
    import torch
    _on_gpu(q, q_scale, input_row_offsets, latent_cache, cache_scale, d_indices, topk_lengths, out)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], 512), dtype=torch.bfloat16, device=q.device)
    _check(library().mla_decode_paged_sparse_shared(
        _desc(q), _desc(q_scale), _offsets(input_row_offsets), _desc(latent_cache),
        _desc(cache_scale), _desc(d_indices), _desc(topk_lengths), float(scale),
        int(num_partitions), _desc(out), _stream(stream)))
    return out


def decode_paged_sparse_ext(q, q_scale, input_row_offsets, latent_cache, cache_scale, d_indices,
                            topk_lengths, scale, attn_sink=None, extra_cache=None, extra_cache_scale=None,
                            extra_d_indices=None, extra_topk_lengths=None, num_partitions=0, out=None,
                            stream=None):
    """Sparse MLA decode with an attention sink (f32 [H] logits) and a second KV stream
    (mla_decode_paged_sparse_ext); returns out bf16 [T, H, 512]."""
    import torch
    _on_gpu(q, q_scale, input_row_offsets, latent_cache, cache_scale, d_indices, topk_lengths, attn_sink,
            extra_cache, extra_cache_scale, extra_d_indices, extra_topk_lengths, out)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], 512), dtype=torch.bfloat16, device=q.device)
    _check(library().mla_decode_paged_sparse_ext(
        _desc(q), _desc(q_scale), _offsets(input_row_offsets), _desc(latent_cache),
        _desc(cache_scale), _desc(d_indices), _desc(topk_lengths), _desc(attn_sink), _desc(extra_cache),
        _desc(extra_cache_scale), _desc(extra_d_indices), _desc(extra_topk_lengths), float(scale),
        int(num_partitions), _desc(out), _stream(stream)))
    return out


def decode_paged_fp8(q, q_scale, input_row_offsets, page_table, cache_lens, latent_cache, cache_scale,
                     scale, mask="causal", local_window_size=-1, num_partitions=0, out=None, stream=None):
    """Dense MLA decode over a paged fp8 cache (mla_decode_paged_fp8).  q fp8 e4m3
    [T, H, 576] with q_scale f32 [T] or None; latent_cache fp8 e4m3 [num_pages, PS, 576]
    with cache_scale f32 [num_pages, PS] or None (torch float8_e4m3fn or uint8 codes);
    q [T, H, 640] and latent_cache [num_pages, PS, 640] (uint8) select the rope-aware
    layout (512 e4m3 latent codes, then 64 little-endian bf16 rope values, the scale on the
    codes only); returns out bf16 [T, H, 512]."""
    import torch
    _on_gpu(q, q_scale, input_row_offsets, page_table, cache_lens, latent_cache, cache_scale, out)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], 512), dtype=torch.bfloat16, device=q.device)
    _check(library().mla_decode_paged_fp8(
        _desc(q), _desc(q_scale), _offsets(input_row_offsets), _desc(page_table), _desc(cache_lens),
        _desc(latent_cache), _desc(cache_scale), float(scale),
        MASKS[mask] if isinstance(mask, str) else int(mask), int(local_window_size),
        int(num_partitions), _desc(out), _stream(stream)))
    return out


def indexer_paged_fp8(q, q_s, input_row_offsets, page_table, cache_lens, k_cache, k_scale, top_k,
                      mask="causal", local_window_size=-1, out=None, stream=None):
    """FP8 top-k indexer (mla_indexer_paged_fp8).  q fp8 e4m3 [T, NH, D] with q_s f32
    [T, NH]; k_cache fp8 e4m3 [num_pages, PS, D] with k_scale f32 [num_pages, PS] or None;
    returns int32 [T, top_k] physical rows, -1 filled."""
    import torch
    _on_gpu(q, q_s, input_row_offsets, page_table, cache_lens, k_cache, k_scale, out)
    if out is None:
        out = torch.empty((q.shape[0], int(top_k)), dtype=torch.int32, device=q.device)
    _check(library().mla_indexer_paged_fp8(
        _desc(q), _desc(q_s), _offsets(input_row_offsets), _desc(page_table), _desc(cache_lens),
        _desc(k_cache), _desc(k_scale), MASKS[mask] if isinstance(mask, str) else int(mask),
        int(local_window_size), _desc(out), _stream(stream)))
    return out


def prefill_paged(q, k, v, buffer_row_offsets, cache_offsets, input_row_offsets, page_table,
                  cache_lens, latent_cache, scale, mask="causal", out=None, stream=None):
    """Ragged MLA prefill (mla_prefill_paged); returns out bf16 [Tq, H, 128]."""
    import torch
    _on_gpu(q, k, v, buffer_row_offsets, cache_offsets, input_row_offsets, page_table,
            cache_lens, latent_cache, out)
    if out is None:
        out = torch.empty((q.shape[0], q.shape[1], 128), dtype=torch.bfloat16, device=q.device)
    _check(library().mla_prefill_paged(
        _desc(q), _desc(k), _desc(v), _offsets(buffer_row_offsets), _offsets(cache_offsets),
        _offsets(input_row_offsets), _desc(page_table), _desc(cache_lens), _desc(latent_cache),
        float(scale), MASKS[mask] if isinstance(mask, str) else int(mask), _desc(out),
        _stream(stream)))
    return out


def decode_num_partitions(batch, num_heads, max_pages, page_size) -> int:
    """The split-KV partition count the balanced split gives each row of a batch of
    `batch` single-token sequences of max_pages * page_size keys (mla_decode_num_partitions;
    0 for out-of-range arguments)."""
    return int(library().mla_decode_num_partitions(int(batch), int(num_heads), int(max_pages),
                                                   int(page_size)))


def decode_workspace_bytes(total_q, num_heads, num_partitions=0, device=-1) -> int:
    return int(library().mla_decode_workspace_bytes(int(total_q), int(num_heads),
                                                    int(num_partitions), int(device)))


def indexer_workspace_bytes(total_q, max_pages, page_size) -> int:
    return int(library().mla_indexer_workspace_bytes(int(total_q), int(max_pages), int(page_size)))


def reserve_workspace(nbytes, device=-1, stream=None) -> None:
    _check(library().mla_reserve_workspace(int(device), _stream(stream), int(nbytes)))


def check_device_errors(device=-1, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _check(library().mla_check_device_errors(int(device), _stream(stream), ctypes.byref(flags)))
    return int(flags.value)


def profile_enable(enable: bool = True) -> None:
    """Bracket each call's main kernel with HIP events on the call's stream."""
    _check(library().mla_profile_enable(1 if enable else 0))


def profile_read() -> tuple[float, int]:
    """(summed milliseconds, launches) of the bracketed kernels since the last read."""
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _check(library().mla_profile_read(ctypes.byref(ms), ctypes.byref(n)))
    return float(ms.value), int(n.value)


def profile_read_each(capacity: int = 4096) -> list[float]:
    """Milliseconds of each bracketed kernel since the last read, in call order."""
    buf = (ctypes.c_double * max(1, int(capacity)))()
    n = ctypes.c_int64(0)
    _check(library().mla_profile_read_each(buf, int(capacity), ctypes.byref(n)))
    return [float(buf[i]) for i in range(min(int(n.value), int(capacity)))]


def shutdown() -> None:
    library().mla_shutdown()


def version() -> str:
    return library().mla_version().decode()
