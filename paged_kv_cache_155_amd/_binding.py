"""ctypes binding of libpa.so (declared in include/pa.h).

Argument marshalling only: shape/dtype/device checks, raw pointers and the
current HIP stream.  torch supplies device memory and streams; every step of
the computation runs in the library's HIP kernels.  There is no fallback:
if libpa.so is missing or cannot be loaded, every call raises.
"""
import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PA_LIB", os.path.join(_PKG, "libpa.so"))

PA_OK = 0

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_lib = None


class PAError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, code, where):
        self.code = code
        super().__init__(f"{where}: {status_string(code)} ({code})")


def load(path=None):
    """Load (once) and return the ctypes handle on libpa.so."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"HIP library not built: {p} is missing (build it with "
            f"`python -m paged_kv_cache_155_amd._build` or __graft_entry__.build())")
    # torch ships its own HIP runtime (torch/lib/libamdhip64.so).  libpa.so
    # must bind to that one: loaded before torch, it would pull in the system
    # runtime as well, and its launches could not use torch's memory and
    # streams.  With torch loaded, libpa.so's libamdhip64.so.7 dependency
    # resolves to the runtime already in the process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(p)
    lib.pa_reshape_and_cache.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P]
    lib.pa_reshape_and_cache.restype = ctypes.c_int
    lib.pa_decode_workspace_size.argtypes = [_I32] * 6
    lib.pa_decode_workspace_size.restype = ctypes.c_size_t
    lib.pa_decode.argtypes = ([_P] * 6 + [_I32] * 6 + [ctypes.c_float, _I32, _P, ctypes.c_size_t,
                                                       _P])
    lib.pa_decode.restype = ctypes.c_int
    lib.pa_decode_noalloc.argtypes = [_P] * 6 + [_I32] * 6 + [ctypes.c_float, _I32, _P]
    lib.pa_decode_noalloc.restype = ctypes.c_int
    lib.pa_reshape_and_cache_fp8.argtypes = ([_P, _P, _P, _P, _P] + [_I32] * 5
                                             + [ctypes.c_float, ctypes.c_float, _P])
    lib.pa_reshape_and_cache_fp8.restype = ctypes.c_int
    lib.pa_decode_fp8.argtypes = ([_P] * 6 + [_I32] * 6 + [ctypes.c_float] * 3
                                  + [_I32, _P, ctypes.c_size_t, _P])
    lib.pa_decode_fp8.restype = ctypes.c_int
    lib.pa_decode_cascade_workspace_size.argtypes = [_I32] * 7
    lib.pa_decode_cascade_workspace_size.restype = ctypes.c_size_t
    lib.pa_decode_cascade.argtypes = ([_P] * 5 + [_I32] + [_P] * 2 + [_I32] * 6
                                      + [ctypes.c_float, _I32, _P, ctypes.c_size_t, _P])
    lib.pa_decode_cascade.restype = ctypes.c_int
    lib.pa_decode_cascade_append.argtypes = ([_P] * 8 + [_I32] + [_P] * 2 + [_I32] * 6
                                             + [ctypes.c_float, _I32, _P, ctypes.c_size_t, _P])
    lib.pa_decode_cascade_append.restype = ctypes.c_int
    lib.pa_decode_cascade_fp8.argtypes = ([_P] * 5 + [_I32] + [_P] * 2 + [_I32] * 6
                                          + [ctypes.c_float] * 3
                                          + [_I32, _P, ctypes.c_size_t, _P])
    lib.pa_decode_cascade_fp8.restype = ctypes.c_int
    lib.pa_decode_cascade_append_fp8.argtypes = ([_P] * 8 + [_I32] + [_P] * 2 + [_I32] * 6
                                                 + [ctypes.c_float] * 3
                                                 + [_I32, _P, ctypes.c_size_t, _P])
    lib.pa_decode_cascade_append_fp8.restype = ctypes.c_int
    lib.pa_multi_query.argtypes = [_P] * 7 + [_I32] * 8 + [ctypes.c_float, _P]
    lib.pa_multi_query.restype = ctypes.c_int
    lib.pa_multi_query_fp8.argtypes = [_P] * 7 + [_I32] * 8 + [ctypes.c_float] * 3 + [_P]
    lib.pa_multi_query_fp8.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P]
    lib.pa_copy_blocks.restype = ctypes.c_int
    lib.pa_swap_blocks.argtypes = [_P, _P, _P, _I32, _I32, _I32, ctypes.c_int64, _P]
    lib.pa_swap_blocks.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def status_string(code):
    return load().pa_status_string(int(code)).decode()


def _stream_ptr(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(t, name, dtype, shape=None, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _alloc_workspace(nbytes, device, stream):
    """A uint8 workspace for kernels launched on `stream` (None: the current
    stream).  It is allocated while that stream is current, so when the
    tensor is released the caching allocator hands its memory only to work
    ordered after these kernels on the same stream."""
    import torch
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, stream=None):
    """Write key/value [T, H, D] fp16 into k_cache/v_cache [NB, B, H, D] at
    slot_mapping [T] int64 (slot = block * B + offset; out-of-range slots,
    e.g. -1, are skipped).  Bit-exact; enqueued on the current stream."""
    import torch
    _check(k_cache, "k_cache", torch.float16, ndim=4)
    NB, B, H, D = k_cache.shape
    _check(v_cache, "v_cache", torch.float16, shape=k_cache.shape)
    _check(key, "key", torch.float16, ndim=3)
    T = key.shape[0]
    _check(key, "key", torch.float16, shape=(T, H, D))
    _check(value, "value", torch.float16, shape=(T, H, D))
    _check(slot_mapping, "slot_mapping", torch.int64, shape=(T,))
    rc = load().pa_reshape_and_cache(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(slot_mapping), T, H, D, NB, B, _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_reshape_and_cache")


def decode_workspace_size(num_seqs, num_heads, head_dim, block_size, max_blocks_per_seq,
                          partition_size):
    return int(load().pa_decode_workspace_size(num_seqs, num_heads, head_dim, block_size,
                                               max_blocks_per_seq, partition_size))


def decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, partition_size=512,
           workspace=None, stream=None):
    """Paged-attention decode into out [S, H, D] fp16 (returned).

    q [S, H, D] fp16; k_cache/v_cache [NB, B, H, D] fp16; block_tables
    [S, MB] int32; context_lens [S] int32; partition_size 0 (no split) or a
    multiple of B.  workspace: uint8 GPU tensor of at least
    decode_workspace_size(...) bytes, allocated here if None."""
    import torch
    _check(k_cache, "k_cache", torch.float16, ndim=4)
    NB, B, H, D = k_cache.shape
    _check(v_cache, "v_cache", torch.float16, shape=k_cache.shape)
    _check(q, "q", torch.float16, ndim=3)
    S = q.shape[0]
    _check(q, "q", torch.float16, shape=(S, H, D))
    _check(out, "out", torch.float16, shape=(S, H, D))
    _check(block_tables, "block_tables", torch.int32, ndim=2)
    MB = block_tables.shape[1]
    _check(block_tables, "block_tables", torch.int32, shape=(S, MB))
    _check(context_lens, "context_lens", torch.int32, shape=(S,))
    need = decode_workspace_size(S, H, D, B, MB, partition_size)
    if workspace is None:
        workspace = _alloc_workspace(need, q.device, stream) if need else None
    elif need:
        _check(workspace, "workspace", torch.uint8, ndim=1)
    wbytes = workspace.numel() if workspace is not None else 0
    rc = load().pa_decode(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                          _ptr(context_lens), S, H, D, NB, B, MB, float(scale), int(partition_size),
                          _ptr(workspace), wbytes, _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_decode")
    return out


def decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                   partition_size=512, stream=None):
    """decode() that allocates nothing: the split partials go to the library's
    static per-GPU scratch (PA_NOALLOC_SCRATCH_BYTES, 32 MiB).  Calls that
    may overlap in time on one GPU (different streams, unordered) race on
    that scratch.  A split whose partials do not fit raises PAError
    (PA_ERR_SCRATCH)."""
    import torch
    _check(k_cache, "k_cache", torch.float16, ndim=4)
    NB, B, H, D = k_cache.shape
    _check(v_cache, "v_cache", torch.float16, shape=k_cache.shape)
    _check(q, "q", torch.float16, ndim=3)
    S = q.shape[0]
    _check(q, "q", torch.float16, shape=(S, H, D))
    _check(out, "out", torch.float16, shape=(S, H, D))
    _check(block_tables, "block_tables", torch.int32, ndim=2)
    MB = block_tables.shape[1]
    _check(block_tables, "block_tables", torch.int32, shape=(S, MB))
    _check(context_lens, "context_lens", torch.int32, shape=(S,))
    rc = load().pa_decode_noalloc(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(block_tables), _ptr(context_lens), S, H, D, NB, B, MB,
                                  float(scale), int(partition_size), _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_decode_noalloc")
    return out


def _check_new_tokens(key, value, slot_mapping, S, H, D):
    import torch
    _check(key, "key", torch.float16, shape=(S, H, D))
    _check(value, "value", torch.float16, shape=(S, H, D))
    _check(slot_mapping, "slot_mapping", torch.int64, shape=(S,))


def copy_blocks(k_cache, v_cache, block_mapping, stream=None):
    """Copy-on-write: for each (src, dst) row of block_mapping (int64 [N, 2] GPU
    tensor), block dst of k_cache and v_cache ([NB, B, H, D] fp16) becomes a
    bitwise copy of block src.  Enqueued on the current stream."""
    import torch
    _check(k_cache, "k_cache", torch.float16, ndim=4)
    NB, B, H, D = k_cache.shape
    _check(v_cache, "v_cache", torch.float16, shape=k_cache.shape)
    _check(block_mapping, "block_mapping", torch.int64, ndim=2)
    if block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [N, 2]")
    rc = load().pa_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(block_mapping),
                               block_mapping.shape[0], NB, B, H, D, _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_copy_blocks")


def swap_blocks(src, dst, block_mapping, stream=None):
    """Swap-out / swap-in: for each (a, b) row of block_mapping (int64 [N, 2]
    CPU tensor), block b of dst becomes a copy of block a of src.  src and dst
    are [NB, B, H, D] fp16 tensors with the same block shape, on the GPU or in
    host memory.  With pinned host memory the move is one asynchronous kernel
    on the current stream; pageable host memory falls back to copies that
    complete before the call returns."""
    import torch
    for t, n in ((src, "src"), (dst, "dst")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_contiguous() \
                or t.dim() != 4:
            raise ValueError(f"{n} must be a contiguous fp16 [NB, B, H, D] tensor")
    if tuple(src.shape[1:]) != tuple(dst.shape[1:]):
        raise ValueError("src and dst must have the same block shape")
    m = block_mapping
    if not isinstance(m, torch.Tensor) or m.is_cuda or m.dtype != torch.int64 or m.dim() != 2 \
            or m.shape[1] != 2:
        raise ValueError("block_mapping must be a CPU int64 [N, 2] tensor")
    m = m.contiguous()
    block_bytes = src[0].numel() * 2
    rc = load().pa_swap_blocks(_ptr(src), _ptr(dst), _ptr(m), m.shape[0], src.shape[0],
                               dst.shape[0], block_bytes, _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_swap_blocks")


def _check_fp8_cache(t, name, shape=None):
    import torch
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise ValueError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn)")
    _check(t, name, t.dtype, shape=shape, ndim=4)


def reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping, k_scale, v_scale,
                          stream=None):
    """reshape_and_cache into FP8 (OCP E4M3) caches [NB, B, H, D] of uint8 /
    float8_e4m3fn, quantising with code = E4M3(x * (1/scale))."""
    import torch
    _check_fp8_cache(k_cache, "k_cache")
    NB, B, H, D = k_cache.shape
    _check_fp8_cache(v_cache, "v_cache", shape=k_cache.shape)
    _check(key, "key", torch.float16, ndim=3)
    T = key.shape[0]
    _check(key, "key", torch.float16, shape=(T, H, D))
    _check(value, "value", torch.float16, shape=(T, H, D))
    _check(slot_mapping, "slot_mapping", torch.int64, shape=(T,))
    rc = load().pa_reshape_and_cache_fp8(_ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(slot_mapping), T, H, D, NB, B, float(k_scale),
                                         float(v_scale), _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_reshape_and_cache_fp8")


def decode_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale, k_scale, v_scale,
               partition_size=512, workspace=None, stream=None):
    """Paged-attention decode over FP8 caches (values = code * scale); the
    other arguments as decode()."""
    import torch
    _check_fp8_cache(k_cache, "k_cache")
    NB, B, H, D = k_cache.shape
    _check_fp8_cache(v_cache, "v_cache", shape=k_cache.shape)
    _check(q, "q", torch.float16, ndim=3)
    S = q.shape[0]
    _check(q, "q", torch.float16, shape=(S, H, D))
    _check(out, "out", torch.float16, shape=(S, H, D))
    _check(block_tables, "block_tables", torch.int32, ndim=2)
    MB = block_tables.shape[1]
    _check(block_tables, "block_tables", torch.int32, shape=(S, MB))
    _check(context_lens, "context_lens", torch.int32, shape=(S,))
    need = decode_workspace_size(S, H, D, B, MB, partition_size)
    if workspace is None:
        workspace = _alloc_workspace(need, q.device, stream) if need else None
    elif need:
        _check(workspace, "workspace", torch.uint8, ndim=1)
    wbytes = workspace.numel() if workspace is not None else 0
    rc = load().pa_decode_fp8(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                              _ptr(block_tables), _ptr(context_lens), S, H, D, NB, B, MB,
                              float(scale), float(k_scale), float(v_scale), int(partition_size),
                              _ptr(workspace), wbytes, _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_decode_fp8")
    return out


def decode_cascade_workspace_size(num_seqs, num_heads, head_dim, block_size, prefix_len,
                                  max_blocks_per_seq, partition_size):
    return int(load().pa_decode_cascade_workspace_size(num_seqs, num_heads, head_dim, block_size,
                                                       prefix_len, max_blocks_per_seq,
                                                       partition_size))


def decode_cascade(out, q, k_cache, v_cache, prefix_table, prefix_len, block_tables,
                   context_lens, scale, partition_size=512, workspace=None, stream=None):
    """Decode for sequences that all start with the same prefix: prefix_table
    (int32 [prefix_len / B] GPU tensor) lists the prefix's blocks,
    block_tables / context_lens the private suffixes.  Equals decode() over
    prefix_table ++ block_tables[s] with context prefix_len + context_lens[s]."""
    import torch
    _check(k_cache, "k_cache", torch.float16, ndim=4)
    NB, B, H, D = k_cache.shape
    _check(v_cache, "v_cache", torch.float16, shape=k_cache.shape)
    _check(q, "q", torch.float16, ndim=3)
    S = q.shape[0]
    _check(q, "q", torch.float16, shape=(S, H, D))
    _check(out, "out", torch.float16, shape=(S, H, D))
    _check(prefix_table, "prefix_table", torch.int32, ndim=1)
    if prefix_len % B or prefix_table.numel() * B < prefix_len:
        raise ValueError("prefix_len must be a multiple of the block size covered by prefix_table")
    _check(block_tables, "block_tables", torch.int32, ndim=2)
    MB = block_tables.shape[1]
    _check(block_tables, "block_tables", torch.int32, shape=(S, MB))
    _check(context_lens, "context_lens", torch.int32, shape=(S,))
    need = decode_cascade_workspace_size(S, H, D, B, int(prefix_len), MB, partition_size)
    if workspace is None:
        workspace = _alloc_workspace(max(need, 1), q.device, stream)
    else:
        _check(workspace, "workspace", torch.uint8, ndim=1)
    rc = load().pa_decode_cascade(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                  _ptr(prefix_table), int(prefix_len), _ptr(block_tables),
                                  _ptr(context_lens), S, H, D, NB, B, MB, float(scale),
                                  int(partition_size), _ptr(workspace), workspace.numel(),
                                  _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_decode_cascade")
    return out


def decode_cascade_fp8(out, q, k_cache, v_cache, prefix_table, prefix_len, block_tables,
                       context_lens, scale, k_scale, v_scale, partition_size=512, workspace=None,
                       stream=None):
    """decode_cascade() over FP8 caches (values = code * scale, as decode_fp8)."""
    import torch
    _check_fp8_cache(k_cache, "k_cache")
    NB, B, H, D = k_cache.shape
    _check_fp8_cache(v_cache, "v_cache", shape=k_cache.shape)
    _check(q, "q", torch.float16, ndim=3)
    S = q.shape[0]
    _check(q, "q", torch.float16, shape=(S, H, D))
    _check(out, "out", torch.float16, shape=(S, H, D))
    _check(prefix_table, "prefix_table", torch.int32, ndim=1)
    if prefix_len % B or prefix_table.numel() * B < prefix_len:
        raise ValueError("prefix_len must be a multiple of the block size covered by prefix_table")
    _check(block_tables, "block_tables", torch.int32, ndim=2)
    MB = block_tables.shape[1]
    _check(block_tables, "block_tables", torch.int32, shape=(S, MB))
    _check(context_lens, "context_lens", torch.int32, shape=(S,))
    need = decode_cascade_workspace_size(S, H, D, B, int(prefix_len), MB, partition_size)
    if workspace is None:
        workspace = _alloc_workspace(max(need, 1), q.device, stream)
    else:
        _check(workspace, "workspace", torch.uint8, ndim=1)
    rc = load().pa_decode_cascade_fp8(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                      _ptr(prefix_table), int(prefix_len), _ptr(block_tables),
                                      _ptr(context_lens), S, H, D, NB, B, MB, float(scale),
                                      float(k_scale), float(v_scale), int(partition_size),
                                      _ptr(workspace), workspace.numel(), _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_decode_cascade_fp8")
    return out


def decode_cascade_append_fp8(out, q, key, value, k_cache, v_cache, slot_mapping, prefix_table,
                              prefix_len, block_tables, context_lens, scale, k_scale, v_scale,
                              partition_size=512, workspace=None, stream=None):
    """decode_cascade_append() over FP8 caches: the new rows are quantised as
    reshape_and_cache_fp8 quantises them (values = code * scale)."""
    import torch
    _check_fp8_cache(k_cache, "k_cache")
    NB, B, H, D = k_cache.shape
    _check_fp8_cache(v_cache, "v_cache", shape=k_cache.shape)
    _check(q, "q", torch.float16, ndim=3)
    S = q.shape[0]
    _check(q, "q", torch.float16, shape=(S, H, D))
    _check(out, "out", torch.float16, shape=(S, H, D))
    _check_new_tokens(key, value, slot_mapping, S, H, D)
    _check(prefix_table, "prefix_table", torch.int32, ndim=1)
    if prefix_len % B or prefix_table.numel() * B < prefix_len:
        raise ValueError("prefix_len must be a multiple of the block size covered by prefix_table")
    _check(block_tables, "block_tables", torch.int32, ndim=2)
    MB = block_tables.shape[1]
    _check(block_tables, "block_tables", torch.int32, shape=(S, MB))
    _check(context_lens, "context_lens", torch.int32, shape=(S,))
    need = decode_cascade_workspace_size(S, H, D, B, int(prefix_len), MB, partition_size)
    if workspace is None:
        workspace = _alloc_workspace(max(need, 1), q.device, stream)
    else:
        _check(workspace, "workspace", torch.uint8, ndim=1)
    rc = load().pa_decode_cascade_append_fp8(
        _ptr(out), _ptr(q), _ptr(key), _ptr(value), _ptr(k_cache), _ptr(v_cache),
        _ptr(slot_mapping), _ptr(prefix_table), int(prefix_len), _ptr(block_tables),
        _ptr(context_lens), S, H, D, NB, B, MB, float(scale), float(k_scale), float(v_scale),
        int(partition_size), _ptr(workspace), workspace.numel(), _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_decode_cascade_append_fp8")
    return out


def decode_cascade_append(out, q, key, value, k_cache, v_cache, slot_mapping, prefix_table,
                          prefix_len, block_tables, context_lens, scale, partition_size=512,
                          workspace=None, stream=None):
    """reshape_and_cache(key, value, k_cache, v_cache, slot_mapping) followed by
    decode_cascade(...), in the launches of decode_cascade alone: row s of key
    / value [S, H, D] is sequence s's new token, slot_mapping [S] int64 its
    slot in a private suffix block (negative: not written)."""
    import torch
    _check(k_cache, "k_cache", torch.float16, ndim=4)
    NB, B, H, D = k_cache.shape
    _check(v_cache, "v_cache", torch.float16, shape=k_cache.shape)
    _check(q, "q", torch.float16, ndim=3)
    S = q.shape[0]
    _check(q, "q", torch.float16, shape=(S, H, D))
    _check(out, "out", torch.float16, shape=(S, H, D))
    _check_new_tokens(key, value, slot_mapping, S, H, D)
    _check(prefix_table, "prefix_table", torch.int32, ndim=1)
    if prefix_len % B or prefix_table.numel() * B < prefix_len:
        raise ValueError("prefix_len must be a multiple of the block size covered by prefix_table")
    _check(block_tables, "block_tables", torch.int32, ndim=2)
    MB = block_tables.shape[1]
    _check(block_tables, "block_tables", torch.int32, shape=(S, MB))
    _check(context_lens, "context_lens", torch.int32, shape=(S,))
    need = decode_cascade_workspace_size(S, H, D, B, int(prefix_len), MB, partition_size)
    if workspace is None:
        workspace = _alloc_workspace(max(need, 1), q.device, stream)
    else:
        _check(workspace, "workspace", torch.uint8, ndim=1)
    rc = load().pa_decode_cascade_append(_ptr(out), _ptr(q), _ptr(key), _ptr(value),
                                         _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping),
                                         _ptr(prefix_table), int(prefix_len), _ptr(block_tables),
                                         _ptr(context_lens), S, H, D, NB, B, MB, float(scale),
                                         int(partition_size), _ptr(workspace), workspace.numel(),
                                         _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_decode_cascade_append")
    return out


def multi_query(out, q, k_cache, v_cache, block_tables, context_lens, query_start, max_query_len,
                scale, stream=None):
    """Multi-query (chunked-prefill) paged attention: the rows
    query_start[s] .. query_start[s+1]-1 of q [T, H, D] are the last positions
    of sequence s and attend causally through its block table."""
    import torch
    _check(k_cache, "k_cache", torch.float16, ndim=4)
    NB, B, H, D = k_cache.shape
    _check(v_cache, "v_cache", torch.float16, shape=k_cache.shape)
    _check(q, "q", torch.float16, ndim=3)
    T = q.shape[0]
    _check(q, "q", torch.float16, shape=(T, H, D))
    _check(out, "out", torch.float16, shape=(T, H, D))
    _check(block_tables, "block_tables", torch.int32, ndim=2)
    S, MB = block_tables.shape
    _check(context_lens, "context_lens", torch.int32, shape=(S,))
    _check(query_start, "query_start", torch.int32, shape=(S + 1,))
    rc = load().pa_multi_query(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(block_tables), _ptr(context_lens), _ptr(query_start), S, T,
                               int(max_query_len), H, D, NB, B, MB, float(scale),
                               _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_multi_query")
    return out


def multi_query_fp8(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                    max_query_len, scale, k_scale, v_scale, stream=None):
    """multi_query() over FP8 caches (values = code * scale, as decode_fp8)."""
    import torch
    _check_fp8_cache(k_cache, "k_cache")
    NB, B, H, D = k_cache.shape
    _check_fp8_cache(v_cache, "v_cache", shape=k_cache.shape)
    _check(q, "q", torch.float16, ndim=3)
    T = q.shape[0]
    _check(q, "q", torch.float16, shape=(T, H, D))
    _check(out, "out", torch.float16, shape=(T, H, D))
    _check(block_tables, "block_tables", torch.int32, ndim=2)
    S, MB = block_tables.shape
    _check(context_lens, "context_lens", torch.int32, shape=(S,))
    _check(query_start, "query_start", torch.int32, shape=(S + 1,))
    rc = load().pa_multi_query_fp8(_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(block_tables), _ptr(context_lens), _ptr(query_start), S,
                                   T, int(max_query_len), H, D, NB, B, MB, float(scale),
                                   float(k_scale), float(v_scale), _stream_ptr(stream))
    if rc != PA_OK:
        raise PAError(rc, "pa_multi_query_fp8")
    return out
