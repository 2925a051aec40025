"""Python binding of the gfx950 chunked LZSS coder (``libgpulz.so``).

Argument marshalling only: every step of encode and decode runs in the HIP
kernels behind the C ABI declared in ``include/gpulz.h``.  PyTorch supplies
device memory and the current HIP stream.  If the shared library has not been
built, every call raises; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# GPULZ_LIB names another build of the same library (the host-sanitizer test
# loads one built with ASan/UBSan on its host code); default: the in-tree build.
LIB_PATH = os.environ.get("GPULZ_LIB") or os.path.join(_HERE, "libgpulz.so")

OK, ERR_INVALID_ARG, ERR_CAPACITY, ERR_CORRUPT, ERR_HIP = 0, -1, -2, -3, -4
STATUS_OK, STATUS_CAPACITY, STATUS_CORRUPT = 0, 2, 3
SYMBOLS = ("gpulz_max_compressed_size", "gpulz_encode_workspace_size", "gpulz_decode_workspace_size",
           "gpulz_encode", "gpulz_decode", "gpulz_stream_info", "gpulz_encode_timed", "gpulz_decode_timed",
           "gpulz_split_bounds", "gpulz_encode_split_workspace_size", "gpulz_encode_split",
           "gpulz_decode_split_workspace_size", "gpulz_decode_split", "gpulz_decode_one_thread_per_chunk",
           "gpulz_lorenzo_quant", "gpulz_encode_window", "gpulz_encode_advancing_search", "gpulz_split_info",
           "gpulz_decode_noalloc")

_lib = None


class GpulzError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libgpulz.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    try:  # bind to the HIP runtime torch already uses (same soname), never a second one
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise GpulzError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    u64, u32, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p
    L.gpulz_max_compressed_size.argtypes = [u64, u32]
    L.gpulz_max_compressed_size.restype = u64
    L.gpulz_encode_workspace_size.argtypes = [u64, u32]
    L.gpulz_encode_workspace_size.restype = u64
    L.gpulz_decode_workspace_size.argtypes = [u64]
    L.gpulz_decode_workspace_size.restype = u64
    L.gpulz_encode.argtypes = [vp, u64, u32, u32, u32, vp, u64, vp, vp, u64, vp]
    L.gpulz_encode.restype = ctypes.c_int
    L.gpulz_decode.argtypes = [vp, u64, vp, u64, vp, vp, vp, u64, vp]
    L.gpulz_decode.restype = ctypes.c_int
    L.gpulz_stream_info.argtypes = [vp, u64, ctypes.POINTER(u64), ctypes.POINTER(u64), ctypes.POINTER(u32),
                                    ctypes.POINTER(u32)]
    L.gpulz_stream_info.restype = ctypes.c_int
    L.gpulz_encode_timed.argtypes = L.gpulz_encode.argtypes + [vp, vp]
    L.gpulz_encode_timed.restype = ctypes.c_int
    L.gpulz_decode_timed.argtypes = L.gpulz_decode.argtypes + [vp, vp]
    L.gpulz_decode_timed.restype = ctypes.c_int
    L.gpulz_split_bounds.argtypes = [u64, u32, u32, ctypes.POINTER(u64), ctypes.POINTER(u64), ctypes.POINTER(u64)]
    L.gpulz_split_bounds.restype = ctypes.c_int
    L.gpulz_encode_split_workspace_size.argtypes = [u64, u32]
    L.gpulz_encode_split_workspace_size.restype = u64
    L.gpulz_encode_split.argtypes = [vp, u64, u32, u32, u32, vp, u64, vp, vp, u64, vp, u64, vp, vp, u64, vp]
    L.gpulz_encode_split.restype = ctypes.c_int
    L.gpulz_decode_split_workspace_size.argtypes = [u64]
    L.gpulz_decode_split_workspace_size.restype = u64
    L.gpulz_decode_split.argtypes = [vp, u64, vp, vp, u64, vp, u64, vp, u64, vp, vp, vp, u64, vp]
    L.gpulz_decode_split.restype = ctypes.c_int
    L.gpulz_decode_one_thread_per_chunk.argtypes = L.gpulz_decode.argtypes + [vp, vp]
    L.gpulz_decode_one_thread_per_chunk.restype = ctypes.c_int
    L.gpulz_encode_window.argtypes = [vp, u64, u32, u32, u32, u32, vp, u64, vp, vp, u64, vp]
    L.gpulz_encode_advancing_search.argtypes = [vp, u64, u32, u32, vp, u64, vp, vp, u64, vp, vp, vp]
    L.gpulz_encode_advancing_search.restype = ctypes.c_int
    L.gpulz_encode_window.restype = ctypes.c_int
    L.gpulz_lorenzo_quant.argtypes = [vp, u32, u32, u32, ctypes.c_double, vp, vp, vp]
    L.gpulz_lorenzo_quant.restype = ctypes.c_int
    L.gpulz_split_info.argtypes = L.gpulz_stream_info.argtypes
    L.gpulz_split_info.restype = ctypes.c_int
    L.gpulz_decode_noalloc.argtypes = [vp, u64, vp, u64, vp, vp, vp]
    L.gpulz_decode_noalloc.restype = ctypes.c_int
    _lib = L
    return L


def _check(rc: int, what: str) -> None:
    if rc != OK:
        raise GpulzError(f"{what} returned {rc}")


def max_compressed_size(n_bytes: int, chunk_size: int) -> int:
    return int(lib().gpulz_max_compressed_size(n_bytes, chunk_size))


def encode_workspace_size(n_bytes: int, chunk_size: int) -> int:
    return int(lib().gpulz_encode_workspace_size(n_bytes, chunk_size))


def decode_workspace_size(in_bytes: int) -> int:
    return int(lib().gpulz_decode_workspace_size(in_bytes))


def _ptr(t) -> int | None:
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _torch_stream(stream):
    import torch
    return stream if stream is not None else torch.cuda.current_stream()


def _stream(stream):
    return ctypes.c_void_p(_torch_stream(stream).cuda_stream)


def _on(stream):
    """Context in which torch allocates and copies on the call's stream, so
    workspaces and temporaries belong to the stream the kernels run on (the
    caching allocator then never hands them to other work while the kernels
    still use them)."""
    import torch
    return torch.cuda.stream(_torch_stream(stream))


def _u8_view(t):
    import torch
    if not t.is_cuda:
        raise GpulzError("input must be a CUDA (HIP) tensor")
    t = t.contiguous()
    return t.view(torch.uint8).reshape(-1) if t.dtype != torch.uint8 else t.reshape(-1)


def encode_into(d_in, chunk_size: int, word_size: int, match_level: int, out, out_bytes, workspace,
                stream=None, events=None) -> None:
    """Enqueue gpulz_encode with caller-provided buffers (no allocation).
    events: optional (start, stop) raw hipEvent_t handles, recorded around the
    chunk encode kernel (gpulz_encode_timed)."""
    with _on(stream):
        src = _u8_view(d_in)
        args = (_ptr(src), src.numel(), chunk_size, word_size, match_level, _ptr(out), out.numel(),
                _ptr(out_bytes), _ptr(workspace), workspace.numel(), _stream(stream))
        if events is None:
            _check(lib().gpulz_encode(*args), "gpulz_encode")
        else:
            _check(lib().gpulz_encode_timed(*args, events[0], events[1]), "gpulz_encode_timed")


def encode_window_into(d_in, chunk_size: int, word_size: int, match_level: int, window: int, out, out_bytes,
                       workspace, stream=None) -> None:
    """Enqueue gpulz_encode_window (gpulz_window.h): encode_into with a near
    window of 32, 48 or 64 offsets."""
    with _on(stream):
        src = _u8_view(d_in)
        _check(lib().gpulz_encode_window(_ptr(src), src.numel(), chunk_size, word_size, match_level, window, _ptr(out),
                                         out.numel(), _ptr(out_bytes), _ptr(workspace), workspace.numel(),
                                         _stream(stream)), "gpulz_encode_window")


def encode_advancing_into(d_in, chunk_size: int, word_size: int, out, out_bytes, workspace, stream=None,
                          events=None) -> None:
    """Enqueue gpulz_encode_advancing_search (gpulz_baseline.h): the level-0
    stream with the upstream-style advancing-window search, same buffers as
    encode_into."""
    with _on(stream):
        src = _u8_view(d_in)
        ev = events if events is not None else (None, None)
        _check(lib().gpulz_encode_advancing_search(_ptr(src), src.numel(), chunk_size, word_size, _ptr(out),
                                                   out.numel(), _ptr(out_bytes), _ptr(workspace), workspace.numel(),
                                                   _stream(stream), ev[0], ev[1]), "gpulz_encode_advancing_search")


def encode(d_in, chunk_size: int = 2048, word_size: int = 4, match_level: int = 0, stream=None):
    """Encode a CUDA tensor (any dtype, its bytes are coded).

    Returns (stream_buffer uint8 tensor of the worst-case size, out_bytes
    uint64 tensor on the device).  The stream is the first out_bytes bytes."""
    with _on(stream):
        import torch
        src = _u8_view(d_in)
        cap = max_compressed_size(src.numel(), chunk_size)
        if cap == 0:
            raise GpulzError(f"unsupported chunk_size {chunk_size}")
        dev = src.device
        out = torch.empty(cap, dtype=torch.uint8, device=dev)
        out_bytes = torch.zeros(1, dtype=torch.uint64, device=dev)
        ws = torch.empty(max(encode_workspace_size(src.numel(), chunk_size), 1), dtype=torch.uint8, device=dev)
        encode_into(src, chunk_size, word_size, match_level, out, out_bytes, ws, stream)
        return out, out_bytes


def decode_into(d_stream, in_bytes: int, out, out_bytes, status, workspace, stream=None, events=None) -> None:
    """Enqueue gpulz_decode with caller-provided buffers (no allocation).
    events: optional (start, stop) raw hipEvent_t handles, recorded around the
    chunk decode kernel (gpulz_decode_timed)."""
    with _on(stream):
        s = _u8_view(d_stream)
        if in_bytes > s.numel():
            raise GpulzError("in_bytes exceeds the stream buffer")
        args = (_ptr(s), in_bytes, _ptr(out), out.numel(), _ptr(out_bytes), _ptr(status), _ptr(workspace),
                workspace.numel(), _stream(stream))
        if events is None:
            _check(lib().gpulz_decode(*args), "gpulz_decode")
        else:
            _check(lib().gpulz_decode_timed(*args, events[0], events[1]), "gpulz_decode_timed")


DECODE_NOALLOC_MAX_CHUNKS = 1 << 22


def decode_noalloc_into(d_stream, in_bytes: int, out, out_bytes, status, stream=None) -> None:
    """Enqueue gpulz_decode_noalloc: decode_into without a workspace (the
    library's static device array serves as one; calls whose work overlaps on
    one GPU race).  Raises GpulzError if the call's chunk bound exceeds
    DECODE_NOALLOC_MAX_CHUNKS."""
    with _on(stream):
        s = _u8_view(d_stream)
        if in_bytes > s.numel():
            raise GpulzError("in_bytes exceeds the stream buffer")
        _check(lib().gpulz_decode_noalloc(_ptr(s), in_bytes, _ptr(out), out.numel(), _ptr(out_bytes), _ptr(status),
                                          _stream(stream)), "gpulz_decode_noalloc")


def decode_one_thread_per_chunk_into(d_stream, in_bytes: int, out, out_bytes, status, workspace, stream=None,
                                     events=None) -> None:
    """The one-thread-per-chunk baseline decoder (gpulz_baseline.h), same
    buffers as decode_into."""
    with _on(stream):
        s = _u8_view(d_stream)
        if in_bytes > s.numel():
            raise GpulzError("in_bytes exceeds the stream buffer")
        ev = events if events is not None else (None, None)
        _check(lib().gpulz_decode_one_thread_per_chunk(_ptr(s), in_bytes, _ptr(out), out.numel(), _ptr(out_bytes),
                                                       _ptr(status), _ptr(workspace), workspace.numel(),
                                                       _stream(stream), ev[0], ev[1]),
               "gpulz_decode_one_thread_per_chunk")


def decode(d_stream, in_bytes: int | None = None, out_capacity: int | None = None, stream=None):
    """Decode a stream held in a CUDA uint8 tensor.

    out_capacity: bytes to allocate for the output; if None the 32-byte
    header is copied to the host once to size it.  Returns (out uint8 tensor,
    out_bytes uint64 device tensor, status uint32 device tensor)."""
    with _on(stream):
        import torch
        s = _u8_view(d_stream)
        in_bytes = s.numel() if in_bytes is None else in_bytes
        if out_capacity is None:
            info = stream_info(s[:32].cpu().numpy().tobytes())
            if info is None:
                raise GpulzError("not a gpulz stream")
            out_capacity = info[0]
        dev = s.device
        out = torch.empty(max(out_capacity, 1), dtype=torch.uint8, device=dev)[:out_capacity]
        out_bytes = torch.zeros(1, dtype=torch.uint64, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        ws = torch.empty(max(decode_workspace_size(in_bytes), 1), dtype=torch.uint8, device=dev)
        decode_into(s, in_bytes, out, out_bytes, status, ws, stream)
        return out, out_bytes, status


def stream_info(prefix: bytes):
    """(original_size, stream_bytes, chunk_size, word_size) from a host copy of
    the first 32+ bytes, or None if they are not a valid header."""
    buf = ctypes.create_string_buffer(bytes(prefix), len(prefix))
    n, t = ctypes.c_uint64(), ctypes.c_uint64()
    cs, ws = ctypes.c_uint32(), ctypes.c_uint32()
    rc = lib().gpulz_stream_info(ctypes.cast(buf, ctypes.c_void_p), len(prefix), ctypes.byref(n), ctypes.byref(t),
                                 ctypes.byref(cs), ctypes.byref(ws))
    if rc != OK:
        return None
    return n.value, t.value, cs.value, ws.value


# ---- split mode: literals / lengths / offsets / meta ports ----------------

def split_info(prefix: bytes):
    """(original_size, meta_bytes, chunk_size, word_size) from a host copy of
    the first 32+ bytes of a meta port, or None if they are not a valid
    split-mode header."""
    buf = ctypes.create_string_buffer(bytes(prefix), len(prefix))
    n, m = ctypes.c_uint64(), ctypes.c_uint64()
    cs, ws = ctypes.c_uint32(), ctypes.c_uint32()
    rc = lib().gpulz_split_info(ctypes.cast(buf, ctypes.c_void_p), len(prefix), ctypes.byref(n), ctypes.byref(m),
                                ctypes.byref(cs), ctypes.byref(ws))
    if rc != OK:
        return None
    return n.value, m.value, cs.value, ws.value


def split_bounds(n_bytes: int, chunk_size: int, word_size: int) -> tuple[int, int, int]:
    """Port capacities that always suffice: (literals, lengths = offsets, meta)."""
    a, b, c = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    _check(lib().gpulz_split_bounds(n_bytes, chunk_size, word_size, ctypes.byref(a), ctypes.byref(b),
                                    ctypes.byref(c)), "gpulz_split_bounds")
    return a.value, b.value, c.value


def encode_split_workspace_size(n_bytes: int, chunk_size: int) -> int:
    return int(lib().gpulz_encode_split_workspace_size(n_bytes, chunk_size))


def decode_split_workspace_size(meta_bytes: int) -> int:
    return int(lib().gpulz_decode_split_workspace_size(meta_bytes))


def encode_split_into(d_in, chunk_size: int, word_size: int, match_level: int, lit, lens, offs, meta, port_bytes,
                      workspace, stream=None) -> None:
    """Enqueue gpulz_encode_split with caller-provided buffers (no allocation).
    lens and offs must have the same size; port_bytes is a device uint64[4]."""
    with _on(stream):
        src = _u8_view(d_in)
        if lens.numel() != offs.numel():
            raise GpulzError("lengths and offsets buffers differ in size")
        _check(lib().gpulz_encode_split(_ptr(src), src.numel(), chunk_size, word_size, match_level, _ptr(lit),
                                        lit.numel(), _ptr(lens), _ptr(offs), lens.numel(), _ptr(meta), meta.numel(),
                                        _ptr(port_bytes), _ptr(workspace), workspace.numel(), _stream(stream)),
               "gpulz_encode_split")


def encode_split(d_in, chunk_size: int = 2048, word_size: int = 4, match_level: int = 0, stream=None):
    """Encode into four ports.  Returns (literals, lengths, offsets, meta)
    uint8 tensors of the worst-case sizes and port_bytes, a device uint64[4]
    with the bytes used in each."""
    with _on(stream):
        import torch
        src = _u8_view(d_in)
        bl, bt, bm = split_bounds(src.numel(), chunk_size, word_size)
        dev = src.device
        lit = torch.empty(max(bl, 1), dtype=torch.uint8, device=dev)
        lens = torch.empty(max(bt, 1), dtype=torch.uint8, device=dev)
        offs = torch.empty(max(bt, 1), dtype=torch.uint8, device=dev)
        meta = torch.empty(max(bm, 1), dtype=torch.uint8, device=dev)
        pbytes = torch.zeros(4, dtype=torch.uint64, device=dev)
        ws = torch.empty(max(encode_split_workspace_size(src.numel(), chunk_size), 1), dtype=torch.uint8, device=dev)
        encode_split_into(src, chunk_size, word_size, match_level, lit, lens, offs, meta, pbytes, ws, stream)
        return lit, lens, offs, meta, pbytes


def decode_split_into(lit, lit_bytes: int, lens, offs, tok_bytes: int, meta, meta_bytes: int, out, out_bytes,
                      status, workspace, stream=None) -> None:
    """Enqueue gpulz_decode_split with caller-provided buffers (no allocation)."""
    with _on(stream):
        if lit_bytes > lit.numel() or tok_bytes > min(lens.numel(), offs.numel()) or meta_bytes > meta.numel():
            raise GpulzError("port byte counts exceed the port buffers")
        _check(lib().gpulz_decode_split(_ptr(lit), lit_bytes, _ptr(lens), _ptr(offs), tok_bytes, _ptr(meta), meta_bytes,
                                        _ptr(out), out.numel(), _ptr(out_bytes), _ptr(status), _ptr(workspace),
                                        workspace.numel(), _stream(stream)), "gpulz_decode_split")


def decode_split(lit, lens, offs, meta, port_bytes=None, out_capacity: int | None = None, stream=None):
    """Decode four ports held in CUDA uint8 tensors.  port_bytes: the
    (literals, tokens, meta) byte counts, or a uint64[4] tensor from
    encode_split, or None for the whole tensors.  out_capacity: if None the
    header is copied to the host once to size the output.  Returns (out,
    out_bytes, status) like decode."""
    with _on(stream):
        import torch
        if port_bytes is None:
            nl, nt, nm = lit.numel(), lens.numel(), meta.numel()
        elif hasattr(port_bytes, "cpu"):
            v = [int(x) for x in port_bytes.cpu().tolist()]
            nl, nt, nm = v[0], v[1], v[3]
        else:
            nl, nt, nm = port_bytes
        if out_capacity is None:
            info = split_info(meta[:32].cpu().numpy().tobytes())
            if info is None:
                raise GpulzError("not a split-mode meta port")
            out_capacity = info[0]
        dev = meta.device
        out = torch.empty(max(out_capacity, 1), dtype=torch.uint8, device=dev)[:out_capacity]
        out_bytes = torch.zeros(1, dtype=torch.uint64, device=dev)
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        ws = torch.empty(max(decode_split_workspace_size(nm), 1), dtype=torch.uint8, device=dev)
        decode_split_into(lit, nl, lens, offs, nt, meta, nm, out, out_bytes, status, ws, stream)
        return out, out_bytes, status


def lorenzo_quant_into(d_field, eb: float, codes, clamped, stream=None) -> None:
    """Enqueue gpulz_lorenzo_quant (gpulz_lorenzo.h): a float32 CUDA tensor of
    1, 2 or 3 dimensions (last one fastest) and an absolute error bound ->
    u32 codes in `codes` (int32 or uint32 tensor, same number of cells) and
    the clamped-cell count in `clamped` (one 64-bit integer)."""
    with _on(stream):
        import torch
        if not d_field.is_cuda or d_field.dtype != torch.float32 or d_field.dim() not in (1, 2, 3):
            raise GpulzError("field must be a 1-D, 2-D or 3-D float32 CUDA tensor")
        f = d_field.contiguous()
        dims = (1,) * (3 - f.dim()) + tuple(f.shape)  # (nz, ny, nx)
        if codes.numel() != f.numel() or codes.element_size() != 4 or clamped.element_size() != 8:
            raise GpulzError("codes must hold one 4-byte code per cell, clamped one 8-byte count")
        _check(lib().gpulz_lorenzo_quant(_ptr(f), dims[2], dims[1], dims[0], float(eb), _ptr(codes), _ptr(clamped),
                                         _stream(stream)), "gpulz_lorenzo_quant")


def lorenzo_quant(d_field, eb: float, stream=None):
    """Lorenzo-quantize a float32 CUDA tensor; returns (codes as a uint32
    tensor of the field's shape, clamped count as a one-element int64
    tensor), both on the device."""
    with _on(stream):
        import torch
        codes = torch.empty(d_field.shape, dtype=torch.uint32, device=d_field.device)
        clamped = torch.zeros(1, dtype=torch.int64, device=d_field.device)
        lorenzo_quant_into(d_field, eb, codes, clamped, stream)
        return codes, clamped
