"""Python binding of libmrr, the MI355X N-rank allreduce reduction library.

Argument marshalling only: every function forwards to the C entry point of the
same name in ``libmrr.so`` (declared in ``include/mrr.h``) and returns its
``mrr_status`` as an int.  Buffers may be torch tensors (their ``data_ptr()``
is passed) or raw device addresses (ints).  ``stream=None`` means torch's
current HIP stream on the current device.

The library must have been built (``__graft_entry__.build()`` or
``python allreduce_reduction_nranks_amd/build.py``); without it every call
raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmrr.so")

# mrr_status
MRR_OK, MRR_EINVAL, MRR_EUNSUPPORTED, MRR_EALIGN, MRR_EOVERLAP, MRR_ESCRATCH, \
    MRR_ETIMEDOUT, MRR_EHIP = range(8)
STATUS_NAMES = ["MRR_OK", "MRR_EINVAL", "MRR_EUNSUPPORTED", "MRR_EALIGN", "MRR_EOVERLAP",
                "MRR_ESCRATCH", "MRR_ETIMEDOUT", "MRR_EHIP"]
# mrr_dtype
MRR_AUTO, MRR_F32, MRR_F16, MRR_BF16, MRR_FP8_E4M3B15, MRR_FP8_E4M3FN = range(6)
DTYPES = {"auto": MRR_AUTO, "f32": MRR_F32, "f16": MRR_F16, "bf16": MRR_BF16,
          "fp8": MRR_FP8_E4M3B15, "fp8_e4m3b15": MRR_FP8_E4M3B15,
          "fp8fn": MRR_FP8_E4M3FN, "fp8_e4m3fn": MRR_FP8_E4M3FN}
MAX_RANKS = 32
PKT_FLAG_SLOTS = 1024
MRR_NOALLOC_SCRATCH_BYTES = 32 << 20  # packet scratch of mrr_allreduce_packet_noalloc


class MrrError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        name = STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else str(status)
        super().__init__("%s%s" % (name, (": " + what) if what else ""))


_lock = threading.Lock()
_lib = None


def load_library() -> ctypes.CDLL:
    """Loads libmrr.so (once).  Raises if it has not been built."""
    global _lib
    lib = _lib
    if lib is not None:  # loaded: no lock on the per-call path
        return lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmrr.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i, u32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint32
        pp = ctypes.POINTER(vp)
        sigs = {
            "mrr_allreduce_rsag": ([pp, pp, sz, i, i, vp], i),
            "mrr_allreduce_rsag_ex": ([pp, pp, sz, i, i, i, i, i, vp], i),
            "mrr_allreduce_rsag_dual": ([pp, pp, pp, sz, i, i, i, i, vp], i),
            "mrr_packet_scratch_bytes": ([sz, i, i], sz),
            "mrr_packet_flag_bytes": ([i], sz),
            "mrr_allreduce_packet": ([pp, pp, vp, sz, vp, sz, i, i, i, u32, vp, vp], i),
            "mrr_allreduce_packet_ex": ([pp, pp, vp, sz, vp, sz, i, i, i, u32, vp, i, i, vp], i),
            "mrr_allreduce_packet_noalloc": ([pp, pp, sz, i, i, i, u32, vp, vp], i),
            "mrr_packet_reduce": ([pp, vp, sz, i, i, i, u32, u32, u32, vp, vp], i),
            "mrr_allreduce": ([pp, pp, sz, i, i, i, vp, sz, vp, sz, u32, vp, vp], i),
            "mrr_packet_rsag_scratch_bytes": ([sz, i, i], sz),
            "mrr_allreduce_packet_rsag": ([pp, pp, vp, sz, vp, sz, i, i, i, u32, vp, i, i, vp], i),
            "mrr_fullmesh_scratch_bytes": ([sz, i, i], sz),
            "mrr_allreduce_fullmesh": ([pp, pp, vp, sz, vp, sz, i, i, i, u32, vp, i, i, vp], i),
            "mrr_pack": ([vp, vp, sz, u32, vp], i),
            "mrr_unpack": ([vp, vp, sz, vp], i),
            "mrr_fp8b15_to_f16": ([vp, vp, sz, vp], i),
            "mrr_fp8b15_to_f32": ([vp, vp, sz, vp], i),
            "mrr_f16_to_fp8b15": ([vp, vp, sz, vp], i),
            "mrr_f32_to_fp8b15": ([vp, vp, sz, vp], i),
            "mrr_stream_copy": ([vp, vp, sz, vp], i),
            "mrr_rank_buffer_pitch": ([sz, i], sz),
            "mrr_status_string": ([i], ctypes.c_char_p),
            "mrr_version": ([], i),
            "mrr_reload_env": ([], None),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
        return _lib


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _ptrs(xs):
    if xs is None:
        return None  # the C ABI refuses a null array with MRR_EINVAL
    return (ctypes.c_void_p * len(xs))(*[_ptr(x) for x in xs])


def _dt(d) -> int:
    v = DTYPES.get(d) if type(d) is str else None
    if v is not None:
        return v
    if isinstance(d, int):
        return d
    if isinstance(d, str):
        raise KeyError("unknown type name %r" % d)
    import torch
    return {torch.float32: MRR_F32, torch.float16: MRR_F16, torch.bfloat16: MRR_BF16,
            torch.uint8: MRR_FP8_E4M3B15}[d]


_ESIZE = {MRR_F32: 4, MRR_F16: 2, MRR_BF16: 2, MRR_FP8_E4M3B15: 1, MRR_FP8_E4M3FN: 1}


def _nbytes(count, dtype) -> int:
    """Bytes of `count` elements of dtype (0 for AUTO or an unknown id, which
    the C ABI refuses on its own)."""
    return (count if count > 0 else 0) * _ESIZE.get(_dt(dtype), 0)


def _room(x, nbytes: int, what: str) -> None:
    """A tensor argument must hold at least nbytes bytes.  Raw addresses
    (ints) and None pass unchecked: the C ABI validates what it can see."""
    if x is None or isinstance(x, int):
        return
    if x.nbytes < nbytes:
        raise ValueError("%s holds %d bytes, the call needs %d" % (what, x.nbytes, nbytes))


def _rank_ptrs(xs, nranks: int, nbytes: int, what: str):
    """Host array of device pointers for a per-rank argument.  The C ABI reads
    `nranks` entries, so a shorter list is refused here rather than letting it
    read past the array; tensor entries must hold nbytes bytes each."""
    if xs is None:
        return None
    if nranks > 0 and len(xs) < nranks:
        raise ValueError("%s has %d entries, nranks is %d" % (what, len(xs), nranks))
    ptrs = []
    for x in xs:
        if x is None or type(x) is int:
            ptrs.append(x or 0)
        else:
            if x.nbytes < nbytes and len(ptrs) < nranks:
                _room(x, nbytes, "%s[%d]" % (what, len(ptrs)))
            ptrs.append(x.data_ptr())
    return (_VP * len(ptrs))(*ptrs)


_VP = ctypes.c_void_p


_raw_stream = None


def _stream(stream) -> int:
    """HIP stream handle: torch's current stream on the current device when
    stream is None.  torch's raw-handle getter is used when it exists: it
    returns the same handle as torch.cuda.current_stream().cuda_stream without
    building a Stream object (measured on MI355X: 0.07 us against 2.96 us,
    a third of an eager call's host cost)."""
    global _raw_stream
    if stream is None:
        if _raw_stream is None:
            import torch
            getter = getattr(torch._C, "_cuda_getCurrentRawStream", None)
            device = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device
            _raw_stream = (lambda: getter(device())) if getter else \
                (lambda: int(torch.cuda.current_stream().cuda_stream))
        return _raw_stream()
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def check(status: int, what: str = "") -> None:
    """Raises MrrError for a non-OK status."""
    if status != MRR_OK:
        raise MrrError(status, what)


def mrr_status_string(status: int) -> str:
    return load_library().mrr_status_string(status).decode()


def mrr_version() -> int:
    return load_library().mrr_version()


def mrr_reload_env() -> None:
    """Makes the library read its MRR_* environment overrides again."""
    load_library().mrr_reload_env()


def mrr_rank_buffer_pitch(bytes_per_rank: int, nranks: int) -> int:
    return load_library().mrr_rank_buffer_pitch(bytes_per_rank, nranks)


def alloc_rank_buffers(nranks: int, count: int, dtype, device=None):
    """N rank buffers of `count` elements carved from one device allocation
    at mrr_rank_buffer_pitch() spacing.  Returns (pool, [views])."""
    import torch
    tdt = dtype if isinstance(dtype, torch.dtype) else \
        {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
         "fp8": torch.uint8, "fp8_e4m3b15": torch.uint8, "fp8fn": torch.uint8,
         "fp8_e4m3fn": torch.uint8}[dtype]
    esize = torch.empty((), dtype=tdt).element_size()
    nbytes = count * esize
    pitch = mrr_rank_buffer_pitch(nbytes, nranks)
    pool = torch.empty(max(1, nranks * pitch), dtype=torch.uint8,
                       device=device if device is not None else "cuda")
    views = [pool[r * pitch: r * pitch + nbytes].view(tdt) for r in range(nranks)]
    return pool, views


def mrr_allreduce_rsag(inputs, outputs, count, dtype, nranks, stream=None) -> int:
    nb = _nbytes(count, dtype)
    return load_library().mrr_allreduce_rsag(_rank_ptrs(inputs, nranks, nb, "inputs"),
                                             _rank_ptrs(outputs, nranks, nb, "outputs"), count,
                                             _dt(dtype), nranks, _stream(stream))


def mrr_allreduce_rsag_ex(inputs, outputs, count, dtype_in, accum, dtype_out, nranks, rank=-1,
                          stream=None) -> int:
    tout = dtype_in if _dt(dtype_out) == MRR_AUTO else dtype_out
    return load_library().mrr_allreduce_rsag_ex(
        _rank_ptrs(inputs, nranks, _nbytes(count, dtype_in), "inputs"),
        _rank_ptrs(outputs, nranks, _nbytes(count, tout), "outputs"), count, _dt(dtype_in),
        _dt(accum), _dt(dtype_out), nranks, rank, _stream(stream))


def mrr_allreduce_rsag_dual(inputs, outputs, outputs2, count, dtype_in, accum, nranks, rank=-1,
                            stream=None) -> int:
    nb = _nbytes(count, dtype_in)
    return load_library().mrr_allreduce_rsag_dual(
        _rank_ptrs(inputs, nranks, nb, "inputs"),
        _rank_ptrs(outputs, nranks, _nbytes(count, MRR_F16), "outputs"),
        _rank_ptrs(outputs2, nranks, nb, "outputs2"), count, _dt(dtype_in), _dt(accum), nranks,
        rank, _stream(stream))


def mrr_packet_scratch_bytes(count, dtype, nranks) -> int:
    return load_library().mrr_packet_scratch_bytes(count, _dt(dtype), nranks)


def mrr_packet_flag_bytes(nranks) -> int:
    return load_library().mrr_packet_flag_bytes(nranks)


def mrr_allreduce_packet(inputs, outputs, scratch, scratch_bytes, flags, count, dtype, accum,
                         nranks, max_spins, dev_err=None, stream=None) -> int:
    nb = _nbytes(count, dtype)
    _room(scratch, scratch_bytes, "scratch")
    _room(flags, 4 * PKT_FLAG_SLOTS * max(0, nranks), "flags")
    return load_library().mrr_allreduce_packet(
        _rank_ptrs(inputs, nranks, nb, "inputs"), _rank_ptrs(outputs, nranks, nb, "outputs"),
        _ptr(scratch), scratch_bytes, _ptr(flags), count, _dt(dtype), _dt(accum), nranks,
        max_spins, _ptr(dev_err), _stream(stream))


def mrr_allreduce_packet_ex(inputs, outputs, scratch, scratch_bytes, flags, count, dtype, accum,
                            nranks, max_spins, dev_err=None, blocks_per_rank=0, threads=0,
                            stream=None) -> int:
    nb = _nbytes(count, dtype)
    _room(scratch, scratch_bytes, "scratch")
    _room(flags, 4 * PKT_FLAG_SLOTS * max(0, nranks), "flags")
    return load_library().mrr_allreduce_packet_ex(
        _rank_ptrs(inputs, nranks, nb, "inputs"), _rank_ptrs(outputs, nranks, nb, "outputs"),
        _ptr(scratch), scratch_bytes, _ptr(flags), count, _dt(dtype), _dt(accum), nranks,
        max_spins, _ptr(dev_err), blocks_per_rank, threads, _stream(stream))


def mrr_allreduce_packet_noalloc(inputs, outputs, count, dtype, accum, nranks, max_spins,
                                 dev_err=None, stream=None) -> int:
    nb = _nbytes(count, dtype)
    return load_library().mrr_allreduce_packet_noalloc(
        _rank_ptrs(inputs, nranks, nb, "inputs"), _rank_ptrs(outputs, nranks, nb, "outputs"),
        count, _dt(dtype), _dt(accum), nranks, max_spins, _ptr(dev_err), _stream(stream))


def mrr_packet_rsag_scratch_bytes(count, dtype, nranks) -> int:
    return load_library().mrr_packet_rsag_scratch_bytes(count, _dt(dtype), nranks)


def mrr_allreduce_packet_rsag(inputs, outputs, scratch, scratch_bytes, flags, count, dtype, accum,
                              nranks, max_spins, dev_err=None, blocks_per_rank=0, threads=0,
                              stream=None) -> int:
    nb = _nbytes(count, dtype)
    _room(scratch, scratch_bytes, "scratch")
    _room(flags, 4 * PKT_FLAG_SLOTS * max(0, nranks), "flags")
    return load_library().mrr_allreduce_packet_rsag(
        _rank_ptrs(inputs, nranks, nb, "inputs"), _rank_ptrs(outputs, nranks, nb, "outputs"),
        _ptr(scratch), scratch_bytes, _ptr(flags), count, _dt(dtype), _dt(accum), nranks,
        max_spins, _ptr(dev_err), blocks_per_rank, threads, _stream(stream))


def mrr_fullmesh_scratch_bytes(count, dtype, nranks) -> int:
    return load_library().mrr_fullmesh_scratch_bytes(count, _dt(dtype), nranks)


def mrr_allreduce_fullmesh(inputs, outputs, scratch, scratch_bytes, flags, count, dtype, accum,
                           nranks, max_spins, dev_err=None, blocks_per_rank=0, threads=0,
                           stream=None) -> int:
    nb = _nbytes(count, dtype)
    _room(scratch, scratch_bytes, "scratch")
    _room(flags, 4 * PKT_FLAG_SLOTS * max(0, nranks), "flags")
    return load_library().mrr_allreduce_fullmesh(
        _rank_ptrs(inputs, nranks, nb, "inputs"), _rank_ptrs(outputs, nranks, nb, "outputs"),
        _ptr(scratch), scratch_bytes, _ptr(flags), count, _dt(dtype), _dt(accum), nranks,
        max_spins, _ptr(dev_err), blocks_per_rank, threads, _stream(stream))


def mrr_allreduce(inputs, outputs, count, dtype, accum, nranks, scratch=None, scratch_bytes=0,
                  flags=None, packet_max_bytes=0, max_spins=0, dev_err=None, stream=None) -> int:
    nb = _nbytes(count, dtype)
    _room(scratch, scratch_bytes, "scratch")
    _room(flags, 4 * PKT_FLAG_SLOTS * max(0, nranks), "flags")
    return load_library().mrr_allreduce(_rank_ptrs(inputs, nranks, nb, "inputs"),
                                        _rank_ptrs(outputs, nranks, nb, "outputs"), count,
                                        _dt(dtype), _dt(accum), nranks, _ptr(scratch),
                                        scratch_bytes, _ptr(flags), packet_max_bytes, max_spins,
                                        _ptr(dev_err), _stream(stream))


def mrr_packet_reduce(in_pkts, out_pkts, npkts, dtype, accum, nranks, flag_in, flag_out,
                      max_spins, dev_err=None, stream=None) -> int:
    _room(out_pkts, 8 * max(0, int(npkts)), "out_pkts")
    return load_library().mrr_packet_reduce(_rank_ptrs(in_pkts, nranks, 8 * max(0, int(npkts)),
                                                       "in_pkts"), _ptr(out_pkts), npkts,
                                            _dt(dtype), _dt(accum), nranks, flag_in, flag_out,
                                            max_spins, _ptr(dev_err), _stream(stream))


def mrr_pack(src, pkts, nbytes, flag, stream=None) -> int:
    _room(src, nbytes, "src")
    _room(pkts, (max(0, int(nbytes)) + 3) // 4 * 8, "pkts")
    return load_library().mrr_pack(_ptr(src), _ptr(pkts), nbytes, flag, _stream(stream))


def mrr_unpack(pkts, dst, nbytes, stream=None) -> int:
    _room(pkts, (max(0, int(nbytes)) + 3) // 4 * 8, "pkts")
    _room(dst, nbytes, "dst")
    return load_library().mrr_unpack(_ptr(pkts), _ptr(dst), nbytes, _stream(stream))


def _codec_room(src, ein, dst, eout, n):
    _room(src, max(0, int(n)) * ein, "src")
    _room(dst, max(0, int(n)) * eout, "dst")


def mrr_fp8b15_to_f16(src, dst, n, stream=None) -> int:
    _codec_room(src, 1, dst, 2, n)
    return load_library().mrr_fp8b15_to_f16(_ptr(src), _ptr(dst), n, _stream(stream))


def mrr_fp8b15_to_f32(src, dst, n, stream=None) -> int:
    _codec_room(src, 1, dst, 4, n)
    return load_library().mrr_fp8b15_to_f32(_ptr(src), _ptr(dst), n, _stream(stream))


def mrr_f16_to_fp8b15(src, dst, n, stream=None) -> int:
    _codec_room(src, 2, dst, 1, n)
    return load_library().mrr_f16_to_fp8b15(_ptr(src), _ptr(dst), n, _stream(stream))


def mrr_f32_to_fp8b15(src, dst, n, stream=None) -> int:
    _codec_room(src, 4, dst, 1, n)
    return load_library().mrr_f32_to_fp8b15(_ptr(src), _ptr(dst), n, _stream(stream))


def mrr_stream_copy(src, dst, nbytes, stream=None) -> int:
    _room(src, nbytes, "src")
    _room(dst, nbytes, "dst")
    return load_library().mrr_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream))
