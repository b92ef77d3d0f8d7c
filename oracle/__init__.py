"""CPU oracle for the N-rank allreduce reduction -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports or calls it, and the two share no code.

The arithmetic lives in ``mrr_oracle.c`` (plain C, table-driven rounding,
sequential rank-order sums); this module only builds it with gcc and marshals
numpy arrays through ctypes.  Values travel as raw bits: f32 as ``float32``,
f16 and bf16 as ``uint16`` codes, FP8 E4M3B15 ("fp8") and OCP FP8 E4M3FN
("fp8fn") as ``uint8`` codes.

What each function computes, and which passage it follows, is stated in the C
source next to the function.  Parity status of every function is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mrr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_mrr.so")

# Type ids private to the oracle (mirrors the enum at the top of mrr_oracle.c).
TYPE_IDS = {"f32": 1, "f16": 2, "bf16": 3, "fp8": 4, "fp8fn": 5}
NP_BITS = {"f32": np.float32, "f16": np.uint16, "bf16": np.uint16, "fp8": np.uint8,
           "fp8fn": np.uint8}
ELEM_SIZE = {"f32": 4, "f16": 2, "bf16": 2, "fp8": 1, "fp8fn": 1}

_lock = threading.Lock()
_lib = None


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compiles the C oracle into a shared library (gcc -O2, no fast-math)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def _declare(L: ctypes.CDLL) -> ctypes.CDLL:
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    u32 = ctypes.c_uint32
    L.orc_allreduce.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), sz, i, i, i, i, i]
    L.orc_allreduce.restype = i
    L.orc_convert.argtypes = [vp, vp, sz, i, i]
    L.orc_convert.restype = i
    L.orc_narrow_f64.argtypes = [vp, vp, sz, i]
    L.orc_narrow_f64.restype = i
    L.orc_widen_f64.argtypes = [vp, vp, sz, i]
    L.orc_widen_f64.restype = i
    L.orc_pack.argtypes = [vp, sz, u32, vp]
    L.orc_pack.restype = None
    L.orc_unpack.argtypes = [vp, sz, vp]
    L.orc_unpack.restype = None
    L.orc_next_flag.argtypes = [u32]
    L.orc_next_flag.restype = u32
    L.orc_allreduce_packet.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), vp, sz,
                                       i, i, i, u32]
    L.orc_allreduce_packet.restype = i
    L.orc_packet_reduce.argtypes = [ctypes.POINTER(vp), vp, sz, i, i, i, u32, u32]
    L.orc_packet_reduce.restype = i
    L.orc_allreduce_packet_rsag.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), vp, sz,
                                            i, i, i, u32]
    L.orc_allreduce_packet_rsag.restype = i
    L.orc_allreduce_fullmesh.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), vp, sz, i, i, i,
                                         i, u32]
    L.orc_allreduce_fullmesh.restype = i
    return L


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _bits(a, t: str) -> np.ndarray:
    a = np.ascontiguousarray(a)
    want = np.dtype(NP_BITS[t])
    if a.dtype != want:
        if a.dtype.itemsize != want.itemsize:
            raise TypeError("array of %s cannot hold %s bits" % (a.dtype, t))
        a = a.view(want)
    return a


def _ptr_array(arrs):
    return (ctypes.c_void_p * len(arrs))(*[_ptr(a) for a in arrs])


def _accum(t_in: str, accum: str) -> str:
    # AUTO resolves to the input type (the pages' default for accumDtype).
    return t_in if accum in (None, "auto") else accum


class Oracle:
    """The oracle's entry points, bound to one build of the C library."""

    def __init__(self, L: ctypes.CDLL):
        self.L = L

    def allreduce(self, inputs, t_in: str, accum: str = "f32", t_out: str | None = None,
                  out: np.ndarray | None = None) -> np.ndarray:
        """Elementwise sum over ranks in order 0..N-1 (the RS/AG result).

        Returns ONE output array: by definition all N outputs are this array.
        `out`, when given, is a contiguous array of count elements of the
        output type's bits that receives the result (and is returned).
        """
        t_out = t_out or t_in
        accum = _accum(t_in, accum)
        ins = [_bits(a, t_in) for a in inputs]
        count = ins[0].size
        assert all(a.size == count for a in ins)
        if out is None:
            out = np.empty(count, dtype=NP_BITS[t_out])
        else:
            assert out.flags.c_contiguous and out.size == count
            assert out.dtype == np.dtype(NP_BITS[t_out])
        rc = self.L.orc_allreduce(_ptr_array(ins), _ptr_array([out]), count, TYPE_IDS[t_in],
                                 TYPE_IDS[accum], TYPE_IDS[t_out], len(ins), 1)
        if rc != 0:
            raise ValueError("oracle rejected types %s/%s/%s" % (t_in, accum, t_out))
        return out

    def allreduce_all(self, inputs, t_in: str, accum: str = "f32", t_out: str | None = None):
        """Same as allreduce(), writing N separate outputs (the all-gather)."""
        t_out = t_out or t_in
        accum = _accum(t_in, accum)
        ins = [_bits(a, t_in) for a in inputs]
        count = ins[0].size
        outs = [np.empty(count, dtype=NP_BITS[t_out]) for _ in ins]
        rc = self.L.orc_allreduce(_ptr_array(ins), _ptr_array(outs), count, TYPE_IDS[t_in],
                                 TYPE_IDS[accum], TYPE_IDS[t_out], len(ins), len(outs))
        if rc != 0:
            raise ValueError("oracle rejected types")
        return outs

    def convert(self, a, t_in: str, t_out: str, out: np.ndarray | None = None) -> np.ndarray:
        """Elementwise conversion: exact decode, one RNE rounding (FP8 saturates).
        `out` as for allreduce()."""
        a = _bits(a, t_in)
        if out is None:
            out = np.empty(a.size, dtype=NP_BITS[t_out])
        else:
            assert out.flags.c_contiguous and out.size == a.size
            assert out.dtype == np.dtype(NP_BITS[t_out])
        if self.L.orc_convert(_ptr(a), _ptr(out), a.size, TYPE_IDS[t_in], TYPE_IDS[t_out]) != 0:
            raise ValueError("bad types")
        return out

    def narrow_f64(self, x, t: str) -> np.ndarray:
        """Rounds float64 values into type t (bits)."""
        x = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(x.size, dtype=NP_BITS[t])
        self.L.orc_narrow_f64(_ptr(x), _ptr(out), x.size, TYPE_IDS[t])
        return out

    def widen_f64(self, a, t: str) -> np.ndarray:
        """Exact value of each code of type t, as float64."""
        a = _bits(a, t)
        out = np.empty(a.size, dtype=np.float64)
        self.L.orc_widen_f64(_ptr(a), _ptr(out), a.size, TYPE_IDS[t])
        return out

    def pack(self, data: bytes | np.ndarray, flag: int) -> np.ndarray:
        """LL packets of a byte buffer: uint64 (flag << 32) | word_k."""
        b = np.frombuffer(bytes(data), dtype=np.uint8) if not isinstance(data, np.ndarray) \
            else np.ascontiguousarray(data).view(np.uint8).ravel()
        n = (b.size + 3) // 4
        pk = np.empty(n, dtype=np.uint64)
        self.L.orc_pack(_ptr(b) if b.size else None, b.size, flag, _ptr(pk) if n else None)
        return pk

    def unpack(self, pkts: np.ndarray, nbytes: int) -> np.ndarray:
        pkts = np.ascontiguousarray(pkts, dtype=np.uint64)
        out = np.empty(nbytes, dtype=np.uint8)
        if nbytes:
            self.L.orc_unpack(_ptr(pkts), nbytes, _ptr(out))
        return out

    def next_flag(self, prev: int) -> int:
        return int(self.L.orc_next_flag(prev))

    def allreduce_packet(self, inputs, t: str, accum: str, flag: int):
        """Expected (scratch, output) after one allpair packet allreduce with flag F.

        scratch has shape (N, N, npkt) indexed [dst][src][k]; its self slots
        (d == s) are zero here and carry no meaning.
        """
        accum = _accum(t, accum)
        ins = [_bits(a, t) for a in inputs]
        n = len(ins)
        count = ins[0].size
        npkt = (count * ELEM_SIZE[t] + 3) // 4
        scratch = np.zeros((n, n, npkt), dtype=np.uint64)
        outs = [np.empty(count, dtype=NP_BITS[t]) for _ in ins]
        rc = self.L.orc_allreduce_packet(_ptr_array(ins), _ptr_array(outs), _ptr(scratch), count,
                                        TYPE_IDS[t], TYPE_IDS[accum], n, flag)
        if rc != 0:
            raise ValueError("oracle rejected types")
        return scratch, outs[0]

    def allreduce_packet_rsag(self, inputs, t: str, accum: str, flag: int):
        """Expected (rs, ag, output) after one two-phase packet allreduce with
        flag F: rs and ag have shape (N, N, cw) indexed [dst][src][word];
        slots the call does not write are zero here."""
        accum = _accum(t, accum)
        ins = [_bits(a, t) for a in inputs]
        n = len(ins)
        count = ins[0].size
        e = ELEM_SIZE[t]
        per = -(-count // n)
        chunk = -(-per // (16 // e)) * (16 // e)
        cw = chunk * e // 4
        scratch = np.zeros((2, n, n, cw), dtype=np.uint64)
        outs = [np.empty(count, dtype=NP_BITS[t]) for _ in ins]
        rc = self.L.orc_allreduce_packet_rsag(_ptr_array(ins), _ptr_array(outs), _ptr(scratch),
                                              count, TYPE_IDS[t], TYPE_IDS[accum], n, flag)
        if rc != 0:
            raise ValueError("oracle rejected types")
        return scratch[0], scratch[1], outs[0]

    @staticmethod
    def fullmesh_layout(count: int, t: str, nranks: int):
        """(chunk elements C, semaphore bytes, inbox bytes) of the full-mesh
        scratch image: N*N*1024 uint64 semaphores, then N*N*C*e inbox bytes."""
        e = ELEM_SIZE[t]
        per = -(-count // nranks)
        chunk = -(-per // (16 // e)) * (16 // e)
        return chunk, nranks * nranks * 1024 * 8, nranks * nranks * chunk * e

    def allreduce_fullmesh(self, inputs, t: str, accum: str, flag: int, nblocks: int,
                           scratch: np.ndarray | None = None):
        """Expected (scratch image, output) after one full-mesh allreduce with
        flag F and nblocks blocks per rank, starting from `scratch` (a uint8
        image of the whole scratch; zeros when None).  The returned image is a
        new array; see the C source for what the call writes."""
        accum = _accum(t, accum)
        ins = [_bits(a, t) for a in inputs]
        n = len(ins)
        count = ins[0].size
        _, sem_b, box_b = self.fullmesh_layout(count, t, n)
        img = np.zeros(sem_b + box_b, dtype=np.uint8) if scratch is None else \
            np.array(scratch, dtype=np.uint8, copy=True).ravel()
        assert img.size >= sem_b + box_b
        outs = [np.empty(count, dtype=NP_BITS[t]) for _ in ins]
        rc = self.L.orc_allreduce_fullmesh(_ptr_array(ins), _ptr_array(outs), _ptr(img), count,
                                           TYPE_IDS[t], TYPE_IDS[accum], n, nblocks, flag)
        if rc != 0:
            raise ValueError("oracle rejected arguments")
        return img, outs[0]

    def packet_reduce(self, in_pkts, t: str, accum: str, flag_in: int, flag_out: int):
        """Receive step alone.  Returns the output packets, or None when some input
        packet does not carry flag_in (the call would keep waiting)."""
        accum = _accum(t, accum)
        ins = [np.ascontiguousarray(p, dtype=np.uint64) for p in in_pkts]
        npk = ins[0].size
        out = np.empty(npk, dtype=np.uint64)
        rc = self.L.orc_packet_reduce(_ptr_array(ins), _ptr(out), npk, TYPE_IDS[t], TYPE_IDS[accum],
                                     len(ins), flag_in, flag_out)
        if rc == -2:
            return None
        if rc != 0:
            raise ValueError("oracle rejected arguments")
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle(lib())
    return _default


def load(path: str) -> Oracle:
    """An Oracle bound to another build of the C source (used by the tests
    that plant mistakes in a copy of the oracle)."""
    return Oracle(_declare(ctypes.CDLL(path)))


def __getattr__(name):
    # module-level access (oracle.allreduce, ...) goes to the default build
    if name in Oracle.__dict__ and not name.startswith("_"):
        return getattr(default(), name)
    raise AttributeError(name)
