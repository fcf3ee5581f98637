"""ctypes binding of libra.so (the C ABI in include/ra.h). Argument marshalling only:
every step of the computation runs in the library's HIP kernels. torch supplies device
memory and the current stream.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libra.so")

RA_BF16, RA_F32 = 0, 1
RA_OK, RA_ERR_ARG, RA_ERR_SHAPE, RA_ERR_UNSUPPORTED, RA_ERR_ALIGN, RA_ERR_LAUNCH = 0, -1, -2, -3, -4, -5
# Names every build of the library exports (the entry points include/ra.h declares).
EXPORTED = ("ra_rank_forward", "ra_rank_forward_doc", "ra_rank_forward_accumulate", "ra_merge", "ra_last_error",
            "ra_version")

_lib = None


class RaError(RuntimeError):
    """A nonzero status from the library, with ra_last_error()'s text."""

    def __init__(self, code: int, where: str, text: str):
        super().__init__(f"{where} failed with status {code}: {text}")
        self.code = code


class RaValueError(RaError, ValueError):
    """Argument, shape, support or alignment errors (codes -1 .. -4)."""


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libra.so once. Raises if it has not been built: there is no fallback."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m blockwise_ring_attention_amd.csrc.build` "
                           "(or __graft_entry__.build()); there is no CPU fallback")
    lib = ctypes.CDLL(p)
    vp, ci, cll = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong
    lib.ra_rank_forward.argtypes = [vp, vp, vp, vp, vp] + [ci] * 13 + [vp]
    lib.ra_rank_forward.restype = ci
    lib.ra_rank_forward_doc.argtypes = [vp, vp, vp, vp, vp, vp] + [ci] * 12 + [vp]
    lib.ra_rank_forward_doc.restype = ci
    lib.ra_rank_forward_accumulate.argtypes = [vp, vp, vp, vp, vp, vp] + [ci] * 14 + [vp]
    lib.ra_rank_forward_accumulate.restype = ci
    lib.ra_merge.argtypes = [vp, vp, vp, vp, vp, vp, cll, ci, ci, vp]
    lib.ra_merge.restype = ci
    lib.ra_last_error.argtypes = []
    lib.ra_last_error.restype = ctypes.c_char_p
    lib.ra_version.argtypes = []
    lib.ra_version.restype = ci
    if path is None:
        _lib = lib
    return lib


def use_library(path: str) -> ctypes.CDLL:
    """Make the library at `path` (same C ABI: a design-choice comparison build made by
    the build script) the one every later call goes through."""
    global _lib
    _lib = load(path)
    return _lib


def last_error() -> str:
    return load().ra_last_error().decode()


def version() -> int:
    return load().ra_version()


def check(code: int, where: str) -> None:
    if code == RA_OK:
        return
    text = last_error()
    if code in (RA_ERR_ARG, RA_ERR_SHAPE, RA_ERR_UNSUPPORTED, RA_ERR_ALIGN):
        raise RaValueError(code, where, text)
    raise RaError(code, where, text)


def ra_rank_forward(q, k_blocks, v_blocks, out, lse, batch, hq, hkv, nq, nkv, head_dim, c, rank, causal, zigzag,
                    round_begin, round_end, dtype, stream) -> int:
    """Raw call with integer pointers; returns the status code."""
    return load().ra_rank_forward(q, k_blocks, v_blocks, out, lse, batch, hq, hkv, nq, nkv, head_dim, c, rank,
                                  int(causal), int(zigzag), round_begin, round_end, dtype, stream)


def ra_rank_forward_doc(q, k_blocks, v_blocks, doc_start, out, lse, batch, hq, hkv, nq, nkv, head_dim, c, rank,
                        zigzag, round_begin, round_end, dtype, stream) -> int:
    """Raw call with integer pointers; returns the status code."""
    return load().ra_rank_forward_doc(q, k_blocks, v_blocks, doc_start, out, lse, batch, hq, hkv, nq, nkv, head_dim,
                                      c, rank, int(zigzag), round_begin, round_end, dtype, stream)


def ra_rank_forward_accumulate(q, k_blocks, v_blocks, doc_start, out, lse, batch, hq, hkv, nq, nkv, head_dim, c,
                               rank, causal, zigzag, round_begin, round_end, dtype, out_dtype, stream) -> int:
    """Raw call with integer pointers (doc_start 0 or None: no document mask)."""
    return load().ra_rank_forward_accumulate(q, k_blocks, v_blocks, doc_start or None, out, lse, batch, hq, hkv, nq,
                                             nkv, head_dim, c, rank, int(causal), int(zigzag), round_begin,
                                             round_end, dtype, out_dtype, stream)


def ra_merge(out_a, lse_a, out_b, lse_b, out, lse, rows, head_dim, dtype, stream) -> int:
    return load().ra_merge(out_a, lse_a, out_b, lse_b, out, lse, rows, head_dim, dtype, stream)
