"""Per-rank blockwise Ring Attention for AMD MI355X (gfx950).

``rank_forward`` computes one rank's share of Ring Attention: the rank's queries against
the c key/value blocks of the ring, folded in ring order with the online softmax (the
result equals full-row softmax attention), with the causal mask, zigzag chunk
ownership, grouped-query heads and per-row logsumexp. ``merge`` combines two partial
results over disjoint key sets; ``rank_forward_accumulate`` folds some rounds straight into
a running (out, lse), the streamed form of the ring. All are thin wrappers over the C ABI of ``libra.so``
(``include/ra.h``): torch tensors supply device memory and the current stream; all
arithmetic runs in the library's HIP kernels.
"""

from __future__ import annotations

from . import _binding
from ._binding import RaError, RaValueError, last_error, version  # noqa: F401

__all__ = ["rank_forward", "rank_forward_doc", "rank_forward_accumulate", "merge", "version", "last_error",
           "RaError", "RaValueError"]


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return _binding.RA_BF16
    if t.dtype == torch.float32:
        return _binding.RA_F32
    raise ValueError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _ptr(t):
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def _stream_handle(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def rank_forward(q, k_blocks, v_blocks, c: int, rank: int, causal: bool, zigzag: bool,
                 round_begin: int = 0, round_end: int | None = None, *, out=None, lse=None,
                 with_lse: bool = True):
    """One rank's share of Ring Attention over rounds [round_begin, round_end).

    q        [B, Hq, Nq, d]       bf16 or fp32, on the GPU, contiguous
    k_blocks [c, B, Hkv, n, d]    block j = rank j's keys (owner order), same dtype
    v_blocks [c, B, Hkv, n, d]
    Returns (out [B, Hq, Nq, d] in q's dtype, lse [B, Hq, Nq] fp32 or None).
    ``out``/``lse`` may be preallocated; the call is asynchronous on the current stream.
    """
    return _forward(q, k_blocks, v_blocks, None, c, rank, causal, zigzag, round_begin, round_end, out, lse, with_lse)


def rank_forward_doc(q, k_blocks, v_blocks, doc_start, c: int, rank: int, zigzag: bool,
                     round_begin: int = 0, round_end: int | None = None, *, out=None, lse=None,
                     with_lse: bool = True):
    """``rank_forward`` (causal) with the document mask of a packed sequence: the query
    at global position p sees the keys at positions doc_start[p] <= x <= p.

    doc_start [c * n] int32 on the GPU: for each global position, where its document
    begins. Other arguments and the result are those of ``rank_forward``.
    """
    _check_doc(doc_start, c, k_blocks)
    return _forward(q, k_blocks, v_blocks, doc_start, c, rank, True, zigzag, round_begin, round_end, out, lse,
                    with_lse)


def rank_forward_accumulate(q, k_blocks, v_blocks, out, lse, c: int, rank: int, causal: bool, zigzag: bool,
                            round_begin: int = 0, round_end: int | None = None, *, doc_start=None):
    """Fold rounds [round_begin, round_end) into the running result (out, lse) in place.

    ``out`` [B, Hq, Nq, d] and ``lse`` [B, Hq, Nq] fp32 hold the result over the keys
    folded so far (lse = -inf where none: start from ``lse.fill_(-inf)``; out is then
    ignored). Afterwards they hold the result over those keys and this call's rounds,
    which must not repeat a round already folded in. ``out`` has q's dtype or, with
    bf16 inputs, fp32: an fp32 running output does not gain bf16 rounding at every call.
    ``doc_start`` (optional) adds the document mask of ``rank_forward_doc`` (causal
    only). Returns (out, lse).
    """
    import torch
    if out is None or lse is None:
        raise ValueError("rank_forward_accumulate needs the running out and lse tensors")
    if doc_start is not None:
        if not causal:
            raise ValueError("a document mask needs causal=True")
        _check_doc(doc_start, c, k_blocks)
    return _forward(q, k_blocks, v_blocks, doc_start, c, rank, causal, zigzag, round_begin, round_end, out, lse,
                    True, accumulate=True)


def _check_doc(doc_start, c, k_blocks):
    import torch
    if (not doc_start.is_cuda or doc_start.dtype != torch.int32 or not doc_start.is_contiguous()
            or doc_start.device != k_blocks.device):
        raise ValueError("doc_start must be a contiguous int32 GPU tensor on the inputs' device")
    if doc_start.dim() != 1 or doc_start.numel() != c * k_blocks.shape[3]:
        raise ValueError(f"doc_start needs c * n = {c * k_blocks.shape[3]} entries, got {tuple(doc_start.shape)}")


def _forward(q, k_blocks, v_blocks, doc_start, c, rank, causal, zigzag, round_begin, round_end, out, lse, with_lse,
             accumulate=False):
    import torch
    if round_end is None:
        round_end = c
    for name, t in (("q", q), ("k_blocks", k_blocks), ("v_blocks", v_blocks)):
        if not t.is_cuda or t.device != q.device:
            raise ValueError(f"{name} must be a GPU tensor on q's device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dtype != q.dtype:
            raise ValueError(f"{name} dtype {t.dtype} differs from q's {q.dtype}")
    if q.dim() != 4 or k_blocks.dim() != 5 or v_blocks.shape != k_blocks.shape:
        raise ValueError("expected q [B,Hq,Nq,d] and k_blocks, v_blocks [c,B,Hkv,n,d] of equal shape")
    B, hq, nq, d = q.shape
    cc, b2, hkv, nkv, d2 = k_blocks.shape
    if cc != c or b2 != B or d2 != d:
        raise ValueError(f"k_blocks shape {tuple(k_blocks.shape)} does not match q {tuple(q.shape)} and c={c}")
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous tensor like q")
    elif out.dtype != q.dtype and not (accumulate and q.dtype == torch.bfloat16 and out.dtype == torch.float32):
        raise ValueError(f"out dtype {out.dtype} does not match q's {q.dtype}")
    if lse is None and with_lse:
        lse = torch.empty((B, hq, nq), dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != (B, hq, nq) or lse.dtype != torch.float32 or not lse.is_contiguous()
                              or lse.device != q.device):
        raise ValueError("lse must be a contiguous fp32 tensor [B, Hq, Nq] on q's device")
    if accumulate:
        code = _binding.ra_rank_forward_accumulate(_ptr(q), _ptr(k_blocks), _ptr(v_blocks), _ptr(doc_start),
                                                   _ptr(out), _ptr(lse), B, hq, hkv, nq, nkv, d, c, rank, causal,
                                                   zigzag, round_begin, round_end, dt, _dtype_code(out),
                                                   _stream_handle(q.device))
        _binding.check(code, "ra_rank_forward_accumulate")
    elif doc_start is None:
        code = _binding.ra_rank_forward(_ptr(q), _ptr(k_blocks), _ptr(v_blocks), _ptr(out), _ptr(lse),
                                        B, hq, hkv, nq, nkv, d, c, rank, causal, zigzag, round_begin, round_end, dt,
                                        _stream_handle(q.device))
        _binding.check(code, "ra_rank_forward")
    else:
        code = _binding.ra_rank_forward_doc(_ptr(q), _ptr(k_blocks), _ptr(v_blocks), _ptr(doc_start), _ptr(out),
                                            _ptr(lse), B, hq, hkv, nq, nkv, d, c, rank, zigzag, round_begin,
                                            round_end, dt, _stream_handle(q.device))
        _binding.check(code, "ra_rank_forward_doc")
    return out, lse


def merge(out_a, lse_a, out_b, lse_b, *, out=None, lse=None):
    """Merge two partial results (out [..., d], lse [...]) over disjoint key sets.
    ``out``/``lse`` may be ``out_a``/``lse_a`` for an in-place update."""
    import torch
    if out_a.shape != out_b.shape or lse_a.shape != lse_b.shape or out_a.shape[:-1] != lse_a.shape:
        raise ValueError("merge needs out_a/out_b [..., d] and lse_a/lse_b [...] of matching shapes")
    for t in (out_a, lse_a, out_b, lse_b):
        if not t.is_cuda or not t.is_contiguous() or t.device != out_a.device:
            raise ValueError("merge inputs must be contiguous GPU tensors on one device")
    if lse_a.dtype != torch.float32 or lse_b.dtype != torch.float32 or out_b.dtype != out_a.dtype:
        raise ValueError("lse must be fp32 and both outputs share a dtype")
    dt = _dtype_code(out_a)
    if out is None:
        out = torch.empty_like(out_a)
    elif (out.shape != out_a.shape or out.dtype != out_a.dtype or not out.is_contiguous()
          or out.device != out_a.device):
        raise ValueError("out must be a contiguous tensor of out_a's shape, dtype and device")
    if lse is None:
        lse = torch.empty_like(lse_a)
    elif (lse.shape != lse_a.shape or lse.dtype != torch.float32 or not lse.is_contiguous()
          or lse.device != out_a.device):
        raise ValueError("lse must be a contiguous fp32 tensor of lse_a's shape on out_a's device")
    rows = lse_a.numel()
    code = _binding.ra_merge(_ptr(out_a), _ptr(lse_a), _ptr(out_b), _ptr(lse_b), _ptr(out), _ptr(lse), rows,
                             out_a.shape[-1], dt, _stream_handle(out_a.device))
    _binding.check(code, "ra_merge")
    return out, lse
