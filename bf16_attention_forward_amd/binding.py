"""ctypes binding of libattn_fwd.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; torch is
used here only for device memory and the current stream.  If the library is
missing the binding raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn_fwd.so")

ATTN_LAYOUT = {"bshd": 0, "bhsd": 1}
ATTN_ROUND = {"rtne": 0, "rtna": 1, "rtz": 2}
ATTN_ROUND_WEIGHTS = 0x100   # round_mode flag: the in-loop softmax weights use the output's mode too
ATTN_OK = 0
ARGUMENT_ERRORS = {-1, -2, -3, -4, -5, -6, -7, -11}
HEAD_DIM = 128

# names of every entry point the header declares
EXPORTS = ("attn_fwd_bf16", "attn_fwd_bf16_ex", "attn_fwd_bf16_gqa", "attn_fwd_bf16_hd", "attn_fwd_bf16_hd_noalloc",
           "attn_fwd_bf16_paged", "attn_fwd_bf16_varlen",
           "attn_bwd_bf16", "attn_status_string", "attn_version")
NOALLOC_SCRATCH_BYTES = 34078720   # ATTN_NOALLOC_SCRATCH_BYTES
HEAD_DIMS = (128, 64)

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"attn_fwd_bf16 failed ({status}): {message}")
        self.status = status


def load_library(path: str | None = None):
    """Load and type the C ABI.  Raises if the built library is absent."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built: run bf16_attention_forward_amd.build.build() "
                           "(there is no fallback path)")
    lib = ctypes.CDLL(p)
    args = [ctypes.c_void_p] * 4 + [ctypes.c_int] + [ctypes.c_int64] * 4 + \
           [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.attn_fwd_bf16.argtypes = args
    lib.attn_fwd_bf16.restype = ctypes.c_int
    lib.attn_fwd_bf16_ex.argtypes = args + [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.attn_fwd_bf16_ex.restype = ctypes.c_int
    lib.attn_fwd_bf16_gqa.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] + [ctypes.c_int64] * 5 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.attn_fwd_bf16_gqa.restype = ctypes.c_int
    lib.attn_fwd_bf16_hd.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] + [ctypes.c_int64] * 6 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.attn_fwd_bf16_hd.restype = ctypes.c_int
    lib.attn_fwd_bf16_hd_noalloc.argtypes = lib.attn_fwd_bf16_hd.argtypes
    lib.attn_fwd_bf16_hd_noalloc.restype = ctypes.c_int
    lib.attn_fwd_bf16_paged.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int] + [ctypes.c_int64] * 9 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.attn_fwd_bf16_paged.restype = ctypes.c_int
    lib.attn_fwd_bf16_varlen.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 8 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.attn_fwd_bf16_varlen.restype = ctypes.c_int
    lib.attn_bwd_bf16.argtypes = [ctypes.c_void_p] * 9 + [ctypes.c_int] + [ctypes.c_int64] * 6 + \
        [ctypes.c_float, ctypes.c_int, ctypes.c_void_p]
    lib.attn_bwd_bf16.restype = ctypes.c_int
    lib.attn_status_string.argtypes = [ctypes.c_int]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def attn_status_string(status: int) -> str:
    return load_library().attn_status_string(int(status)).decode()


def attn_version() -> int:
    return int(load_library().attn_version())


def _raise(status: int):
    msg = attn_status_string(status)
    if status in ARGUMENT_ERRORS:
        raise ValueError(f"attn_fwd_bf16 argument error ({status}): {msg}")
    raise AttnError(status, msg)


def _dims(q: torch.Tensor, k: torch.Tensor, layout: str, grouped: bool = False, head_dims=(HEAD_DIM,)):
    """(B, Hq, Hkv, Sq, Skv) from the tensor shapes."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D")
    if layout == "bshd":
        B, Sq, H, D = q.shape
        Bk, Skv, Hk, Dk = k.shape
    elif layout == "bhsd":
        B, H, Sq, D = q.shape
        Bk, Hk, Skv, Dk = k.shape
    else:
        raise ValueError(f"layout must be 'bshd' or 'bhsd', got {layout!r}")
    if D not in head_dims or Dk != D:
        raise ValueError(f"head dimension must be one of {head_dims} (the same for q and k)")
    if Bk != B:
        raise ValueError("q and k/v must share the batch count")
    if grouped:
        if Hk < 1 or H % Hk != 0:
            raise ValueError("query heads must be a multiple of key/value heads")
    elif Hk != H:
        raise ValueError("q and k/v must share the head count (use attn_fwd_bf16_gqa for grouped heads)")
    return B, H, Hk, Sq, Skv


def _mode(round_mode: str, round_weights: bool) -> int:
    if round_mode not in ATTN_ROUND:
        raise ValueError(f"round_mode must be one of {sorted(ATTN_ROUND)}")
    return ATTN_ROUND[round_mode] | (ATTN_ROUND_WEIGHTS if round_weights else 0)


def _check_tensors(q, k, v, o):
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bfloat16")
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if o is None:
        return torch.empty_like(q)
    if o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous() or not o.is_cuda:
        raise ValueError("o must be a contiguous bfloat16 device tensor shaped like q")
    return o


def attn_fwd_bf16(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None, *,
                  layout: str = "bshd", scale: float | None = None, round_mode: str = "rtne",
                  stream: torch.cuda.Stream | None = None, kv_splits: int = 0,
                  block_order: int = 0, waves: int = 0, grid: int = 0,
                  round_weights: bool = False) -> torch.Tensor:
    """O = softmax(Q K^T * scale) V on the gfx950 library (bf16 in/out).

    q, k, v, o: contiguous bfloat16 CUDA tensors in the given layout.  o is
    allocated when None.  scale defaults to 1/sqrt(128) (as fp32).  The
    launch goes to ``stream`` (default: torch's current stream) and is
    asynchronous.  With kv_splits, block_order, waves and grid all 0
    (automatic) the call goes to the C entry point attn_fwd_bf16; otherwise
    to attn_fwd_bf16_ex with those planner overrides (waves 8 or 4 per
    work-group; grid: at most that many work-groups).  round_weights: round the in-loop
    softmax weights with ``round_mode`` too (ATTN_ROUND_WEIGHTS; default:
    nearest-even).
    """
    lib = load_library()
    o = _check_tensors(q, k, v, o)
    B, H, _, Sq, Skv = _dims(q, k, layout)
    sc = float(1.0 / math.sqrt(HEAD_DIM)) if scale is None else float(scale)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        if kv_splits == 0 and block_order == 0 and waves == 0 and grid == 0:
            # the planner's own choices: the plain entry point
            rc = lib.attn_fwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   ATTN_LAYOUT[layout], B, H, Sq, Skv, sc, _mode(round_mode, round_weights),
                                   st.cuda_stream)
        else:
            rc = lib.attn_fwd_bf16_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      ATTN_LAYOUT[layout], B, H, Sq, Skv, sc, _mode(round_mode, round_weights),
                                      st.cuda_stream, int(kv_splits), int(block_order), int(waves), int(grid))
    if rc != ATTN_OK:
        _raise(rc)
    return o


def attn_fwd_bf16_gqa(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None, *,
                      layout: str = "bshd", scale: float | None = None, causal: bool = False,
                      round_mode: str = "rtne", stream: torch.cuda.Stream | None = None,
                      lse: torch.Tensor | None = None, return_lse: bool = False,
                      round_weights: bool = False):
    """Grouped-query attention with an optional causal mask (attn_fwd_bf16_gqa).

    k and v may have fewer heads than q (query head h reads key/value head
    h // (Hq // Hkv)).  causal: query i sees keys j <= i + Skv - Sq; rows that
    see no key come out as zeros.  lse (float32 [B, Hq, Sq], or allocated when
    return_lse) receives each row's log-sum-exp of its scaled scores; then
    (o, lse) is returned.  Other arguments as attn_fwd_bf16.
    """
    lib = load_library()
    o = _check_tensors(q, k, v, o)
    B, Hq, Hkv, Sq, Skv = _dims(q, k, layout, grouped=True)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq)
                            or not lse.is_contiguous() or not lse.is_cuda):
        raise ValueError("lse must be a contiguous float32 device tensor shaped [B, Hq, Sq]")
    sc = float(1.0 / math.sqrt(HEAD_DIM)) if scale is None else float(scale)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd_bf16_gqa(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr() if lse is not None else None,
                                   ATTN_LAYOUT[layout], B, Hq, Hkv, Sq, Skv, sc, 1 if causal else 0,
                                   _mode(round_mode, round_weights), st.cuda_stream)
    if rc != ATTN_OK:
        _raise(rc)
    return (o, lse) if lse is not None else o


def attn_fwd_bf16_hd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor | None = None, *,
                     layout: str = "bshd", scale: float | None = None, causal: bool = False,
                     round_mode: str = "rtne", stream: torch.cuda.Stream | None = None,
                     lse: torch.Tensor | None = None, return_lse: bool = False,
                     round_weights: bool = False):
    """attn_fwd_bf16_gqa for head dimension 128 or 64 (attn_fwd_bf16_hd), taken
    from the tensors' last axis; scale defaults to 1/sqrt(head_dim)."""
    lib = load_library()
    o = _check_tensors(q, k, v, o)
    B, Hq, Hkv, Sq, Skv = _dims(q, k, layout, grouped=True, head_dims=HEAD_DIMS)
    hd = int(q.shape[-1])
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq)
                            or not lse.is_contiguous() or not lse.is_cuda):
        raise ValueError("lse must be a contiguous float32 device tensor shaped [B, Hq, Sq]")
    sc = float(1.0 / math.sqrt(hd)) if scale is None else float(scale)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd_bf16_hd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr() if lse is not None else None,
                                  ATTN_LAYOUT[layout], B, Hq, Hkv, Sq, Skv, hd, sc, 1 if causal else 0,
                                  _mode(round_mode, round_weights), st.cuda_stream)
    if rc != ATTN_OK:
        _raise(rc)
    return (o, lse) if lse is not None else o


def attn_fwd_bf16_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                        kv_lens: torch.Tensor, o: torch.Tensor | None = None, *, max_kv_len: int,
                        layout: str = "bshd", scale: float | None = None, causal: bool = False,
                        round_mode: str = "rtne", stream: torch.cuda.Stream | None = None,
                        lse: torch.Tensor | None = None, return_lse: bool = False,
                        round_weights: bool = False):
    """attn_fwd_bf16_hd on a paged key/value cache (attn_fwd_bf16_paged):
    k_cache, v_cache [num_pages, page_size, Hkv, head_dim] bf16, block_table
    int32 [B, pages_per_seq], kv_lens int32 [B] (keys per batch entry, at most
    max_kv_len); q and o in `layout`.  Scale defaults to 1/sqrt(head_dim)."""
    lib = load_library()
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor")
    if k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("k_cache and v_cache must be [num_pages, page_size, Hkv, head_dim] of one shape")
    for name, t in (("block_table", block_table), ("kv_lens", kv_lens)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
    if q.dim() != 4:
        raise ValueError("q must be 4-D")
    num_pages, page_size, Hkv, hd = (int(x) for x in k_cache.shape)
    if layout == "bshd":
        B, Sq, Hq, D = (int(x) for x in q.shape)
    elif layout == "bhsd":
        B, Hq, Sq, D = (int(x) for x in q.shape)
    else:
        raise ValueError(f"layout must be 'bshd' or 'bhsd', got {layout!r}")
    if D != hd or hd not in HEAD_DIMS:
        raise ValueError(f"head dimension must be one of {HEAD_DIMS} in q and the caches")
    if block_table.dim() != 2 or block_table.shape[0] != B or tuple(kv_lens.shape) != (B,):
        raise ValueError("block_table must be [B, pages_per_seq] and kv_lens [B]")
    if o is None:
        o = torch.empty_like(q)
    elif o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous() or not o.is_cuda:
        raise ValueError("o must be a contiguous bfloat16 device tensor shaped like q")
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq)
                            or not lse.is_contiguous() or not lse.is_cuda):
        raise ValueError("lse must be a contiguous float32 device tensor shaped [B, Hq, Sq]")
    sc = float(1.0 / math.sqrt(hd)) if scale is None else float(scale)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd_bf16_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), block_table.data_ptr(),
                                     kv_lens.data_ptr(), o.data_ptr(), lse.data_ptr() if lse is not None else None,
                                     ATTN_LAYOUT[layout], B, Hq, Hkv, Sq, int(max_kv_len), page_size,
                                     int(block_table.shape[1]), num_pages, hd, sc, 1 if causal else 0,
                                     _mode(round_mode, round_weights), st.cuda_stream)
    if rc != ATTN_OK:
        _raise(rc)
    return (o, lse) if lse is not None else o


def attn_fwd_bf16_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                         cu_seqlens_k: torch.Tensor, o: torch.Tensor | None = None, *, max_seqlen_q: int,
                         max_seqlen_k: int, scale: float | None = None, causal: bool = False,
                         round_mode: str = "rtne", stream: torch.cuda.Stream | None = None,
                         lse: torch.Tensor | None = None, return_lse: bool = False,
                         round_weights: bool = False):
    """attn_fwd_bf16_hd over packed sequences (attn_fwd_bf16_varlen): q, o
    [total_q, Hq, head_dim] and k, v [total_k, Hkv, head_dim] bf16 hold the rows
    of all sequences; cu_seqlens_q, cu_seqlens_k int32 [B + 1] are the prefix
    sums of their row counts.  lse, if wanted, is [Hq, total_q].  Scale
    defaults to 1/sqrt(head_dim)."""
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 3:
            raise ValueError(f"{name} must be a contiguous 3-D bfloat16 device tensor")
    for name, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous() or t.dim() != 1:
            raise ValueError(f"{name} must be a contiguous 1-D int32 device tensor")
    if cu_seqlens_q.shape != cu_seqlens_k.shape or cu_seqlens_q.shape[0] < 2:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both be [B + 1], B >= 1")
    total_q, Hq, D = (int(x) for x in q.shape)
    total_k, Hkv, Dk = (int(x) for x in k.shape)
    if k.shape != v.shape or D != Dk or D not in HEAD_DIMS:
        raise ValueError(f"k and v must be [total_k, Hkv, head_dim] alike, head_dim one of {HEAD_DIMS} as in q")
    B = int(cu_seqlens_q.shape[0]) - 1
    if o is None:
        o = torch.empty_like(q)
    elif o.shape != q.shape or o.dtype != torch.bfloat16 or not o.is_contiguous() or not o.is_cuda:
        raise ValueError("o must be a contiguous bfloat16 device tensor shaped like q")
    if lse is None and return_lse:
        lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (Hq, total_q)
                            or not lse.is_contiguous() or not lse.is_cuda):
        raise ValueError("lse must be a contiguous float32 device tensor shaped [Hq, total_q]")
    sc = float(1.0 / math.sqrt(D)) if scale is None else float(scale)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd_bf16_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                      lse.data_ptr() if lse is not None else None, cu_seqlens_q.data_ptr(),
                                      cu_seqlens_k.data_ptr(), B, Hq, Hkv, total_q, total_k, int(max_seqlen_q),
                                      int(max_seqlen_k), D, sc, 1 if causal else 0,
                                      _mode(round_mode, round_weights), st.cuda_stream)
    if rc != ATTN_OK:
        _raise(rc)
    return (o, lse) if lse is not None else o


def attn_fwd_bf16_hd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, *,
                             layout: str = "bshd", scale: float | None = None, causal: bool = False,
                             round_mode: str = "rtne", stream: torch.cuda.Stream | None = None,
                             lse: torch.Tensor | None = None, round_weights: bool = False):
    """attn_fwd_bf16_hd through the allocation-free entry point
    (attn_fwd_bf16_hd_noalloc): the split partials go to the library's fixed
    device array, so nothing is allocated -- o (and lse, if wanted) must be
    passed in.  Calls on one GPU that overlap in time race on that array."""
    lib = load_library()
    if o is None:
        raise ValueError("o must be given: the allocation-free call allocates nothing")
    o = _check_tensors(q, k, v, o)
    B, Hq, Hkv, Sq, Skv = _dims(q, k, layout, grouped=True, head_dims=HEAD_DIMS)
    hd = int(q.shape[-1])
    if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq)
                            or not lse.is_contiguous() or not lse.is_cuda):
        raise ValueError("lse must be a contiguous float32 device tensor shaped [B, Hq, Sq]")
    sc = float(1.0 / math.sqrt(hd)) if scale is None else float(scale)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        rc = lib.attn_fwd_bf16_hd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                          lse.data_ptr() if lse is not None else None,
                                          ATTN_LAYOUT[layout], B, Hq, Hkv, Sq, Skv, hd, sc, 1 if causal else 0,
                                          _mode(round_mode, round_weights), st.cuda_stream)
    if rc != ATTN_OK:
        _raise(rc)
    return (o, lse) if lse is not None else o


def attn_bwd_bf16(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, do: torch.Tensor,
                  lse: torch.Tensor, *, layout: str = "bshd", scale: float | None = None,
                  causal: bool = False, stream: torch.cuda.Stream | None = None, dq: torch.Tensor | None = None,
                  dk: torch.Tensor | None = None, dv: torch.Tensor | None = None):
    """Backward pass (attn_bwd_bf16): returns (dq, dk, dv) for the output
    gradient ``do``, from the forward's output ``o`` and log-sum-exp ``lse``
    (float32 [B, Hq, Sq]).  Head dimension 128 or 64; k and v may have fewer heads
    than q (the forward's grouping; dk, dv then sum over each group);
    causal: the forward's mask (query i sees keys j <= i + Skv - Sq)."""
    lib = load_library()
    _check_tensors(q, k, v, o)
    B, H, Hkv, Sq, Skv = _dims(q, k, layout, grouped=True, head_dims=HEAD_DIMS)
    D = q.shape[-1]
    for name, t in (("do", do),):
        if t.dtype != torch.bfloat16 or t.shape != q.shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor shaped like q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous() or not lse.is_cuda:
        raise ValueError("lse must be a contiguous float32 device tensor shaped [B, H, Sq]")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.dtype != torch.bfloat16 or t.shape != ref.shape or not t.is_contiguous() or not t.is_cuda:
            raise ValueError(f"{name} must be a contiguous bfloat16 device tensor shaped like its input")
    sc = float(1.0 / math.sqrt(D)) if scale is None else float(scale)
    st = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):
        rc = lib.attn_bwd_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ATTN_LAYOUT[layout],
                               B, H, Hkv, Sq, Skv, D, sc, 1 if causal else 0, st.cuda_stream)
    if rc != ATTN_OK:
        _raise(rc)
    return dq, dk, dv


def attn_fwd_bf16_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, layout: int, B: int, H: int,
                      Sq: int, Skv: int, scale: float, round_mode: int, stream_ptr: int,
                      kv_splits: int = 0, block_order: int = 0, waves: int = 0, grid: int = 0) -> int:
    """Call the C entry point with raw integers; returns the status code."""
    lib = load_library()
    return int(lib.attn_fwd_bf16_ex(q_ptr, k_ptr, v_ptr, o_ptr, layout, B, H, Sq, Skv, scale,
                                    round_mode, stream_ptr, kv_splits, block_order, waves, grid))
