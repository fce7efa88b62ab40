"""ctypes binding of libbsattn.so.  Argument marshalling only: torch supplies device memory and
the current stream; every step of the layer runs in the library's HIP kernels.  There is no
fallback: if the library is missing or a call fails, an exception is raised."""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
# BSATTN_LIB names another build of the same library (the host-sanitizer build of the tests)
LIB_PATH = os.environ.get("BSATTN_LIB") or os.path.join(HERE, "libbsattn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "bsattn.h")

BSA_OK, BSA_E_ARG, BSA_E_UNSUPPORTED, BSA_E_WORKSPACE, BSA_E_HIP = 0, -1, -2, -3, -4
BSA_F32, BSA_BF16 = 0, 1
BSA_MEANPOOL, BSA_EXACT_ONLY, BSA_COMPRESSED_ONLY, BSA_TAIL_BLOCK = 1, 2, 4, 8
BSA_CHECK_LISTS = 16
BLOCK = 64


class BsaDesc(ctypes.Structure):
    _fields_ = [("heads", ctypes.c_int32), ("tokens", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class BsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"bsattn status {status}: {msg}")
        self.status = status


_P = ctypes.c_void_p
_SIGS = {
    "bsa_status_str": (ctypes.c_char_p, [ctypes.c_int32]),
    "bsa_last_error": (ctypes.c_char_p, []),
    "bsa_topk_count": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_float]),
    "bsa_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(BsaDesc)]),
    "bsa_reblock": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), _P, _P, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P]),
    "bsa_reblock_layout": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), _P, _P, ctypes.c_int32, _P,
                                            _P, _P, _P, ctypes.c_size_t, _P]),
    "bsa_reblock_ex": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), _P, _P, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_uint32, _P, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "bsa_reblock_side": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), _P, _P, ctypes.c_int32,
                                          ctypes.c_int32, ctypes.c_uint32, _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "bsa_select": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), _P, _P, _P, _P, ctypes.c_float,
                                    ctypes.c_int32, _P, _P, _P, ctypes.c_size_t, _P]),
    "bsa_sparse_attn": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), _P, _P, _P, _P, _P, _P,
                                         ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, _P, _P,
                                         _P, ctypes.c_size_t, _P]),
    "bsa_prepare_kv": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), _P, _P, _P, _P, ctypes.c_uint32,
                                        ctypes.c_float, _P, ctypes.c_size_t, _P]),
    "bsa_attend": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), _P, _P, _P, _P, _P, _P,
                                    ctypes.c_int32, ctypes.c_uint32, ctypes.c_float, _P, _P, _P,
                                    ctypes.c_size_t, _P]),
    "bsa_summaries": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), _P, _P, _P, _P, ctypes.c_uint32,
                                       ctypes.c_float, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "bsa_summaries_noalloc_bytes": (ctypes.c_size_t, [ctypes.POINTER(BsaDesc)]),
    "bsa_summaries_noalloc": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), _P, _P, _P, _P,
                                               ctypes.c_uint32, ctypes.c_float, _P, _P, _P, _P]),
    "bsa_workspace_bytes_ctx": (ctypes.c_size_t, [ctypes.POINTER(BsaDesc), ctypes.c_int32]),
    "bsa_sparse_attn_ctx": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), ctypes.c_int32, _P, _P, _P,
                                             _P, _P, _P, _P, _P, _P, ctypes.c_int32,
                                             ctypes.c_uint32, ctypes.c_float, _P, _P, _P, _P, _P,
                                             ctypes.c_size_t, _P]),
    "bsa_prepare_kv_ctx": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), ctypes.c_int32, _P, _P, _P,
                                            _P, _P, _P, ctypes.c_uint32, ctypes.c_float, _P,
                                            ctypes.c_size_t, _P]),
    "bsa_attend_ctx": (ctypes.c_int32, [ctypes.POINTER(BsaDesc), ctypes.c_int32, _P, _P, _P, _P,
                                        _P, _P, _P, _P, _P, ctypes.c_int32, ctypes.c_uint32,
                                        ctypes.c_float, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "bsa_partition_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int32, ctypes.c_int32]),
    "bsa_reblock_from_projections": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, _P, _P, _P,
                                                      ctypes.c_size_t, _P]),
    "bsa_tile_layout": (ctypes.c_int32, [ctypes.c_int32] * 7 + [_P, _P]),
    "bsa_check_lists": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                         _P]),
    "bsa_list_status": (ctypes.c_int32, [_P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32), _P]),
    "bsa_topk_from_scores": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P,
                                              _P, _P]),
}

_lib = None


def header_functions() -> list:
    """Names of the functions include/bsattn.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(bsa_\w+)\s*\(", text, re.M)))


def lib():
    """Load libbsattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_video_reblock_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != BSA_OK:
        raise BsaError(status, lib().bsa_last_error().decode())


# ------------------------------------------------------------------------ torch helpers

def _torch():
    import torch
    return torch


def _dev_ptr(t, dtype=None):
    torch = _torch()
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"tensor dtype {t.dtype} != {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def desc_for(x) -> BsaDesc:
    torch = _torch()
    if x.dim() != 3:
        raise ValueError("expected [heads][tokens][head_dim]")
    dt = {torch.bfloat16: BSA_BF16, torch.float32: BSA_F32}.get(x.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {x.dtype}")
    return BsaDesc(x.shape[0], x.shape[1], x.shape[2], dt)


def workspace(desc: BsaDesc, device="cuda"):
    n = lib().bsa_workspace_bytes(ctypes.byref(desc))
    if n == 0:
        raise BsaError(BSA_E_ARG, lib().bsa_last_error().decode() or "invalid descriptor")
    return _torch().empty(n, dtype=_torch().uint8, device=device)


def topk_count(n_blocks: int, ratio: float) -> int:
    return int(lib().bsa_topk_count(n_blocks, ratio))


BSA_LAYOUT_SEPARATE = 0
BSA_LAYOUT_Q_REUSE_K = 1
_LAYOUTS = {"separate": BSA_LAYOUT_SEPARATE, "q_reuse_k": BSA_LAYOUT_Q_REUSE_K}


BSA_POWER_ITERS, BSA_POWER_ITERS_LITE, BSA_TREE_SHARED_DEEP = 8, 2, 1
BSA_DEFAULT_SUBTREE_BLOCKS, BSA_MAX_SUBTREE_BLOCKS, BSA_LITE_SUBTREE_BLOCKS = 8, 64, 64


def tree_flags(shared_deep=False, subtree_blocks=0):
    """Reblock tree flags: the Lite tree's shared subtrees, optionally with their size."""
    if not shared_deep:
        return 0 if not subtree_blocks else (int(subtree_blocks) << 8)
    return BSA_TREE_SHARED_DEEP | (int(subtree_blocks) << 8)


def reblock(q, k, ws=None, with_proj=False, layout="separate", power_iters=BSA_POWER_ITERS,
            shared_deep=False, subtree_blocks=0):
    """(perm_q, perm_k[, proj]) int32 [H][N] (and float [H][2][levels][N]).
    layout "separate" (bsa_reblock) or "q_reuse_k" (perm_q is a copy of the key layout);
    power_iters: power steps per split; shared_deep: one direction per subtree of at most
    subtree_blocks blocks (0: BSA_DEFAULT_SUBTREE_BLOCKS); the Lite reblock is
    power_iters=BSA_POWER_ITERS_LITE, shared_deep=True, subtree_blocks=BSA_LITE_SUBTREE_BLOCKS."""
    torch = _torch()
    if layout not in _LAYOUTS:
        raise BsaError(BSA_E_ARG, f"unknown layout {layout!r}")
    d = desc_for(q)
    ws = workspace(d, q.device) if ws is None else ws
    H, N = q.shape[0], q.shape[1]
    perm_q = torch.empty(H, N, dtype=torch.int32, device=q.device)
    perm_k = torch.empty_like(perm_q)
    levels = max(0, (N // BLOCK - 1).bit_length())
    proj = torch.empty(H, 2, levels, N, dtype=torch.float32, device=q.device) if with_proj else None
    check(lib().bsa_reblock_ex(ctypes.byref(d), _dev_ptr(q, q.dtype), _dev_ptr(k, q.dtype),
                               _LAYOUTS[layout], int(power_iters),
                               tree_flags(shared_deep, subtree_blocks), _dev_ptr(perm_q),
                               _dev_ptr(perm_k), _dev_ptr(proj), _dev_ptr(ws), ws.numel(),
                               _stream()))
    return (perm_q, perm_k, proj) if with_proj else (perm_q, perm_k)


def reblock_side(q, k, side, ws=None, power_iters=BSA_POWER_ITERS, with_proj=False,
                 shared_deep=False, subtree_blocks=0):
    """One side of the reblock: side 0 the query layouts, side 1 the key layouts (int32 [H][N]),
    and with_proj its projections (float [H][2][levels][N], the other side's rows 0)."""
    torch = _torch()
    d = desc_for(q)
    ws = workspace(d, q.device) if ws is None else ws
    H, N = q.shape[0], q.shape[1]
    perm = torch.empty(H, N, dtype=torch.int32, device=q.device)
    levels = max(0, (N // BLOCK - 1).bit_length())
    proj = torch.empty(H, 2, levels, N, dtype=torch.float32, device=q.device) if with_proj \
        else None
    check(lib().bsa_reblock_side(ctypes.byref(d), _dev_ptr(q, q.dtype), _dev_ptr(k, q.dtype),
                                 int(side), int(power_iters),
                                 tree_flags(shared_deep, subtree_blocks), _dev_ptr(perm),
                                 _dev_ptr(proj),
                                 _dev_ptr(ws), ws.numel(), _stream()))
    return (perm, proj) if with_proj else perm


def select(q, k, perm_q, perm_k, topk_ratio=0.0, topk_blocks=0, ws=None, with_scores=False):
    """lists int32 [H][nb][K] (and scores float [H][nb][nb])."""
    torch = _torch()
    d = desc_for(q)
    ws = workspace(d, q.device) if ws is None else ws
    H, nb = q.shape[0], q.shape[1] // BLOCK
    K = topk_blocks if topk_blocks > 0 else topk_count(nb, topk_ratio)
    if K < 1:
        raise BsaError(BSA_E_ARG, f"topk_ratio {topk_ratio} is not in (0, 1]")
    lists = torch.empty(H, nb, K, dtype=torch.int32, device=q.device)
    scores = torch.empty(H, nb, nb, dtype=torch.float32, device=q.device) if with_scores else None
    check(lib().bsa_select(ctypes.byref(d), _dev_ptr(q, q.dtype), _dev_ptr(k, q.dtype),
                           _dev_ptr(perm_q, torch.int32), _dev_ptr(perm_k, torch.int32),
                           float(topk_ratio), int(topk_blocks), _dev_ptr(lists), _dev_ptr(scores),
                           _dev_ptr(ws), ws.numel(), _stream()))
    return (lists, scores) if with_scores else lists


def sparse_attn(q, k, v, perm_q, perm_k, lists, flags=0, scale=0.0, ws=None, with_lse=False,
                out=None):
    torch = _torch()
    d = desc_for(q)
    ws = workspace(d, q.device) if ws is None else ws
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device) \
        if with_lse else None
    check(lib().bsa_sparse_attn(ctypes.byref(d), _dev_ptr(q, q.dtype), _dev_ptr(k, q.dtype),
                                _dev_ptr(v, q.dtype), _dev_ptr(perm_q, torch.int32),
                                _dev_ptr(perm_k, torch.int32), _dev_ptr(lists, torch.int32),
                                int(lists.shape[-1]), int(flags), float(scale),
                                _dev_ptr(o, q.dtype), _dev_ptr(lse), _dev_ptr(ws), ws.numel(),
                                _stream()))
    return (o, lse) if with_lse else o


def workspace_ctx(desc: BsaDesc, n_ctx: int, device="cuda"):
    n = lib().bsa_workspace_bytes_ctx(ctypes.byref(desc), int(n_ctx))
    if n == 0:
        raise BsaError(BSA_E_ARG, "invalid descriptor or context length")
    return _torch().empty(n, dtype=_torch().uint8, device=device)


def sparse_attn_ctx(q, k, v, q_ctx, k_ctx, v_ctx, perm_q, perm_k, lists, flags=0, scale=0.0,
                    ws=None, with_lse=False):
    """Mixed sequence: video q, k, v [H][N][D] (sparse, laid out by perm_q / perm_k and lists)
    and context q_ctx, k_ctx, v_ctx [H][n_ctx][D] (exact).  Returns (o, o_ctx) or, with_lse,
    (o, o_ctx, lse, lse_ctx)."""
    torch = _torch()
    d = desc_for(q)
    H, N, D = q.shape
    n_ctx = q_ctx.shape[1]
    for t in (q_ctx, k_ctx, v_ctx):
        if tuple(t.shape) != (H, n_ctx, D):
            raise ValueError(f"context tensors must be [{H}][n_ctx][{D}], got {tuple(t.shape)}")
    ws = workspace_ctx(d, n_ctx, q.device) if ws is None else ws
    o = torch.empty_like(q)
    o_ctx = torch.empty_like(q_ctx)
    lse = lse_ctx = None
    if with_lse:
        lse = torch.empty(H, N, dtype=torch.float32, device=q.device)
        lse_ctx = torch.empty(H, n_ctx, dtype=torch.float32, device=q.device)
    check(lib().bsa_sparse_attn_ctx(
        ctypes.byref(d), int(n_ctx), _dev_ptr(q, q.dtype), _dev_ptr(k, q.dtype),
        _dev_ptr(v, q.dtype), _dev_ptr(q_ctx, q.dtype), _dev_ptr(k_ctx, q.dtype),
        _dev_ptr(v_ctx, q.dtype), _dev_ptr(perm_q, torch.int32), _dev_ptr(perm_k, torch.int32),
        _dev_ptr(lists, torch.int32), int(lists.shape[-1]), int(flags), float(scale),
        _dev_ptr(o, q.dtype), _dev_ptr(o_ctx, q.dtype), _dev_ptr(lse), _dev_ptr(lse_ctx),
        _dev_ptr(ws), ws.numel(), _stream()))
    return (o, o_ctx, lse, lse_ctx) if with_lse else (o, o_ctx)


def prepare_kv(q, k, v, perm_k, ws, flags=0, scale=0.0):
    """Anchor, summaries and swizzled key/value copies into ws (first phase of sparse_attn)."""
    torch = _torch()
    d = desc_for(q)
    check(lib().bsa_prepare_kv(ctypes.byref(d), _dev_ptr(q, q.dtype), _dev_ptr(k, q.dtype),
                               _dev_ptr(v, q.dtype), _dev_ptr(perm_k, torch.int32), int(flags),
                               float(scale), _dev_ptr(ws), ws.numel(), _stream()))


def attend(q, k, v, perm_q, perm_k, lists, ws, out, flags=0, scale=0.0, lse=None):
    """Attention kernel alone on a ws filled by prepare_kv (second phase of sparse_attn)."""
    torch = _torch()
    d = desc_for(q)
    check(lib().bsa_attend(ctypes.byref(d), _dev_ptr(q, q.dtype), _dev_ptr(k, q.dtype),
                           _dev_ptr(v, q.dtype), _dev_ptr(perm_q, torch.int32),
                           _dev_ptr(perm_k, torch.int32), _dev_ptr(lists, torch.int32),
                           int(lists.shape[-1]), int(flags), float(scale), _dev_ptr(out, q.dtype),
                           _dev_ptr(lse), _dev_ptr(ws), ws.numel(), _stream()))
    return out


def summaries(q, k, v, perm_k, flags=0, scale=0.0, ws=None):
    """fp32 (kt [H][nb][D], vt [H][nb][D], bias [H][nb])."""
    torch = _torch()
    d = desc_for(q)
    ws = workspace(d, q.device) if ws is None else ws
    H, N, D = q.shape
    nb = N // BLOCK
    kt = torch.empty(H, nb, D, dtype=torch.float32, device=q.device)
    vt = torch.empty_like(kt)
    bias = torch.empty(H, nb, dtype=torch.float32, device=q.device)
    check(lib().bsa_summaries(ctypes.byref(d), _dev_ptr(q, q.dtype), _dev_ptr(k, q.dtype),
                              _dev_ptr(v, q.dtype), _dev_ptr(perm_k, torch.int32), int(flags),
                              float(scale), _dev_ptr(kt), _dev_ptr(vt), _dev_ptr(bias),
                              _dev_ptr(ws), ws.numel(), _stream()))
    return kt, vt, bias


def summaries_noalloc(q, k, v, perm_k, flags=0, scale=0.0):
    """bsa_summaries without a workspace (the library's static device scratch):
    fp32 (kt [H][nb][D], vt [H][nb][D], bias [H][nb])."""
    torch = _torch()
    d = desc_for(q)
    H, N, D = q.shape
    nb = N // BLOCK
    kt = torch.empty(H, nb, D, dtype=torch.float32, device=q.device)
    vt = torch.empty_like(kt)
    bias = torch.empty(H, nb, dtype=torch.float32, device=q.device)
    check(lib().bsa_summaries_noalloc(ctypes.byref(d), _dev_ptr(q, q.dtype), _dev_ptr(k, q.dtype),
                                      _dev_ptr(v, q.dtype), _dev_ptr(perm_k, torch.int32),
                                      int(flags), float(scale), _dev_ptr(kt), _dev_ptr(vt),
                                      _dev_ptr(bias), _stream()))
    return kt, vt, bias


def check_lists(lists, n_blocks):
    """bsa_check_lists on int32 lists [..., topk]: (malformed rows, first malformed row or -1)."""
    torch = _torch()
    rows = lists.numel() // lists.shape[-1]
    result = torch.empty(2, dtype=torch.int32, device=lists.device)
    check(lib().bsa_check_lists(int(rows), int(n_blocks), int(lists.shape[-1]),
                                _dev_ptr(lists, torch.int32), _dev_ptr(result), _stream()))
    return tuple(int(x) for x in result.cpu().tolist())


def list_status(ws):
    """bsa_list_status: the list check result of the last BSA_CHECK_LISTS call on ws."""
    out = (ctypes.c_int32 * 2)()
    check(lib().bsa_list_status(_dev_ptr(ws), ws.numel(), out, _stream()))
    return int(out[0]), int(out[1])


def reblock_from_projections(proj):
    """proj float [P][levels][N] (by token id) -> perm int32 [P][N]."""
    torch = _torch()
    P, _, N = proj.shape
    n = lib().bsa_partition_workspace_bytes(P, N)
    if n == 0:
        raise BsaError(BSA_E_ARG, "invalid problem shape")
    ws = torch.empty(n, dtype=torch.uint8, device=proj.device)
    perm = torch.empty(P, N, dtype=torch.int32, device=proj.device)
    check(lib().bsa_reblock_from_projections(P, N, _dev_ptr(proj, torch.float32), _dev_ptr(perm),
                                             _dev_ptr(ws), n, _stream()))
    return perm


def topk_from_scores(scores, topk):
    """scores float [rows][nb] -> lists int32 [rows][topk]."""
    torch = _torch()
    rows, nb = scores.shape
    lists = torch.empty(rows, topk, dtype=torch.int32, device=scores.device)
    check(lib().bsa_topk_from_scores(rows, nb, topk, _dev_ptr(scores, torch.float32),
                                     _dev_ptr(lists), _stream()))
    return lists


def tile_layout(heads, grid, tile=(4, 4, 4), device="cuda"):
    """Fixed-tile layout int32 [heads][T H W] (the positional baseline)."""
    torch = _torch()
    T, H, W = grid
    perm = torch.empty(heads, T * H * W, dtype=torch.int32, device=device)
    check(lib().bsa_tile_layout(heads, T, H, W, *tile, _dev_ptr(perm), _stream()))
    return perm
