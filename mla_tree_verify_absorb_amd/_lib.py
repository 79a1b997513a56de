"""ctypes binding of libddtree.so: the C ABI declared in include/ddtree.h.

Only argument marshalling happens here: torch tensors supply device pointers,
shapes, row strides and the current HIP stream; every step of the path runs in
the library's kernels.  There is no fallback: if the library is not built the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libddtree.so")
_lib = None

DDTREE_OK = 0
DDTREE_ERR_INVALID_ARG = -1
DDTREE_ERR_UNSUPPORTED = -2
DDTREE_ERR_WORKSPACE = -3
DDTREE_ERR_HIP = -4
DDTREE_F32 = 0
DDTREE_BF16 = 1
DDTREE_MAX_NODES = 256
DDTREE_MAX_DEPTH = 64
DDTREE_MAX_PROPOSALS = 64
DDTREE_NOALLOC_SCRATCH_BYTES = 72 << 20

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "ddtree_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ddtree_build_digest": (ctypes.c_char_p, []),
    "ddtree_build_mask": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P, _P, _P, _P]),
    "ddtree_verify_attn_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I64, _I32]),
    "ddtree_verify_attn_auto_splits": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I64]),
    "ddtree_verify_attn": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I64, _P, _I64, _P, _I64,
                                          _P, _I64, _P, _I64, _P, _F32, _I32, _P, _P, _P, _SZ, _P]),
    "ddtree_verify_attn_noalloc": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P, _I64, _P, _I64, _P,
                                                  _I64, _P, _I64, _P, _I64, _P, _F32, _I32, _P, _P, _P]),
    "ddtree_greedy_accept": (ctypes.c_int, [_P, _I64, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "ddtree_compact_kv": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _P, _I64, _P, _I64, _P, _P, _P, _P, _I64, _P,
                                         _I64, _P]),
    "ddtree_build_tree": (ctypes.c_int, [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P]),
    "ddtree_rope_tree": (ctypes.c_int, [_I32, _I32, _I32, _I32, _I32, _P, _P, _I64, _P, _P, _P]),
}


def library_path() -> str:
    return _LIB_PATH


def built_digest(path: str = _LIB_PATH) -> str:
    """The source digest stamped into a built library (loads it under a private handle)."""
    fn = ctypes.CDLL(path).ddtree_build_digest
    fn.restype = ctypes.c_char_p
    return fn().decode()


def is_current(path: str = _LIB_PATH) -> bool:
    """True when the library exists and was built from the sources beside it."""
    from .build import source_digest
    return os.path.exists(path) and built_digest(path) == source_digest()


def lib() -> ctypes.CDLL:
    """Load the in-tree library.  Raises if it is not built, or if it was built from sources other than
    the ones beside it (a stale build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m mla_tree_verify_absorb_amd.build`")
        from .build import source_digest
        handle = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        got, want = handle.ddtree_build_digest().decode(), source_digest()
        if got != want:
            raise RuntimeError(f"{_LIB_PATH} was built from other sources (library digest {got}, sources {want}); "
                               f"rebuild with `python -m mla_tree_verify_absorb_amd.build`")
        _lib = handle
    return _lib


def ddtree_status_string(status: int) -> str:
    return lib().ddtree_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != DDTREE_OK:
        raise RuntimeError(f"{what} failed: {ddtree_status_string(status)} ({status})")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device, stream=None):
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DDTREE_F32
    if t.dtype == torch.bfloat16:
        return DDTREE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _rows_ld(t: torch.Tensor, width: int, name: str) -> int:
    """Row stride (elements) of a 2-D view [rows, >= width] with unit inner stride."""
    if t.dim() == 2 and t.shape[1] == width and t.numel() == 0:
        return width                                   # no rows: the stride is never used
    if t.dim() != 2 or t.shape[1] != width or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name}: expected a [rows, {width}] view with unit inner stride, got {tuple(t.shape)}")
    return t.stride(0) if t.shape[0] > 1 else max(width, t.stride(0))


def _tree_ld(t: torch.Tensor, B: int, N: int, width: int, name: str) -> int:
    """Row stride of a [B, N, width] view whose (b, i) rows are evenly spaced."""
    if t.dim() == 3 and tuple(t.shape) == (B, N, width) and t.numel() == 0:
        return width
    if t.dim() != 3 or tuple(t.shape) != (B, N, width) or (width > 1 and t.stride(2) != 1):
        raise ValueError(f"{name}: expected [{B}, {N}, {width}] with unit inner stride, got {tuple(t.shape)}")
    ld = t.stride(1)
    if B > 1 and t.stride(0) != N * ld:
        raise ValueError(f"{name}: rows of consecutive requests must be evenly spaced")
    return ld if N > 1 or B > 1 else max(width, ld)


# ----------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ----------------------------------------------------------------------------

def ddtree_build_mask(parents: torch.Tensor, prefix_offsets: Optional[torch.Tensor] = None, *,
                      mask: Optional[torch.Tensor] = None, depth: Optional[torch.Tensor] = None,
                      positions: Optional[torch.Tensor] = None, tree_ok: Optional[torch.Tensor] = None,
                      want_positions: bool = True, stream=None):
    """Visibility mask, depth, positions and tree_ok for int32 parents [B, N]."""
    assert parents.dtype == torch.int32 and parents.dim() == 2 and parents.is_contiguous()
    B, N = parents.shape
    dev = parents.device
    W = (N + 31) // 32
    if mask is None:
        mask = torch.empty((B, N, W), dtype=torch.int32, device=dev)     # uint32 bit patterns
    if depth is None:
        depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    if positions is None and want_positions:
        positions = torch.empty((B, N), dtype=torch.int64, device=dev)
    if tree_ok is None:
        tree_ok = torch.empty((B,), dtype=torch.int32, device=dev)
    if prefix_offsets is not None:
        assert prefix_offsets.dtype == torch.int64 and prefix_offsets.numel() == B + 1
    st = lib().ddtree_build_mask(_ptr(parents), B, N, _ptr(prefix_offsets), _ptr(mask), _ptr(depth),
                                 _ptr(positions), _ptr(tree_ok), _stream(dev, stream))
    _check(st, "ddtree_build_mask")
    return mask, depth, positions, tree_ok


def ddtree_verify_attn_workspace_size(dtype_code: int, B: int, N: int, H: int, Dl: int, Dr: int,
                                      max_prefix_len: int, num_splits: int = 0) -> int:
    return int(lib().ddtree_verify_attn_workspace_size(dtype_code, B, N, H, Dl, Dr, max_prefix_len, num_splits))


def ddtree_verify_attn_auto_splits(dtype_code: int, B: int, N: int, H: int, Dl: int, Dr: int,
                                   max_prefix_len: int) -> int:
    return int(lib().ddtree_verify_attn_auto_splits(dtype_code, B, N, H, Dl, Dr, max_prefix_len))


def ddtree_verify_attn(q_lat: torch.Tensor, q_rope: torch.Tensor, ckv: torch.Tensor, krope: torch.Tensor,
                       prefix_offsets: torch.Tensor, max_prefix_len: int, ckv_tree: torch.Tensor,
                       krope_tree: torch.Tensor, mask: torch.Tensor, softmax_scale: float, *,
                       num_splits: int = 0, o: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """Tree-verify attention in absorbed MLA form.

    q_lat [B,N,H,Dl], q_rope [B,N,H,Dr] dense; ckv [T,Dl] / krope [T,Dr] row views of the packed prefix
    cache (may share rows of one fused [T, Dl+Dr] tensor); ckv_tree [B,N,Dl] / krope_tree [B,N,Dr] views;
    mask from ddtree_build_mask.  Returns (o float32 [B,N,H,Dl], lse float32 [B,N,H]).
    """
    B, N, H, Dl = q_lat.shape
    Dr = q_rope.shape[-1]
    assert q_lat.is_contiguous() and q_rope.is_contiguous() and tuple(q_rope.shape[:3]) == (B, N, H)
    code = _dtype_code(q_lat)
    for t in (q_rope, ckv, krope, ckv_tree, krope_tree):
        assert t.dtype == q_lat.dtype, "all latent inputs must share one dtype"
    ld_ckv = _rows_ld(ckv, Dl, "ckv")
    ld_krope = _rows_ld(krope, Dr, "krope")
    ld_ckv_t = _tree_ld(ckv_tree, B, N, Dl, "ckv_tree")
    ld_krope_t = _tree_ld(krope_tree, B, N, Dr, "krope_tree")
    dev = q_lat.device
    if o is None:
        o = torch.empty((B, N, H, Dl), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, N, H), dtype=torch.float32, device=dev)
    need = ddtree_verify_attn_workspace_size(code, B, N, H, Dl, Dr, max_prefix_len, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib().ddtree_verify_attn(code, B, N, H, Dl, Dr, _ptr(q_lat), _ptr(q_rope), _ptr(ckv), ld_ckv, _ptr(krope),
                                  ld_krope, _ptr(prefix_offsets), int(max_prefix_len), _ptr(ckv_tree), ld_ckv_t,
                                  _ptr(krope_tree), ld_krope_t, _ptr(mask), float(softmax_scale), int(num_splits),
                                  _ptr(o), _ptr(lse), _ptr(workspace), ws_bytes, _stream(dev, stream))
    _check(st, "ddtree_verify_attn")
    return o, lse


def ddtree_verify_attn_noalloc(q_lat: torch.Tensor, q_rope: torch.Tensor, ckv: torch.Tensor, krope: torch.Tensor,
                               prefix_offsets: torch.Tensor, max_prefix_len: int, ckv_tree: torch.Tensor,
                               krope_tree: torch.Tensor, mask: torch.Tensor, softmax_scale: float, *,
                               o: torch.Tensor, lse: torch.Tensor, num_splits: int = 0, stream=None):
    """ddtree_verify_attn without a workspace: the library's own per-GPU scratch holds the split partials.
    o and lse are the caller's (nothing is allocated here either)."""
    B, N, H, Dl = q_lat.shape
    Dr = q_rope.shape[-1]
    assert q_lat.is_contiguous() and q_rope.is_contiguous() and tuple(q_rope.shape[:3]) == (B, N, H)
    code = _dtype_code(q_lat)
    for t in (q_rope, ckv, krope, ckv_tree, krope_tree):
        assert t.dtype == q_lat.dtype, "all latent inputs must share one dtype"
    assert o.dtype == torch.float32 and o.is_contiguous() and tuple(o.shape) == (B, N, H, Dl)
    assert lse.dtype == torch.float32 and lse.is_contiguous() and tuple(lse.shape) == (B, N, H)
    st = lib().ddtree_verify_attn_noalloc(code, B, N, H, Dl, Dr, _ptr(q_lat), _ptr(q_rope), _ptr(ckv),
                                          _rows_ld(ckv, Dl, "ckv"), _ptr(krope), _rows_ld(krope, Dr, "krope"),
                                          _ptr(prefix_offsets), int(max_prefix_len), _ptr(ckv_tree),
                                          _tree_ld(ckv_tree, B, N, Dl, "ckv_tree"), _ptr(krope_tree),
                                          _tree_ld(krope_tree, B, N, Dr, "krope_tree"), _ptr(mask),
                                          float(softmax_scale), int(num_splits), _ptr(o), _ptr(lse),
                                          _stream(q_lat.device, stream))
    _check(st, "ddtree_verify_attn_noalloc")
    return o, lse


def ddtree_greedy_accept(logits: torch.Tensor, tokens: torch.Tensor, parents: torch.Tensor, *,
                         target_argmax: Optional[torch.Tensor] = None, accept_len: Optional[torch.Tensor] = None,
                         accept_nodes: Optional[torch.Tensor] = None, commit_tokens: Optional[torch.Tensor] = None,
                         stream=None):
    """Greedy tree accept over float32 logits [B, N, V] (rows may be strided)."""
    assert logits.dtype == torch.float32 and logits.dim() == 3
    B, N, V = logits.shape
    if V > 1 and logits.stride(2) != 1:
        raise ValueError("logits rows must have unit inner stride")
    ld = logits.stride(1) if N > 1 else (logits.stride(0) if B > 1 else V)
    if B > 1 and logits.stride(0) != N * ld:
        raise ValueError("logits rows of consecutive requests must be evenly spaced")
    assert tokens.dtype == torch.int32 and tokens.is_contiguous() and tuple(tokens.shape) == (B, N)
    assert parents.dtype == torch.int32 and parents.is_contiguous() and tuple(parents.shape) == (B, N)
    dev = logits.device
    if target_argmax is None:
        target_argmax = torch.empty((B, N), dtype=torch.int32, device=dev)
    if accept_len is None:
        accept_len = torch.empty((B,), dtype=torch.int32, device=dev)
    if accept_nodes is None:
        accept_nodes = torch.empty((B, N), dtype=torch.int32, device=dev)
    if commit_tokens is None:
        commit_tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    st = lib().ddtree_greedy_accept(_ptr(logits), ld, _ptr(tokens), _ptr(parents), B, N, V, _ptr(target_argmax),
                                    _ptr(accept_len), _ptr(accept_nodes), _ptr(commit_tokens), _stream(dev, stream))
    _check(st, "ddtree_greedy_accept")
    return target_argmax, accept_len, accept_nodes, commit_tokens


def ddtree_compact_kv(ckv_tree: torch.Tensor, krope_tree: torch.Tensor, accept_len: torch.Tensor,
                      accept_nodes: torch.Tensor, dest_rows: torch.Tensor, ckv: torch.Tensor, krope: torch.Tensor, *,
                      stream=None) -> None:
    """Move each request's accepted path rows (root first) to cache rows dest_rows[b] + k, in place.

    ckv_tree [B,N,Dl] / krope_tree [B,N,Dr] views; accept_len int32 [B] and accept_nodes int32 [B,N] from
    ddtree_greedy_accept; dest_rows int64 [B]; ckv [R,Dl] / krope [R,Dr] row views of the cache (updated).
    """
    B, N, Dl = ckv_tree.shape
    Dr = krope_tree.shape[-1]
    code = _dtype_code(ckv_tree)
    for t in (krope_tree, ckv, krope):
        assert t.dtype == ckv_tree.dtype, "tree rows and cache must share one dtype"
    assert accept_len.dtype == torch.int32 and accept_len.is_contiguous() and tuple(accept_len.shape) == (B,)
    assert accept_nodes.dtype == torch.int32 and accept_nodes.is_contiguous() and tuple(accept_nodes.shape) == (B, N)
    assert dest_rows.dtype == torch.int64 and dest_rows.is_contiguous() and tuple(dest_rows.shape) == (B,)
    ld_ct = _tree_ld(ckv_tree, B, N, Dl, "ckv_tree")
    ld_rt = _tree_ld(krope_tree, B, N, Dr, "krope_tree")
    ld_c = _rows_ld(ckv, Dl, "ckv")
    ld_r = _rows_ld(krope, Dr, "krope")
    st = lib().ddtree_compact_kv(code, B, N, Dl, Dr, _ptr(ckv_tree), ld_ct, _ptr(krope_tree), ld_rt, _ptr(accept_len),
                                 _ptr(accept_nodes), _ptr(dest_rows), _ptr(ckv), ld_c, _ptr(krope), ld_r,
                                 _stream(ckv.device, stream))
    _check(st, "ddtree_compact_kv")


def ddtree_build_tree(root_tokens: torch.Tensor, cand_tokens: torch.Tensor, cand_logp: torch.Tensor, N: int, *,
                      parents: Optional[torch.Tensor] = None, tokens: Optional[torch.Tensor] = None,
                      depth: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None, stream=None):
    """Best-first draft trees of N nodes from per-depth proposals cand_tokens / cand_logp [B, D, K].

    Returns (parents int32 [B,N], tokens int32 [B,N], depth int32 [B,N], scores float32 [B,N]).
    """
    B, D, K = cand_tokens.shape
    assert cand_tokens.dtype == torch.int32 and cand_tokens.is_contiguous()
    assert cand_logp.dtype == torch.float32 and cand_logp.is_contiguous() and tuple(cand_logp.shape) == (B, D, K)
    assert root_tokens.dtype == torch.int32 and root_tokens.is_contiguous() and tuple(root_tokens.shape) == (B,)
    dev = cand_tokens.device
    if parents is None:
        parents = torch.empty((B, N), dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if depth is None:
        depth = torch.empty((B, N), dtype=torch.int32, device=dev)
    if scores is None:
        scores = torch.empty((B, N), dtype=torch.float32, device=dev)
    st = lib().ddtree_build_tree(B, int(N), D, K, _ptr(root_tokens), _ptr(cand_tokens), _ptr(cand_logp),
                                 _ptr(parents), _ptr(tokens), _ptr(depth), _ptr(scores), _stream(dev, stream))
    _check(st, "ddtree_build_tree")
    return parents, tokens, depth, scores


def ddtree_rope_tree(q_rope: Optional[torch.Tensor], krope_tree: Optional[torch.Tensor], positions: torch.Tensor,
                     inv_freq: torch.Tensor, *, stream=None) -> None:
    """NeoX rotation, in place, of q_rope [B,N,H,Dr] (dense) and krope_tree [B,N,Dr] rows at positions [B,N]
    (int64) with float64 frequencies inv_freq [Dr/2].  Either array may be None."""
    assert positions.dtype == torch.int64 and positions.is_contiguous() and positions.dim() == 2
    assert inv_freq.dtype == torch.float64 and inv_freq.is_contiguous()
    B, N = positions.shape
    ref = q_rope if q_rope is not None else krope_tree
    Dr = ref.shape[-1]
    H = 1
    if q_rope is not None:
        assert q_rope.is_contiguous() and q_rope.dim() == 4 and tuple(q_rope.shape[:2]) == (B, N)
        H = q_rope.shape[2]
    ld = Dr
    if krope_tree is not None:
        assert krope_tree.dtype == ref.dtype
        ld = _tree_ld(krope_tree, B, N, Dr, "krope_tree")
    assert inv_freq.numel() == Dr // 2
    st = lib().ddtree_rope_tree(_dtype_code(ref), B, N, H, Dr, _ptr(q_rope), _ptr(krope_tree), ld, _ptr(positions),
                                _ptr(inv_freq), _stream(ref.device, stream))
    _check(st, "ddtree_rope_tree")
