"""Python binding of libbtk: block top-k sparse decode attention on MI355X.

Argument marshalling only: every step of the method runs in the HIP kernels of
``libbtk.so`` (built from ``csrc/`` for gfx950 by ``build.py``).  PyTorch
supplies device memory and the current HIP stream.  Importing works without a
GPU; calling a compute function without the built library raises.

The functions carry the names of the C entry points declared in
``include/btk.h`` and take torch tensors laid out as documented there:
  q, out       [B, Hq, D]                 bf16 or fp32
  k_cache      [num_pages, Hkv, 16, D]    token-major pages
  v_cache      [num_pages, Hkv, D, 16]    dim-major pages
  block_table  [B, max_blocks] int32, seq_lens [B] int32
  centroids    [num_pages, Hkv, D] fp32, indices [B, Hkv, top_k] int32
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# BTK_LIB names another build of the same library (the sanitizer test loads a
# host-instrumented one this way); by default the in-tree libbtk.so.
LIB_PATH = os.environ.get("BTK_LIB") or os.path.join(_HERE, "libbtk.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "btk.h")

BTK_OK, BTK_ERR_NULL, BTK_ERR_SHAPE, BTK_ERR_UNSUPPORTED, BTK_ERR_WORKSPACE, BTK_ERR_HIP = range(6)
BTK_BF16, BTK_F32 = 0, 1
PAGE_SIZE = 16


class btk_problem_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float)]


class BtkError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = _lib().btk_status_string(status).decode()
        if status == BTK_ERR_HIP:
            msg += f" (hipError {_lib().btk_last_hip_error()})"
        super().__init__(f"{what}: {msg}")
        self.status = status


_LIB = None


def _lib():
    """Load libbtk.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libbtk.so not built: run `python {os.path.join(_HERE, 'build.py')}`"
                               " (or __graft_entry__.build())")
        lib = ctypes.CDLL(LIB_PATH)
        P, vp, i32, sz = ctypes.POINTER(btk_problem_t), ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        st = ctypes.c_int
        lib.btk_abi_version.restype = ctypes.c_int
        lib.btk_status_string.restype = ctypes.c_char_p
        lib.btk_status_string.argtypes = [st]
        lib.btk_last_hip_error.restype = ctypes.c_int
        lib.btk_workspace_bytes.restype = sz
        lib.btk_workspace_bytes.argtypes = [P, i32]
        lib.btk_centroid_update.restype = st
        lib.btk_centroid_update.argtypes = [P, vp, vp, vp, vp, vp, vp]
        lib.btk_select.restype = st
        lib.btk_select.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        lib.btk_select_shared.restype = st
        lib.btk_select_shared.argtypes = [P, vp, vp, vp, vp, i32, vp, vp, i32, vp, vp, vp, sz, vp]
        lib.btk_sparse_attend.restype = st
        lib.btk_sparse_attend.argtypes = [P, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        lib.btk_dense_attend.restype = st
        lib.btk_dense_attend.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        lib.btk_local_attend.restype = st
        lib.btk_local_attend.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
        lib.btk_token_workspace_bytes.restype = sz
        lib.btk_token_workspace_bytes.argtypes = [P, i32]
        lib.btk_token_topk_attend.restype = st
        lib.btk_token_topk_attend.argtypes = [P, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        lib.btk_decode_step.restype = st
        lib.btk_decode_step.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
        lib.btk_decode_step_sketch.restype = st
        lib.btk_decode_step_sketch.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, i32, vp, vp,
                                               vp, vp, vp, sz, vp]
        lib.btk_decode_step_noalloc.restype = st
        lib.btk_decode_step_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp]
        lib.btk_decode_step_append.restype = st
        lib.btk_decode_step_append.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp,
                                               vp, sz, vp]
        lib.btk_sketch_bytes.restype = sz
        lib.btk_sketch_bytes.argtypes = [P]
        lib.btk_sketch_update.restype = st
        lib.btk_sketch_update.argtypes = [P, vp, vp, vp, vp, vp, sz, vp, sz, vp]
        lib.btk_select_sketch.restype = st
        lib.btk_select_sketch.argtypes = [P, vp, vp, vp, sz, vp, vp, i32, vp, vp, sz, vp]
        lib.btk_probe_row_read.restype = st
        lib.btk_probe_row_read.argtypes = [vp, sz, vp, ctypes.c_int64, vp, vp]
        _LIB = lib
    return _LIB


def header_symbols() -> list[str]:
    """Names of the functions declared in include/btk.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(btk_[a-z_]+)\s*\(", text)))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BTK_BF16
    if t.dtype == torch.float32:
        return BTK_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def make_problem(q: torch.Tensor, k_cache: torch.Tensor, block_table: torch.Tensor,
                 sm_scale: float = 0.0) -> btk_problem_t:
    B, hq, dim = q.shape
    num_pages, hkv, page, kd = k_cache.shape
    if kd != dim:
        raise ValueError("q and k_cache head_dim differ")
    return btk_problem_t(B, hq, hkv, dim, page, num_pages, block_table.shape[1], _dtype_code(q),
                         float(sm_scale))


def btk_workspace_bytes(problem: btk_problem_t, top_k: int) -> int:
    return int(_lib().btk_workspace_bytes(ctypes.byref(problem), int(top_k)))


def new_workspace(problem: btk_problem_t, top_k: int, device) -> torch.Tensor:
    """A zero-filled workspace tensor of btk_workspace_bytes(problem, top_k) bytes."""
    n = btk_workspace_bytes(problem, top_k)
    if n == 0:
        raise ValueError("invalid problem for this library build")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def workspace_error_bits(workspace: torch.Tensor) -> int:
    """Sticky error bits that kernels set for out-of-range device inputs."""
    return int(workspace[:4].view(torch.int32).item())


# workspace word 0, as include/btk.h defines it
ERROR_BITS = {1: "sequence length out of range", 2: "page id out of range",
              4: "block index out of range", 8: "decode-step wait gave up",
              16: "declared shared prefix differs between members"}


class BtkDeviceError(RuntimeError):
    """Raised by check_workspace when a kernel flagged an input or a wait."""

    def __init__(self, bits: int, what: str):
        names = [n for b, n in ERROR_BITS.items() if bits & b] or [f"bits {bits:#x}"]
        super().__init__(f"{what}: device error bits {bits:#x} ({'; '.join(names)})")
        self.bits = bits


def check_workspace(workspace: torch.Tensor, what: str = "btk") -> None:
    """Waits for the workspace's device (a synchronisation) and raises
    BtkDeviceError if any error bit is set (the bits are sticky: clear word 0 to
    reuse the workspace after an error)."""
    bits = workspace_error_bits(workspace)
    if bits:
        raise BtkDeviceError(bits, what)


def _dev(t: torch.Tensor, name: str, dtype=None, device=None) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    return t.data_ptr()


def _expect(t: Optional[torch.Tensor], name: str, shape) -> None:
    if t is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _check_shapes(p: btk_problem_t, q=None, k_cache=None, v_cache=None, block_table=None,
                  seq_lens=None, centroids=None, indices=None, out=None, lse=None, scores=None,
                  first_pos=None, top_k=None) -> None:
    """The C ABI cannot see device buffer sizes: check every tensor against the problem."""
    B, hq, hkv, D, P = p.batch, p.num_q_heads, p.num_kv_heads, p.head_dim, p.page_size
    _expect(q, "q", (B, hq, D))
    _expect(out, "out", (B, hq, D))
    _expect(k_cache, "k_cache", (p.num_pages, hkv, P, D))
    _expect(v_cache, "v_cache", (p.num_pages, hkv, D, P))
    _expect(block_table, "block_table", (B, p.max_blocks_per_seq))
    _expect(seq_lens, "seq_lens", (B,))
    _expect(first_pos, "first_pos", (B,))
    _expect(centroids, "centroids", (p.num_pages, hkv, D))
    _expect(lse, "lse", (B, hq))
    _expect(scores, "scores", (B, hkv, p.max_blocks_per_seq))
    if indices is not None:
        _expect(indices, "indices", (B, hkv, top_k if top_k is not None else indices.shape[-1]))


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _check(status: int, what: str) -> None:
    if status != BTK_OK:
        raise BtkError(status, what)


def btk_centroid_update(k_cache, block_table, seq_lens, centroids, first_pos=None,
                        problem: Optional[btk_problem_t] = None, q_heads: Optional[int] = None):
    """S1: recompute centroids of the touched pages (all pages if first_pos is None)."""
    dev = k_cache.device
    if problem is None:
        num_pages, hkv, page, dim = k_cache.shape
        problem = btk_problem_t(block_table.shape[0], q_heads or hkv, hkv, dim, page, num_pages,
                                block_table.shape[1], _dtype_code(k_cache), 0.0)
    _check_shapes(problem, k_cache=k_cache, block_table=block_table, seq_lens=seq_lens,
                  centroids=centroids, first_pos=first_pos)
    fp = _dev(first_pos, "first_pos", torch.int32, dev) if first_pos is not None else None
    st = _lib().btk_centroid_update(ctypes.byref(problem), _dev(k_cache, "k_cache", None, dev),
                                    _dev(block_table, "block_table", torch.int32, dev),
                                    _dev(seq_lens, "seq_lens", torch.int32, dev), fp,
                                    _dev(centroids, "centroids", torch.float32, dev), _stream(dev))
    _check(st, "btk_centroid_update")
    return centroids


def btk_select(q, centroids, block_table, seq_lens, top_k, workspace, indices=None, scores=None,
               sm_scale: float = 0.0, problem: Optional[btk_problem_t] = None):
    """S2+S3: group block scores and top-k block indices [B, Hkv, top_k] int32."""
    dev = q.device
    if problem is None:
        num_pages, hkv, dim = centroids.shape
        problem = btk_problem_t(q.shape[0], q.shape[1], hkv, dim, PAGE_SIZE, num_pages,
                                block_table.shape[1], _dtype_code(q), float(sm_scale))
    if indices is None:
        indices = torch.empty((problem.batch, problem.num_kv_heads, int(top_k)), dtype=torch.int32,
                              device=dev)
    _check_shapes(problem, q=q, block_table=block_table, seq_lens=seq_lens, centroids=centroids,
                  indices=indices, scores=scores, top_k=top_k)
    sp = _dev(scores, "scores", torch.float32, dev) if scores is not None else None
    st = _lib().btk_select(ctypes.byref(problem), _dev(q, "q", None, dev),
                           _dev(centroids, "centroids", torch.float32, dev),
                           _dev(block_table, "block_table", torch.int32, dev),
                           _dev(seq_lens, "seq_lens", torch.int32, dev), int(top_k),
                           _dev(indices, "indices", torch.int32, dev), sp,
                           _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(),
                           _stream(dev))
    _check(st, "btk_select")
    return indices


def new_sketch(problem: btk_problem_t, device) -> torch.Tensor:
    """A zero-filled sketch buffer for the problem (no row is usable until
    btk_sketch_update has written it)."""
    n = int(_lib().btk_sketch_bytes(ctypes.byref(problem)))
    if n == 0:
        raise ValueError("invalid problem for a sketch")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def btk_sketch_update(centroids, block_table, seq_lens, sketch, workspace, first_pos=None,
                      problem: Optional[btk_problem_t] = None, q=None, k_cache=None):
    """Writes the sketch rows of the blocks touched since first_pos (all when None)
    from the fp32 centroids.  problem (or q and k_cache to build it) is required."""
    dev = centroids.device
    if problem is None:
        problem = make_problem(q, k_cache, block_table)
    _check_shapes(problem, block_table=block_table, seq_lens=seq_lens, centroids=centroids,
                  first_pos=first_pos)
    fp = _dev(first_pos, "first_pos", torch.int32, dev) if first_pos is not None else None
    st = _lib().btk_sketch_update(ctypes.byref(problem), _dev(centroids, "centroids", torch.float32, dev),
                                  _dev(block_table, "block_table", torch.int32, dev),
                                  _dev(seq_lens, "seq_lens", torch.int32, dev), fp,
                                  _dev(sketch, "sketch", torch.uint8, dev), sketch.numel(),
                                  _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(),
                                  _stream(dev))
    _check(st, "btk_sketch_update")


def btk_select_sketch(q, centroids, sketch, block_table, seq_lens, top_k, workspace, indices=None,
                      sm_scale: float = 0.0, problem: Optional[btk_problem_t] = None,
                      k_cache=None):
    """S2 + S3 through the sketch; the indices equal btk_select's."""
    dev = q.device
    if problem is None:
        problem = make_problem(q, k_cache, block_table, sm_scale)
    if indices is None:
        indices = torch.empty((problem.batch, problem.num_kv_heads, int(top_k)), dtype=torch.int32,
                              device=dev)
    _check_shapes(problem, q=q, block_table=block_table, seq_lens=seq_lens, centroids=centroids,
                  indices=indices, top_k=top_k)
    st = _lib().btk_select_sketch(ctypes.byref(problem), _dev(q, "q", None, dev),
                                  _dev(centroids, "centroids", torch.float32, dev),
                                  _dev(sketch, "sketch", torch.uint8, dev), sketch.numel(),
                                  _dev(block_table, "block_table", torch.int32, dev),
                                  _dev(seq_lens, "seq_lens", torch.int32, dev), int(top_k),
                                  _dev(indices, "indices", torch.int32, dev),
                                  _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(),
                                  _stream(dev))
    _check(st, "btk_select_sketch")
    return indices


def btk_select_shared(q, centroids, block_table, seq_lens, group_start, prefix_blocks, top_k,
                      workspace, indices=None, scores=None, sm_scale: float = 0.0,
                      problem: Optional[btk_problem_t] = None):
    """S2+S3 reading each group's shared prefix once; group_start (num_groups + 1)
    and prefix_blocks (num_groups) are host sequences of ints.  Returns indices."""
    dev = q.device
    if problem is None:
        num_pages, hkv, dim = centroids.shape
        problem = btk_problem_t(q.shape[0], q.shape[1], hkv, dim, PAGE_SIZE, num_pages,
                                block_table.shape[1], _dtype_code(q), float(sm_scale))
    if indices is None:
        indices = torch.empty((problem.batch, problem.num_kv_heads, int(top_k)), dtype=torch.int32,
                              device=dev)
    _check_shapes(problem, q=q, block_table=block_table, seq_lens=seq_lens, centroids=centroids,
                  indices=indices, scores=scores, top_k=top_k)
    gs = (ctypes.c_int32 * len(group_start))(*[int(x) for x in group_start])
    pb = (ctypes.c_int32 * len(prefix_blocks))(*[int(x) for x in prefix_blocks])
    sp = _dev(scores, "scores", torch.float32, dev) if scores is not None else None
    st = _lib().btk_select_shared(ctypes.byref(problem), _dev(q, "q", None, dev),
                                  _dev(centroids, "centroids", torch.float32, dev),
                                  _dev(block_table, "block_table", torch.int32, dev),
                                  _dev(seq_lens, "seq_lens", torch.int32, dev),
                                  len(prefix_blocks), ctypes.cast(gs, ctypes.c_void_p),
                                  ctypes.cast(pb, ctypes.c_void_p), int(top_k),
                                  _dev(indices, "indices", torch.int32, dev), sp,
                                  _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(),
                                  _stream(dev))
    _check(st, "btk_select_shared")
    return indices


def btk_sparse_attend(q, k_cache, v_cache, block_table, seq_lens, indices, workspace, out=None,
                      lse=None, sm_scale: float = 0.0, problem: Optional[btk_problem_t] = None):
    """S4: exact softmax attention over the listed blocks; returns out [B, Hq, D]."""
    dev = q.device
    problem = problem or make_problem(q, k_cache, block_table, sm_scale)
    out = torch.empty_like(q) if out is None else out
    _check_shapes(problem, q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                  seq_lens=seq_lens, indices=indices, out=out, lse=lse)
    lp = _dev(lse, "lse", torch.float32, dev) if lse is not None else None
    st = _lib().btk_sparse_attend(ctypes.byref(problem), _dev(q, "q", None, dev),
                                  _dev(k_cache, "k_cache", q.dtype, dev),
                                  _dev(v_cache, "v_cache", q.dtype, dev),
                                  _dev(block_table, "block_table", torch.int32, dev),
                                  _dev(seq_lens, "seq_lens", torch.int32, dev),
                                  _dev(indices, "indices", torch.int32, dev), indices.shape[-1],
                                  _dev(out, "out", q.dtype, dev), lp,
                                  _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(),
                                  _stream(dev))
    _check(st, "btk_sparse_attend")
    return out


def btk_dense_attend(q, k_cache, v_cache, block_table, seq_lens, workspace, out=None, lse=None,
                     sm_scale: float = 0.0, problem: Optional[btk_problem_t] = None):
    """S5: dense paged decode attention over every block; returns out [B, Hq, D]."""
    dev = q.device
    problem = problem or make_problem(q, k_cache, block_table, sm_scale)
    out = torch.empty_like(q) if out is None else out
    _check_shapes(problem, q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                  seq_lens=seq_lens, out=out, lse=lse)
    lp = _dev(lse, "lse", torch.float32, dev) if lse is not None else None
    st = _lib().btk_dense_attend(ctypes.byref(problem), _dev(q, "q", None, dev),
                                 _dev(k_cache, "k_cache", q.dtype, dev),
                                 _dev(v_cache, "v_cache", q.dtype, dev),
                                 _dev(block_table, "block_table", torch.int32, dev),
                                 _dev(seq_lens, "seq_lens", torch.int32, dev),
                                 _dev(out, "out", q.dtype, dev), lp,
                                 _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(),
                                 _stream(dev))
    _check(st, "btk_dense_attend")
    return out


def btk_local_attend(q, k_cache, v_cache, block_table, seq_lens, window_blocks, workspace,
                     out=None, lse=None, sm_scale: float = 0.0,
                     problem: Optional[btk_problem_t] = None):
    """Local-window baseline: attention over the most recent min(window_blocks, n_b)
    blocks of each sequence; returns out [B, Hq, D]."""
    dev = q.device
    problem = problem or make_problem(q, k_cache, block_table, sm_scale)
    out = torch.empty_like(q) if out is None else out
    _check_shapes(problem, q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                  seq_lens=seq_lens, out=out, lse=lse)
    lp = _dev(lse, "lse", torch.float32, dev) if lse is not None else None
    st = _lib().btk_local_attend(ctypes.byref(problem), _dev(q, "q", None, dev),
                                 _dev(k_cache, "k_cache", q.dtype, dev),
                                 _dev(v_cache, "v_cache", q.dtype, dev),
                                 _dev(block_table, "block_table", torch.int32, dev),
                                 _dev(seq_lens, "seq_lens", torch.int32, dev), int(window_blocks),
                                 _dev(out, "out", q.dtype, dev), lp,
                                 _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(),
                                 _stream(dev))
    _check(st, "btk_local_attend")
    return out


def btk_token_workspace_bytes(problem: btk_problem_t, top_tokens: int) -> int:
    return int(_lib().btk_token_workspace_bytes(ctypes.byref(problem), int(top_tokens)))


def new_token_workspace(problem: btk_problem_t, top_tokens: int, device) -> torch.Tensor:
    """A zero-filled workspace for btk_token_topk_attend."""
    n = btk_token_workspace_bytes(problem, top_tokens)
    if n == 0:
        raise ValueError("invalid problem or top_tokens for this library build")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def btk_token_topk_attend(q, k_cache, v_cache, block_table, seq_lens, top_tokens, workspace,
                          token_indices=None, out=None, lse=None, sm_scale: float = 0.0,
                          problem: Optional[btk_problem_t] = None):
    """Token-level top-k baseline; returns (out [B, Hq, D], token_indices or None)."""
    dev = q.device
    problem = problem or make_problem(q, k_cache, block_table, sm_scale)
    out = torch.empty_like(q) if out is None else out
    _check_shapes(problem, q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                  seq_lens=seq_lens, out=out, lse=lse)
    if token_indices is not None and tuple(token_indices.shape) != (
            problem.batch, problem.num_kv_heads, int(top_tokens)):
        raise ValueError("token_indices must be [B, Hkv, top_tokens]")
    ti = _dev(token_indices, "token_indices", torch.int32, dev) if token_indices is not None else None
    lp = _dev(lse, "lse", torch.float32, dev) if lse is not None else None
    st = _lib().btk_token_topk_attend(ctypes.byref(problem), _dev(q, "q", None, dev),
                                      _dev(k_cache, "k_cache", q.dtype, dev),
                                      _dev(v_cache, "v_cache", q.dtype, dev),
                                      _dev(block_table, "block_table", torch.int32, dev),
                                      _dev(seq_lens, "seq_lens", torch.int32, dev),
                                      int(top_tokens), ti, _dev(out, "out", q.dtype, dev), lp,
                                      _dev(workspace, "workspace", torch.uint8, dev),
                                      workspace.numel(), _stream(dev))
    _check(st, "btk_token_topk_attend")
    return out, token_indices


def btk_decode_step(q, k_cache, v_cache, block_table, seq_lens, centroids, top_k, workspace,
                    first_pos=None, indices=None, out=None, lse=None, sm_scale: float = 0.0,
                    problem: Optional[btk_problem_t] = None, check: bool = False):
    """S1 (touched pages) + S2 + S3 + S4 in one launch; returns (out, indices).
    check=True synchronises and raises BtkDeviceError if the launch set an error
    bit (an out-of-range input, or bit 8: a wait that gave up)."""
    dev = q.device
    problem = problem or make_problem(q, k_cache, block_table, sm_scale)
    out = torch.empty_like(q) if out is None else out
    if indices is None:
        indices = torch.empty((problem.batch, problem.num_kv_heads, int(top_k)), dtype=torch.int32,
                              device=dev)
    _check_shapes(problem, q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                  seq_lens=seq_lens, centroids=centroids, indices=indices, out=out, lse=lse,
                  first_pos=first_pos, top_k=top_k)
    fp = _dev(first_pos, "first_pos", torch.int32, dev) if first_pos is not None else None
    lp = _dev(lse, "lse", torch.float32, dev) if lse is not None else None
    st = _lib().btk_decode_step(ctypes.byref(problem), _dev(q, "q", None, dev),
                                _dev(k_cache, "k_cache", q.dtype, dev),
                                _dev(v_cache, "v_cache", q.dtype, dev),
                                _dev(block_table, "block_table", torch.int32, dev),
                                _dev(seq_lens, "seq_lens", torch.int32, dev), fp,
                                _dev(centroids, "centroids", torch.float32, dev), int(top_k),
                                _dev(indices, "indices", torch.int32, dev),
                                _dev(out, "out", q.dtype, dev), lp,
                                _dev(workspace, "workspace", torch.uint8, dev), workspace.numel(),
                                _stream(dev))
    _check(st, "btk_decode_step")
    if check:
        check_workspace(workspace, "btk_decode_step")
    return out, indices


def btk_decode_step_sketch(q, k_cache, v_cache, block_table, seq_lens, centroids, sketch, top_k,
                           workspace, first_pos=None, indices=None, out=None, lse=None,
                           cand_counts=None, sm_scale: float = 0.0,
                           problem: Optional[btk_problem_t] = None, check: bool = False):
    """btk_decode_step through the block sketch (results identical); the touched
    blocks' sketch rows are rebuilt in the call.  cand_counts ([B, Hkv] int32) receives
    per unit the number of blocks scored from their fp32 rows.  Returns (out, indices)."""
    dev = q.device
    problem = problem or make_problem(q, k_cache, block_table, sm_scale)
    out = torch.empty_like(q) if out is None else out
    if indices is None:
        indices = torch.empty((problem.batch, problem.num_kv_heads, int(top_k)), dtype=torch.int32,
                              device=dev)
    _check_shapes(problem, q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                  seq_lens=seq_lens, centroids=centroids, indices=indices, out=out, lse=lse,
                  first_pos=first_pos, top_k=top_k)
    if cand_counts is not None and tuple(cand_counts.shape) != (problem.batch, problem.num_kv_heads):
        raise ValueError(f"cand_counts: expected shape {(problem.batch, problem.num_kv_heads)}, "
                         f"got {tuple(cand_counts.shape)}")
    fp = _dev(first_pos, "first_pos", torch.int32, dev) if first_pos is not None else None
    lp = _dev(lse, "lse", torch.float32, dev) if lse is not None else None
    cc = _dev(cand_counts, "cand_counts", torch.int32, dev) if cand_counts is not None else None
    st = _lib().btk_decode_step_sketch(ctypes.byref(problem), _dev(q, "q", None, dev),
                                       _dev(k_cache, "k_cache", q.dtype, dev),
                                       _dev(v_cache, "v_cache", q.dtype, dev),
                                       _dev(block_table, "block_table", torch.int32, dev),
                                       _dev(seq_lens, "seq_lens", torch.int32, dev), fp,
                                       _dev(centroids, "centroids", torch.float32, dev),
                                       _dev(sketch, "sketch", torch.uint8, dev), sketch.numel(),
                                       int(top_k), _dev(indices, "indices", torch.int32, dev),
                                       _dev(out, "out", q.dtype, dev), lp, cc,
                                       _dev(workspace, "workspace", torch.uint8, dev),
                                       workspace.numel(), _stream(dev))
    _check(st, "btk_decode_step_sketch")
    if check:
        check_workspace(workspace, "btk_decode_step_sketch")
    return out, indices


def btk_decode_step_noalloc(q, k_cache, v_cache, block_table, seq_lens, centroids, top_k,
                            first_pos=None, indices=None, out=None, lse=None, sm_scale: float = 0.0,
                            problem: Optional[btk_problem_t] = None):
    """btk_decode_step with the library's own per-GPU scratch instead of a workspace
    (the output tensors are allocated here unless given); returns (out, indices)."""
    dev = q.device
    problem = problem or make_problem(q, k_cache, block_table, sm_scale)
    out = torch.empty_like(q) if out is None else out
    if indices is None:
        indices = torch.empty((problem.batch, problem.num_kv_heads, int(top_k)), dtype=torch.int32,
                              device=dev)
    _check_shapes(problem, q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                  seq_lens=seq_lens, centroids=centroids, indices=indices, out=out, lse=lse,
                  first_pos=first_pos, top_k=top_k)
    fp = _dev(first_pos, "first_pos", torch.int32, dev) if first_pos is not None else None
    lp = _dev(lse, "lse", torch.float32, dev) if lse is not None else None
    st = _lib().btk_decode_step_noalloc(ctypes.byref(problem), _dev(q, "q", None, dev),
                                        _dev(k_cache, "k_cache", q.dtype, dev),
                                        _dev(v_cache, "v_cache", q.dtype, dev),
                                        _dev(block_table, "block_table", torch.int32, dev),
                                        _dev(seq_lens, "seq_lens", torch.int32, dev), fp,
                                        _dev(centroids, "centroids", torch.float32, dev),
                                        int(top_k), _dev(indices, "indices", torch.int32, dev),
                                        _dev(out, "out", q.dtype, dev), lp, _stream(dev))
    _check(st, "btk_decode_step_noalloc")
    return out, indices


def btk_probe_row_read(src, rows=None, row_ids=None, sink=None):
    """Counter-calibration read of 512-byte rows of ``src`` (a device tensor),
    in order (``rows`` of them) or at ``row_ids`` (int32); computes nothing."""
    dev = src.device
    nbytes = src.numel() * src.element_size()
    if row_ids is not None:
        rows = row_ids.numel()
    elif rows is None:
        rows = nbytes // 512
    sink = torch.zeros(1, dtype=torch.int32, device=dev) if sink is None else sink
    rp = _dev(row_ids, "row_ids", torch.int32, dev) if row_ids is not None else None
    st = _lib().btk_probe_row_read(_dev(src, "src", None, dev), nbytes, rp, int(rows),
                                   _dev(sink, "sink", None, dev), _stream(dev))
    _check(st, "btk_probe_row_read")


def btk_decode_step_append(q, k_new, v_new, k_cache, v_cache, block_table, seq_lens, centroids,
                           top_k, workspace, indices=None, out=None, lse=None, sm_scale: float = 0.0,
                           problem: Optional[btk_problem_t] = None, check: bool = False):
    """The decode step with the KV append fused in: k_new / v_new [B, Hkv, D] are written
    into the caches at position seq_lens - 1, then S1 + S2 + S3 + S4; returns (out, indices).
    check: as btk_decode_step."""
    dev = q.device
    problem = problem or make_problem(q, k_cache, block_table, sm_scale)
    out = torch.empty_like(q) if out is None else out
    if indices is None:
        indices = torch.empty((problem.batch, problem.num_kv_heads, int(top_k)), dtype=torch.int32,
                              device=dev)
    _check_shapes(problem, q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                  seq_lens=seq_lens, centroids=centroids, indices=indices, out=out, lse=lse,
                  top_k=top_k)
    tok = (problem.batch, problem.num_kv_heads, problem.head_dim)
    _expect(k_new, "k_new", tok)
    _expect(v_new, "v_new", tok)
    lp = _dev(lse, "lse", torch.float32, dev) if lse is not None else None
    st = _lib().btk_decode_step_append(ctypes.byref(problem), _dev(q, "q", None, dev),
                                       _dev(k_new, "k_new", q.dtype, dev),
                                       _dev(v_new, "v_new", q.dtype, dev),
                                       _dev(k_cache, "k_cache", q.dtype, dev),
                                       _dev(v_cache, "v_cache", q.dtype, dev),
                                       _dev(block_table, "block_table", torch.int32, dev),
                                       _dev(seq_lens, "seq_lens", torch.int32, dev),
                                       _dev(centroids, "centroids", torch.float32, dev),
                                       int(top_k), _dev(indices, "indices", torch.int32, dev),
                                       _dev(out, "out", q.dtype, dev), lp,
                                       _dev(workspace, "workspace", torch.uint8, dev),
                                       workspace.numel(), _stream(dev))
    _check(st, "btk_decode_step_append")
    if check:
        check_workspace(workspace, "btk_decode_step_append")
    return out, indices


def sparse_decode_step(q, k_cache, v_cache, block_table, seq_lens, centroids, top_k, workspace,
                       first_pos=None, out=None, indices=None, lse=None, scores=None,
                       sm_scale: float = 0.0, problem: Optional[btk_problem_t] = None,
                       check: bool = False):
    """One decode step of the method: S1 (touched pages), S2+S3, S4, all on the current stream.
    check: as btk_decode_step."""
    problem = problem or make_problem(q, k_cache, block_table, sm_scale)
    btk_centroid_update(k_cache, block_table, seq_lens, centroids, first_pos, problem=problem)
    indices = btk_select(q, centroids, block_table, seq_lens, top_k, workspace,
                         indices=indices, scores=scores, problem=problem)
    out = btk_sparse_attend(q, k_cache, v_cache, block_table, seq_lens, indices, workspace,
                            out=out, lse=lse, problem=problem)
    if check:
        check_workspace(workspace, "sparse_decode_step")
    return out, indices
