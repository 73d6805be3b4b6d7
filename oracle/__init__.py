"""CPU oracle for block top-k sparse decode attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product library never calls it, and it shares
no code with the HIP path: the arithmetic lives in ``oracle.c`` (plain C, double
accumulation, OpenMP over independent units) and this module only marshals
CPU tensors into it.

The method (Pith review of "Kinetics: Rethinking Test-Time Scaling Laws",
section "What carries the argument"): each block of keys is summarised by its
mean key, the query heads of one grouped-query group score every block against
those means, the k best blocks are kept per group, and exact softmax attention
runs over only the kept blocks.  Paging and block = page come from the Kinetics
README (GitLite mirror), section "Benchmark Block TopK Attention throughput".

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force, invariants and library routines; the pages
print no worked numeric example, so values at realistic shapes rest on those pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the loader at a deliberately broken build of oracle.c to show
# that the pins catch the mistake; nothing else sets this.
_LIB_OVERRIDE = os.environ.get("BTK_ORACLE_LIB")

BF16, F32 = 0, 1
_ERRORS = {1: "bad argument", 2: "bad data (table, length or index out of range)",
           3: "out of memory"}


def build(force: bool = True) -> str:
    """Compile ``oracle.c`` into ``liboracle.so`` with gcc and OpenMP."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            _lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB):
                build(force=False)
            _lib = ctypes.CDLL(_LIB)
        i, p, d = ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        _lib.oracle_centroids.argtypes = [i, i, i, i, i, i, i, p, p, p, p, p]
        _lib.oracle_scores.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, d, p]
        _lib.oracle_select.argtypes = [i, i, i, i, p, p, i, p]
        _lib.oracle_attend.argtypes = [i, i, i, i, i, i, i, i, p, p, p, p, p, p, i, d, p, p, p]
        _lib.oracle_round_bf16.argtypes = [p, p, ctypes.c_long]
        _lib.oracle_set_threads.argtypes = [i]
        for fn in (_lib.oracle_centroids, _lib.oracle_scores, _lib.oracle_select,
                   _lib.oracle_attend, _lib.oracle_max_threads, _lib.oracle_abi_version):
            fn.restype = i
    return _lib


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def _cpu(t: torch.Tensor, dtype=None) -> torch.Tensor:
    if t.device.type != "cpu":
        raise ValueError("oracle takes CPU tensors only")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"expected {dtype}, got {t.dtype}")
    return t.contiguous()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _raise(rc: int, what: str) -> None:
    if rc:
        raise RuntimeError(f"oracle {what}: {_ERRORS.get(rc, rc)}")


def centroids(k_cache, block_table, seq_lens, first_pos=None, out=None):
    """Mean key of every touched (page, KV head); returns [num_pages, Hkv, D] float32.

    Pages that are not touched keep the contents of ``out`` (zeros if not given).
    """
    k_cache = _cpu(k_cache)
    num_pages, hkv, page, dim = k_cache.shape
    bt = _cpu(block_table, torch.int32)
    sl = _cpu(seq_lens, torch.int32)
    fp = _cpu(first_pos, torch.int32) if first_pos is not None else None
    if out is None:
        out = torch.zeros(num_pages, hkv, dim, dtype=torch.float32)
    out = _cpu(out, torch.float32)
    rc = lib().oracle_centroids(_dtype_code(k_cache), bt.shape[0], hkv, dim, page, num_pages,
                                bt.shape[1], _ptr(k_cache), _ptr(bt), _ptr(sl), _ptr(fp),
                                _ptr(out))
    _raise(rc, "centroids")
    return out


def scores(q, cents, block_table, seq_lens, page_size=16, sm_scale=0.0):
    """Group block scores [B, Hkv, max_blocks] float32 (NaN where j >= n_b)."""
    q = _cpu(q)
    B, hq, dim = q.shape
    cents = _cpu(cents, torch.float32)
    num_pages, hkv, _ = cents.shape
    bt = _cpu(block_table, torch.int32)
    sl = _cpu(seq_lens, torch.int32)
    out = torch.full((B, hkv, bt.shape[1]), float("nan"), dtype=torch.float32)
    rc = lib().oracle_scores(_dtype_code(q), B, hq, hkv, dim, page_size, num_pages, bt.shape[1],
                             _ptr(q), _ptr(cents), _ptr(bt), _ptr(sl), float(sm_scale), _ptr(out))
    _raise(rc, "scores")
    return out


def select(score, seq_lens, top_k, page_size=16):
    """Top-k block indices [B, Hkv, top_k] int32: ascending, -1 padded."""
    score = _cpu(score, torch.float32)
    B, hkv, max_blocks = score.shape
    sl = _cpu(seq_lens, torch.int32)
    out = torch.empty((B, hkv, top_k), dtype=torch.int32)
    rc = lib().oracle_select(B, hkv, page_size, max_blocks, _ptr(score), _ptr(sl), int(top_k),
                             _ptr(out))
    _raise(rc, "select")
    return out


def attend(q, k_cache, v_cache, block_table, seq_lens, indices=None, sm_scale=0.0,
           want_weights=False):
    """Exact softmax attention over the listed blocks (all blocks if indices is None).

    Returns (out [B,Hq,D] float32, lse [B,Hq] float32, weights or None), where
    weights is float64 [B, Hq, max_blocks*P] at logical token positions.
    """
    q = _cpu(q)
    k_cache = _cpu(k_cache, q.dtype)
    v_cache = _cpu(v_cache, q.dtype)
    B, hq, dim = q.shape
    num_pages, hkv, page, _ = k_cache.shape
    if tuple(v_cache.shape) != (num_pages, hkv, dim, page):
        raise ValueError("v_cache must be [num_pages, Hkv, D, P]")
    bt = _cpu(block_table, torch.int32)
    sl = _cpu(seq_lens, torch.int32)
    idx = _cpu(indices, torch.int32) if indices is not None else None
    top_k = idx.shape[-1] if idx is not None else 0
    out = torch.empty((B, hq, dim), dtype=torch.float32)
    lse = torch.empty((B, hq), dtype=torch.float32)
    w = torch.zeros((B, hq, bt.shape[1] * page), dtype=torch.float64) if want_weights else None
    rc = lib().oracle_attend(_dtype_code(q), B, hq, hkv, dim, page, num_pages, bt.shape[1],
                             _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(sl),
                             _ptr(idx), int(top_k), float(sm_scale), _ptr(out), _ptr(lse), _ptr(w))
    _raise(rc, "attend")
    return out, lse, w


def local_indices(seq_lens, num_kv_heads, window_blocks, page_size=16):
    """The local-window baseline's block lists [B, Hkv, window] int32: the most
    recent min(window, n_b) blocks of each sequence, ascending, -1 padded.
    (scime summary of "Kinetics: Rethinking Test-Time Scaling Law", "Measured
    effects reported in the paper": local attention replaces the top-k selection
    by the most recent KV; here at the same budget of whole blocks.)"""
    sl = [int(x) for x in _cpu(seq_lens, torch.int32)]
    out = torch.full((len(sl), num_kv_heads, window_blocks), -1, dtype=torch.int32)
    for b, L in enumerate(sl):
        nb = (L + page_size - 1) // page_size
        w = min(window_blocks, nb)
        out[b, :, :w] = torch.arange(nb - w, nb, dtype=torch.int32)
    return out


def local_attend(q, k_cache, v_cache, block_table, seq_lens, window_blocks, sm_scale=0.0,
                 want_weights=False):
    """Attention over the local window's blocks (see local_indices): (out, lse, weights)."""
    idx = local_indices(seq_lens, k_cache.shape[1], window_blocks, page_size=k_cache.shape[2])
    return attend(q, k_cache, v_cache, block_table, seq_lens, idx, sm_scale=sm_scale,
                  want_weights=want_weights)


def token_view(k_cache, v_cache, block_table):
    """The same cache seen as one-token pages: (k1 [N*P][Hkv][1][D], v1 [N*P][Hkv][D][1],
    token table [B][max_blocks*P]) with logical token i of sequence b at row
    block_table[b][i // P] * P + i % P.  Layout only, no arithmetic."""
    k_cache, v_cache = _cpu(k_cache), _cpu(v_cache)
    N, hkv, P, D = k_cache.shape
    k1 = k_cache.permute(0, 2, 1, 3).reshape(N * P, hkv, 1, D).contiguous()
    v1 = v_cache.permute(0, 3, 1, 2).reshape(N * P, hkv, D, 1).contiguous()
    bt = _cpu(block_table, torch.int32).to(torch.int64)
    i = torch.arange(bt.shape[1] * P)
    tt = (bt[:, i // P] * P + i % P).to(torch.int32)
    return k1, v1, tt


def token_step(q, k_cache, v_cache, block_table, seq_lens, top_tokens, sm_scale=0.0):
    """Token-level top-k attention, the pages' upper-bound baseline (scime summary
    of "Kinetics: Rethinking Test-Time Scaling Law", "Experimental setup": oracle
    top-k attention; "Limitations": the sparse results use it as an upper bound).

    It is the method with one-token blocks: a one-token block's mean key is the
    key itself, so the group score of token t is (1/r) sum_h scale q_h . k_t, the
    top_tokens best tokens are kept (ties to the lower position) and every head
    attends over exactly those.  Computed by the block functions at page size 1
    on token_view() of the cache.  Returns a dict with scores [B, Hkv, max_tokens],
    indices [B, Hkv, top_tokens] (logical token positions, ascending, -1 padded),
    out and lse.
    """
    k1, v1, tt = token_view(k_cache, v_cache, block_table)
    keys = centroids(k1, tt, seq_lens)
    sc = scores(q, keys, tt, seq_lens, page_size=1, sm_scale=sm_scale)
    idx = select(sc, seq_lens, top_tokens, page_size=1)
    out, lse, _ = attend(q, k1, v1, tt, seq_lens, idx, sm_scale=sm_scale)
    return {"scores": sc, "indices": idx, "out": out, "lse": lse}


def round_bf16(x: torch.Tensor) -> torch.Tensor:
    """float32 -> bfloat16 with round-to-nearest-even (the output rounding)."""
    x = _cpu(x, torch.float32)
    out = torch.empty(x.shape, dtype=torch.int16)
    lib().oracle_round_bf16(_ptr(x), _ptr(out), x.numel())
    return out.view(torch.bfloat16)


def sparse_step(q, k_cache, v_cache, block_table, seq_lens, top_k, cents=None,
                first_pos=None, sm_scale=0.0):
    """One whole decode step of the method: centroids, scores, top-k, attention.

    Returns a dict with centroids, scores, indices, out, lse.
    """
    page = k_cache.shape[2]
    cents = centroids(k_cache, block_table, seq_lens, first_pos=first_pos, out=cents)
    sc = scores(q, cents, block_table, seq_lens, page_size=page, sm_scale=sm_scale)
    idx = select(sc, seq_lens, top_k, page_size=page)
    out, lse, _ = attend(q, k_cache, v_cache, block_table, seq_lens, idx, sm_scale=sm_scale)
    return {"centroids": cents, "scores": sc, "indices": idx, "out": out, "lse": lse}
