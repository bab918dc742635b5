"""ctypes binding to libtreewy.so: the C ABI under the same names, plus small
allocating conveniences.  Argument marshalling only -- every step of the path
runs in the library's HIP kernels; torch supplies device memory and streams.

Loading fails loudly if the library has not been built (there is no fallback).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

# TREEWY_LIB names another build of the library to load instead (the
# host-layer sanitizer build of the test suite uses it)
LIB_PATH = os.environ.get("TREEWY_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                        "libtreewy.so")

TREEWY_OK = 0
TREEWY_ERR_ARG = -1
TREEWY_ERR_TREE = -2
TREEWY_ERR_ALIGN = -3
TREEWY_ERR_DTYPE = -4
TREEWY_ERR_LAUNCH = -5
TREEWY_ERR_SIZE = -6
TREEWY_BF16 = 0
TREEWY_F32 = 1
D = 128
MAX_NODES = 64

EXPORTS = ("treewy_tree_meta", "treewy_verify", "treewy_commit", "treewy_commit_verify",
           "treewy_commit_verify_pool", "treewy_commit_verify_bf16state", "treewy_prefill_chain",
           "treewy_prefill", "treewy_tree_desc_size", "treewy_tree_desc_pack",
           "treewy_commit_verify_pool_trees", "treewy_prefill_chain_noalloc",
           "treewy_commit_verify_bf16state_pool", "treewy_commit_verify_bf16state_pool_trees",
           "treewy_store_all", "treewy_store_all_select",
           "treewy_status_str")

_lib = None


class TreewyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """Load the built library once (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        # torch ships its own HIP runtime under the same soname as the system
        # one the library links; whichever is loaded first serves both.  Load
        # torch first, so that the library and torch share torch's runtime
        # (the library loaded first made torch and the library's launches
        # run on a mixed runtime, and launches failed).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p
        pi32 = ctypes.POINTER(ctypes.c_int32)
        L.treewy_tree_meta.argtypes = [pi32, i32, pi32, ctypes.POINTER(ctypes.c_uint64)]
        L.treewy_verify.argtypes = [vp, vp, vp, vp, vp, vp, pi32, i32, i32, i32, vp, vp, vp, i32, st]
        L.treewy_commit.argtypes = [vp, vp, vp, vp, vp, pi32, i32, i32, i32, vp, i32, st]
        L.treewy_commit_verify.argtypes = [vp, vp, vp, vp, vp, vp, pi32, i32, vp, vp, vp, vp, vp,
                                           pi32, i32, i32, i32, vp, vp, vp, i32, st]
        L.treewy_commit_verify_pool.argtypes = [vp, i32, vp, vp, vp, vp, vp, pi32, i32, vp, vp, vp,
                                                vp, vp, pi32, i32, i32, i32, vp, vp, vp, i32, st]
        L.treewy_commit_verify_bf16state.argtypes = L.treewy_commit_verify.argtypes
        L.treewy_prefill_chain.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp, vp, vp,
                                           i32, st]
        L.treewy_prefill_chain_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, vp,
                                                   i32, st]
        L.treewy_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, vp, i32, st]
        L.treewy_tree_desc_size.argtypes = []
        L.treewy_tree_desc_pack.argtypes = [pi32, pi32, i32, i32, vp, ctypes.POINTER(ctypes.c_int)]
        L.treewy_commit_verify_pool_trees.argtypes = [vp, i32, vp, vp, vp, vp, vp, vp, i32, i32, vp,
                                                      vp, vp, vp, vp, vp, i32, i32, i32, i32, vp,
                                                      vp, vp, i32, st]
        L.treewy_commit_verify_bf16state_pool.argtypes = L.treewy_commit_verify_pool.argtypes
        L.treewy_commit_verify_bf16state_pool_trees.argtypes = L.treewy_commit_verify_pool_trees.argtypes
        L.treewy_store_all.argtypes = [vp, vp, vp, vp, vp, vp, pi32, i32, i32, i32, vp, vp, i32, st]
        L.treewy_store_all_select.argtypes = [vp, vp, i32, i32, i32, vp, st]
        L.treewy_status_str.argtypes = [i32]
        L.treewy_status_str.restype = ctypes.c_char_p
        for name in EXPORTS[:-1]:
            getattr(L, name).restype = ctypes.c_int
        L.treewy_tree_desc_size.restype = ctypes.c_size_t
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().treewy_status_str(int(status)).decode()


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    return int(x)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if hasattr(stream, "cuda_stream"):
        return stream.cuda_stream
    return int(stream)


def _parent_arg(parent):
    if parent is None:
        return None
    arr = np.ascontiguousarray(np.asarray(parent, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _check(status: int, where: str) -> int:
    if status != TREEWY_OK:
        raise TreewyError(status, where)
    return status


# ---------------------------------------------------------------------------
# the C ABI, same names and argument order
# ---------------------------------------------------------------------------

def treewy_tree_meta(parent: Sequence[int]):
    """Returns (depth[N] int32, anc[N] uint64); raises TreewyError on a bad tree."""
    arr, pp = _parent_arg(parent)
    n = len(arr)
    depth = np.zeros(max(n, 1), dtype=np.int32)
    anc = np.zeros(max(n, 1), dtype=np.uint64)
    _check(lib().treewy_tree_meta(pp, n, depth.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                  anc.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))),
           "treewy_tree_meta")
    return depth[:n], anc[:n]


def _parent_n(parent, N):
    if parent is None:
        return None, None
    arr, pp = _parent_arg(parent)
    if N > 0 and len(arr) < N:
        raise ValueError(f"parent has {len(arr)} entries but N={N}")
    return arr, pp


def bind(name, *args, stream=None):
    """One C-ABI call with its arguments converted once: tensors to device
    pointers, int32 numpy arrays (parent arrays) to host pointers kept alive
    with the call, the stream to its handle; other arguments as they are.
    Returns a callable with no arguments that makes the call and raises on a
    bad status.  For launch loops, where converting ~20 arguments per call can
    cost more host time than a kernel takes."""
    fn = getattr(lib(), name)
    keep, conv = [], []
    for a in args:
        if hasattr(a, "data_ptr"):
            conv.append(a.data_ptr())
        elif isinstance(a, np.ndarray):
            arr = np.ascontiguousarray(a, dtype=np.int32)
            keep.append(arr)
            conv.append(arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
        else:
            conv.append(a)
    conv.append(_stream(stream))
    conv = tuple(conv)

    def call():
        s = fn(*conv)
        if s != TREEWY_OK:
            raise TreewyError(s, name)

    call.keep = keep
    return call


def treewy_verify(S0, q, k, v, alpha, beta, parent, B, H, N, out, vtilde, gamma, dtype,
                  stream=None, check=True) -> int:
    arr, pp = _parent_n(parent, N)
    s = lib().treewy_verify(_ptr(S0), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), pp,
                            B, H, N, _ptr(out), _ptr(vtilde), _ptr(gamma), dtype, _stream(stream))
    return _check(s, "treewy_verify") if check else s


def treewy_commit(S0, vtilde, k, gamma, accepted, parent, B, H, N, S_out, dtype,
                  stream=None, check=True) -> int:
    arr, pp = _parent_n(parent, N)
    s = lib().treewy_commit(_ptr(S0), _ptr(vtilde), _ptr(k), _ptr(gamma), _ptr(accepted), pp,
                            B, H, N, _ptr(S_out), dtype, _stream(stream))
    return _check(s, "treewy_commit") if check else s


def treewy_commit_verify(S0, S_out, vtilde_prev, k_prev, gamma_prev, accepted_prev, parent_prev,
                         N_prev, q, k, v, alpha, beta, parent, B, H, N, out, vtilde, gamma, dtype,
                         stream=None, check=True) -> int:
    arr_p, pp_prev = _parent_n(parent_prev, N_prev)
    arr, pp = _parent_n(parent, N)
    s = lib().treewy_commit_verify(_ptr(S0), _ptr(S_out), _ptr(vtilde_prev), _ptr(k_prev),
                                   _ptr(gamma_prev), _ptr(accepted_prev), pp_prev, N_prev,
                                   _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), pp, B, H, N,
                                   _ptr(out), _ptr(vtilde), _ptr(gamma), dtype, _stream(stream))
    return _check(s, "treewy_commit_verify") if check else s


def treewy_commit_verify_pool(pool, n_slots, slots, vtilde_prev, k_prev, gamma_prev, accepted_prev,
                              parent_prev, N_prev, q, k, v, alpha, beta, parent, B, H, N, out,
                              vtilde, gamma, dtype, stream=None, check=True) -> int:
    arr_p, pp_prev = _parent_n(parent_prev, N_prev)
    arr, pp = _parent_n(parent, N)
    s = lib().treewy_commit_verify_pool(_ptr(pool), n_slots, _ptr(slots), _ptr(vtilde_prev),
                                        _ptr(k_prev), _ptr(gamma_prev), _ptr(accepted_prev),
                                        pp_prev, N_prev, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                        _ptr(beta), pp, B, H, N, _ptr(out), _ptr(vtilde),
                                        _ptr(gamma), dtype, _stream(stream))
    return _check(s, "treewy_commit_verify_pool") if check else s


def treewy_commit_verify_bf16state(S0, S_out, vtilde_prev, k_prev, gamma_prev, accepted_prev,
                                   parent_prev, N_prev, q, k, v, alpha, beta, parent, B, H, N, out,
                                   vtilde, gamma, dtype, stream=None, check=True) -> int:
    arr_p, pp_prev = _parent_n(parent_prev, N_prev)
    arr, pp = _parent_n(parent, N)
    s = lib().treewy_commit_verify_bf16state(_ptr(S0), _ptr(S_out), _ptr(vtilde_prev),
                                             _ptr(k_prev), _ptr(gamma_prev), _ptr(accepted_prev),
                                             pp_prev, N_prev, _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(alpha), _ptr(beta), pp, B, H, N, _ptr(out),
                                             _ptr(vtilde), _ptr(gamma), dtype, _stream(stream))
    return _check(s, "treewy_commit_verify_bf16state") if check else s


def treewy_prefill_chain(S, q, k, v, alpha, beta, B, T, H, chunk, out, work_vtilde, work_gamma,
                         dtype, stream=None, check=True) -> int:
    s = lib().treewy_prefill_chain(_ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), B,
                                   T, H, chunk, _ptr(out), _ptr(work_vtilde), _ptr(work_gamma),
                                   dtype, _stream(stream))
    return _check(s, "treewy_prefill_chain") if check else s


def treewy_prefill_chain_noalloc(S, q, k, v, alpha, beta, B, T, H, chunk, out, dtype, stream=None,
                                 check=True) -> int:
    s = lib().treewy_prefill_chain_noalloc(_ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                           _ptr(beta), B, T, H, chunk, _ptr(out), dtype,
                                           _stream(stream))
    return _check(s, "treewy_prefill_chain_noalloc") if check else s


def treewy_prefill(S, q, k, v, alpha, beta, B, T, H, out, dtype, stream=None, check=True) -> int:
    s = lib().treewy_prefill(_ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), B, T, H,
                             _ptr(out), dtype, _stream(stream))
    return _check(s, "treewy_prefill") if check else s


def treewy_tree_desc_size() -> int:
    return int(lib().treewy_tree_desc_size())


def treewy_tree_desc_pack(parents, counts, count, n_max, desc, check=True):
    """parents int32 [count, n_max], counts int32 [count] (host numpy); desc a
    writable host buffer of count * treewy_tree_desc_size() bytes, 8-byte
    aligned.  Returns (status, max_depth)."""
    par = np.ascontiguousarray(np.asarray(parents, dtype=np.int32))
    cnt = np.ascontiguousarray(np.asarray(counts, dtype=np.int32))
    md = ctypes.c_int(-1)
    pp = par.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if par.size else None
    cp = cnt.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if cnt.size else None
    s = lib().treewy_tree_desc_pack(pp, cp, count, n_max, _ptr(desc), ctypes.byref(md))
    if check:
        _check(s, "treewy_tree_desc_pack")
    return s, md.value


def treewy_commit_verify_pool_trees(pool, n_slots, slots, vtilde_prev, k_prev, gamma_prev,
                                    accepted_prev, trees_prev, N_prev, depth_prev, q, k, v, alpha,
                                    beta, trees, N, depth, B, H, out, vtilde, gamma, dtype,
                                    stream=None, check=True) -> int:
    s = lib().treewy_commit_verify_pool_trees(
        _ptr(pool), n_slots, _ptr(slots), _ptr(vtilde_prev), _ptr(k_prev), _ptr(gamma_prev),
        _ptr(accepted_prev), _ptr(trees_prev), N_prev, depth_prev, _ptr(q), _ptr(k), _ptr(v),
        _ptr(alpha), _ptr(beta), _ptr(trees), N, depth, B, H, _ptr(out), _ptr(vtilde), _ptr(gamma),
        dtype, _stream(stream))
    return _check(s, "treewy_commit_verify_pool_trees") if check else s


def treewy_commit_verify_bf16state_pool(pool, n_slots, slots, vtilde_prev, k_prev, gamma_prev,
                                        accepted_prev, parent_prev, N_prev, q, k, v, alpha, beta,
                                        parent, B, H, N, out, vtilde, gamma, dtype, stream=None,
                                        check=True) -> int:
    arr_p, pp_prev = _parent_n(parent_prev, N_prev)
    arr, pp = _parent_n(parent, N)
    s = lib().treewy_commit_verify_bf16state_pool(
        _ptr(pool), n_slots, _ptr(slots), _ptr(vtilde_prev), _ptr(k_prev), _ptr(gamma_prev),
        _ptr(accepted_prev), pp_prev, N_prev, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), pp,
        B, H, N, _ptr(out), _ptr(vtilde), _ptr(gamma), dtype, _stream(stream))
    return _check(s, "treewy_commit_verify_bf16state_pool") if check else s


def treewy_commit_verify_bf16state_pool_trees(pool, n_slots, slots, vtilde_prev, k_prev,
                                              gamma_prev, accepted_prev, trees_prev, N_prev,
                                              depth_prev, q, k, v, alpha, beta, trees, N, depth, B,
                                              H, out, vtilde, gamma, dtype, stream=None,
                                              check=True) -> int:
    s = lib().treewy_commit_verify_bf16state_pool_trees(
        _ptr(pool), n_slots, _ptr(slots), _ptr(vtilde_prev), _ptr(k_prev), _ptr(gamma_prev),
        _ptr(accepted_prev), _ptr(trees_prev), N_prev, depth_prev, _ptr(q), _ptr(k), _ptr(v),
        _ptr(alpha), _ptr(beta), _ptr(trees), N, depth, B, H, _ptr(out), _ptr(vtilde), _ptr(gamma),
        dtype, _stream(stream))
    return _check(s, "treewy_commit_verify_bf16state_pool_trees") if check else s


def treewy_store_all(S0, q, k, v, alpha, beta, parent, B, H, N, out, snapshots, dtype,
                     stream=None, check=True) -> int:
    arr, pp = _parent_n(parent, N)
    s = lib().treewy_store_all(_ptr(S0), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), pp,
                               B, H, N, _ptr(out), _ptr(snapshots), dtype, _stream(stream))
    return _check(s, "treewy_store_all") if check else s


def treewy_store_all_select(snapshots, accepted, B, H, N, S_out, stream=None, check=True) -> int:
    s = lib().treewy_store_all_select(_ptr(snapshots), _ptr(accepted), B, H, N, _ptr(S_out),
                                      _stream(stream))
    return _check(s, "treewy_store_all_select") if check else s


# ---------------------------------------------------------------------------
# allocating conveniences (torch tensors in the layouts of include/treewy.h).
# Shapes, dtypes, devices and contiguity are checked here so that a mis-shaped
# tensor can never reach a kernel as an out-of-bounds buffer.
# ---------------------------------------------------------------------------

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return TREEWY_BF16
    if t.dtype == torch.float32:
        return TREEWY_F32
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _need(name, t, shape, dtype, device):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != device or t.device.type != "cuda":
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _check_parent_len(parent, N):
    if len(np.asarray(parent).reshape(-1)) != N:
        raise ValueError(f"parent has {len(np.asarray(parent).reshape(-1))} entries, expected N={N}")


def _check_tokens(S0, q, k, v, alpha, beta, parent):
    import torch
    B, N, H, d = q.shape
    if d != D:
        raise ValueError(f"head dim {d}, expected {D}")
    dev, dt = q.device, q.dtype
    _need("S0", S0, (B, H, D, D), torch.float32, dev)
    _need("q", q, (B, N, H, D), dt, dev)
    _need("k", k, (B, N, H, D), dt, dev)
    _need("v", v, (B, N, H, D), dt, dev)
    _need("alpha", alpha, (B, N, H), dt, dev)
    _need("beta", beta, (B, N, H), dt, dev)
    _check_parent_len(parent, N)
    return B, N, H, dev


def verify(S0, q, k, v, alpha, beta, parent, stream=None, out=None, vtilde=None, gamma=None):
    """q,k,v [B,N,H,128]; alpha,beta [B,N,H] (bf16 or fp32); S0 [B,H,128,128] fp32.
    Returns (out [B,N,H,128], vtilde [B,H,N,128], gamma [B,H,N]), all fp32."""
    import torch
    B, N, H, dev = _check_tokens(S0, q, k, v, alpha, beta, parent)
    out = torch.empty((B, N, H, D), dtype=torch.float32, device=dev) if out is None else out
    vtilde = torch.empty((B, H, N, D), dtype=torch.float32, device=dev) if vtilde is None else vtilde
    gamma = torch.empty((B, H, N), dtype=torch.float32, device=dev) if gamma is None else gamma
    _need("out", out, (B, N, H, D), torch.float32, dev)
    _need("vtilde", vtilde, (B, H, N, D), torch.float32, dev)
    _need("gamma", gamma, (B, H, N), torch.float32, dev)
    treewy_verify(S0, q, k, v, alpha, beta, parent, B, H, N, out, vtilde, gamma, _dtype_code(q),
                  stream)
    return out, vtilde, gamma


def commit(S0, vtilde, k, gamma, accepted, parent, S_out=None, stream=None):
    """Rebuild S_a for each sequence; S_out may be S0 itself (in place)."""
    import torch
    B, N, H, d = k.shape
    dev = k.device
    _need("S0", S0, (B, H, D, D), torch.float32, dev)
    _need("vtilde", vtilde, (B, H, N, D), torch.float32, dev)
    _need("k", k, (B, N, H, D), k.dtype, dev)
    _need("gamma", gamma, (B, H, N), torch.float32, dev)
    _need("accepted", accepted, (B,), torch.int32, dev)
    _check_parent_len(parent, N)
    S_out = torch.empty_like(S0) if S_out is None else S_out
    _need("S_out", S_out, (B, H, D, D), torch.float32, dev)
    treewy_commit(S0, vtilde, k, gamma, accepted, parent, B, H, N, S_out, _dtype_code(k), stream)
    return S_out


def commit_verify(S0, vtilde_prev, k_prev, gamma_prev, accepted_prev, parent_prev,
                  q, k, v, alpha, beta, parent, S_out=None, stream=None, out=None, vtilde=None,
                  gamma=None):
    """Commit the previous step's accepted node (its vtilde / k / gamma /
    accepted / parent) into S_out (default: in place, S_out = S0), then verify
    the new step (q, k, v, alpha, beta, parent) from it.
    Returns (S_out, out, vtilde, gamma)."""
    import torch
    B, N, H, dev = _check_tokens(S0, q, k, v, alpha, beta, parent)
    Np = k_prev.shape[1]
    _need("vtilde_prev", vtilde_prev, (B, H, Np, D), torch.float32, dev)
    _need("k_prev", k_prev, (B, Np, H, D), q.dtype, dev)
    _need("gamma_prev", gamma_prev, (B, H, Np), torch.float32, dev)
    _need("accepted_prev", accepted_prev, (B,), torch.int32, dev)
    _check_parent_len(parent_prev, Np)
    S_out = S0 if S_out is None else S_out
    _need("S_out", S_out, (B, H, D, D), torch.float32, dev)
    out = torch.empty((B, N, H, D), dtype=torch.float32, device=dev) if out is None else out
    vtilde = torch.empty((B, H, N, D), dtype=torch.float32, device=dev) if vtilde is None else vtilde
    gamma = torch.empty((B, H, N), dtype=torch.float32, device=dev) if gamma is None else gamma
    _need("out", out, (B, N, H, D), torch.float32, dev)
    _need("vtilde", vtilde, (B, H, N, D), torch.float32, dev)
    _need("gamma", gamma, (B, H, N), torch.float32, dev)
    treewy_commit_verify(S0, S_out, vtilde_prev, k_prev, gamma_prev, accepted_prev, parent_prev, Np,
                         q, k, v, alpha, beta, parent, B, H, N, out, vtilde, gamma, _dtype_code(q),
                         stream)
    return S_out, out, vtilde, gamma


def commit_verify_pool(pool, slots, vtilde_prev, k_prev, gamma_prev, accepted_prev, parent_prev,
                       q, k, v, alpha, beta, parent, stream=None, out=None, vtilde=None,
                       gamma=None):
    """Pool form of commit_verify: pool [n_slots, H, 128, 128] fp32 holds one
    state per request; sequence b's state is pool[slots[b]] and is committed
    in place (accepted_prev[b] < 0: no previous step, state left as is).  A
    torch.bfloat16 pool holds bf16 states (treewy_commit_verify_bf16state_pool;
    bf16 inputs).  Returns (out, vtilde, gamma)."""
    import torch
    B, N, H, d = q.shape
    if d != D:
        raise ValueError(f"head dim {d}, expected {D}")
    dev, dt = q.device, q.dtype
    if pool.dim() != 4 or tuple(pool.shape[1:]) != (H, D, D):
        raise ValueError(f"pool: shape {tuple(pool.shape)}, expected (n_slots, {H}, {D}, {D})")
    s16 = pool.dtype == torch.bfloat16
    _need("pool", pool, tuple(pool.shape), torch.bfloat16 if s16 else torch.float32, dev)
    _need("slots", slots, (B,), torch.int32, dev)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _need(name, x, (B, N, H, D), dt, dev)
    _need("alpha", alpha, (B, N, H), dt, dev)
    _need("beta", beta, (B, N, H), dt, dev)
    _check_parent_len(parent, N)
    Np = k_prev.shape[1]
    _need("vtilde_prev", vtilde_prev, (B, H, Np, D), torch.float32, dev)
    _need("k_prev", k_prev, (B, Np, H, D), dt, dev)
    _need("gamma_prev", gamma_prev, (B, H, Np), torch.float32, dev)
    _need("accepted_prev", accepted_prev, (B,), torch.int32, dev)
    _check_parent_len(parent_prev, Np)
    out = torch.empty((B, N, H, D), dtype=torch.float32, device=dev) if out is None else out
    vtilde = torch.empty((B, H, N, D), dtype=torch.float32, device=dev) if vtilde is None else vtilde
    gamma = torch.empty((B, H, N), dtype=torch.float32, device=dev) if gamma is None else gamma
    _need("out", out, (B, N, H, D), torch.float32, dev)
    _need("vtilde", vtilde, (B, H, N, D), torch.float32, dev)
    _need("gamma", gamma, (B, H, N), torch.float32, dev)
    call = treewy_commit_verify_bf16state_pool if s16 else treewy_commit_verify_pool
    call(pool, pool.shape[0], slots, vtilde_prev, k_prev, gamma_prev, accepted_prev, parent_prev, Np,
         q, k, v, alpha, beta, parent, B, H, N, out, vtilde, gamma, _dtype_code(q), stream)
    return out, vtilde, gamma


def pack_trees(parents, n_max=None):
    """Validate and pack one parent array per request (a list of 1-D int
    arrays).  Returns (descriptors as a host uint8 numpy array, n_max, the
    deepest node over all requests)."""
    counts = np.array([len(p) for p in parents], dtype=np.int32)
    n_max = int(counts.max()) if n_max is None else int(n_max)
    par = np.full((len(parents), n_max), -1, dtype=np.int32)
    for i, p in enumerate(parents):
        par[i, :len(p)] = np.asarray(p, dtype=np.int32)
    size = treewy_tree_desc_size()
    buf = np.zeros((len(parents) * size + 7) // 8, dtype=np.uint64)  # 8-byte aligned
    _, md = treewy_tree_desc_pack(par, counts, len(parents), n_max, buf.ctypes.data)
    return buf.view(np.uint8)[:len(parents) * size], n_max, md


def commit_verify_pool_trees(pool, slots, vtilde_prev, k_prev, gamma_prev, accepted_prev,
                             trees_prev, depth_prev, q, k, v, alpha, beta, trees, depth,
                             stream=None, out=None, vtilde=None, gamma=None):
    """Pool form of commit_verify with a tree per request: trees / trees_prev
    are device uint8 tensors of packed descriptors (pack_trees, then copied to
    the device), depth / depth_prev their depth bounds; every per-node array
    is padded to the node-count bound (q.shape[1], k_prev.shape[1]).  Rows
    past a request's own count are not written.  A torch.bfloat16 pool holds
    bf16 states (treewy_commit_verify_bf16state_pool_trees; bf16 inputs).
    Returns (out, vtilde, gamma)."""
    import torch
    B, N, H, d = q.shape
    if d != D:
        raise ValueError(f"head dim {d}, expected {D}")
    dev, dt = q.device, q.dtype
    if pool.dim() != 4 or tuple(pool.shape[1:]) != (H, D, D):
        raise ValueError(f"pool: shape {tuple(pool.shape)}, expected (n_slots, {H}, {D}, {D})")
    size = treewy_tree_desc_size()
    s16 = pool.dtype == torch.bfloat16
    _need("pool", pool, tuple(pool.shape), torch.bfloat16 if s16 else torch.float32, dev)
    _need("slots", slots, (B,), torch.int32, dev)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _need(name, x, (B, N, H, D), dt, dev)
    _need("alpha", alpha, (B, N, H), dt, dev)
    _need("beta", beta, (B, N, H), dt, dev)
    _need("trees", trees, (B * size,), torch.uint8, dev)
    Np = k_prev.shape[1]
    _need("vtilde_prev", vtilde_prev, (B, H, Np, D), torch.float32, dev)
    _need("k_prev", k_prev, (B, Np, H, D), dt, dev)
    _need("gamma_prev", gamma_prev, (B, H, Np), torch.float32, dev)
    _need("accepted_prev", accepted_prev, (B,), torch.int32, dev)
    _need("trees_prev", trees_prev, (B * size,), torch.uint8, dev)
    out = torch.empty((B, N, H, D), dtype=torch.float32, device=dev) if out is None else out
    vtilde = torch.empty((B, H, N, D), dtype=torch.float32, device=dev) if vtilde is None else vtilde
    gamma = torch.empty((B, H, N), dtype=torch.float32, device=dev) if gamma is None else gamma
    _need("out", out, (B, N, H, D), torch.float32, dev)
    _need("vtilde", vtilde, (B, H, N, D), torch.float32, dev)
    _need("gamma", gamma, (B, H, N), torch.float32, dev)
    call = (treewy_commit_verify_bf16state_pool_trees if s16 else treewy_commit_verify_pool_trees)
    call(pool, pool.shape[0], slots, vtilde_prev, k_prev, gamma_prev, accepted_prev, trees_prev, Np,
         depth_prev, q, k, v, alpha, beta, trees, N, depth, B, H, out, vtilde, gamma, _dtype_code(q),
         stream)
    return out, vtilde, gamma


def commit_verify_bf16state(S0, vtilde_prev, k_prev, gamma_prev, accepted_prev, parent_prev,
                            q, k, v, alpha, beta, parent, S_out=None, stream=None, out=None,
                            vtilde=None, gamma=None):
    """commit_verify with the state stored as bf16: S0 / S_out [B, H, 128, 128]
    torch.bfloat16 (default S_out = S0, in place).  Inputs must be bf16.
    Returns (S_out, out, vtilde, gamma)."""
    import torch
    B, N, H, d = q.shape
    if d != D:
        raise ValueError(f"head dim {d}, expected {D}")
    dev = q.device
    if q.dtype != torch.bfloat16:
        raise TypeError("commit_verify_bf16state takes bf16 inputs")
    _need("S0", S0, (B, H, D, D), torch.bfloat16, dev)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _need(name, x, (B, N, H, D), torch.bfloat16, dev)
    _need("alpha", alpha, (B, N, H), torch.bfloat16, dev)
    _need("beta", beta, (B, N, H), torch.bfloat16, dev)
    _check_parent_len(parent, N)
    Np = k_prev.shape[1]
    _need("vtilde_prev", vtilde_prev, (B, H, Np, D), torch.float32, dev)
    _need("k_prev", k_prev, (B, Np, H, D), torch.bfloat16, dev)
    _need("gamma_prev", gamma_prev, (B, H, Np), torch.float32, dev)
    _need("accepted_prev", accepted_prev, (B,), torch.int32, dev)
    _check_parent_len(parent_prev, Np)
    S_out = S0 if S_out is None else S_out
    _need("S_out", S_out, (B, H, D, D), torch.bfloat16, dev)
    out = torch.empty((B, N, H, D), dtype=torch.float32, device=dev) if out is None else out
    vtilde = torch.empty((B, H, N, D), dtype=torch.float32, device=dev) if vtilde is None else vtilde
    gamma = torch.empty((B, H, N), dtype=torch.float32, device=dev) if gamma is None else gamma
    _need("out", out, (B, N, H, D), torch.float32, dev)
    _need("vtilde", vtilde, (B, H, N, D), torch.float32, dev)
    _need("gamma", gamma, (B, H, N), torch.float32, dev)
    treewy_commit_verify_bf16state(S0, S_out, vtilde_prev, k_prev, gamma_prev, accepted_prev,
                                   parent_prev, Np, q, k, v, alpha, beta, parent, B, H, N, out,
                                   vtilde, gamma, TREEWY_BF16, stream)
    return S_out, out, vtilde, gamma


def prefill_chain(S, q, k, v, alpha, beta, chunk=16, stream=None, out=None, work=None):
    """Run the gated delta rule over the T tokens of q,k,v [B,T,H,128] and
    alpha, beta [B,T,H] from the state S [B,H,128,128] (updated in place), in
    chunks of `chunk` tokens.  Returns out [B,T,H,128] fp32.  `work` is an
    optional (vtilde, gamma) workspace pair from prefill_workspace()."""
    import torch
    B, T, H, d = q.shape
    if d != D:
        raise ValueError(f"head dim {d}, expected {D}")
    dev, dt = q.device, q.dtype
    _need("S", S, (B, H, D, D), torch.float32, dev)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _need(name, x, (B, T, H, D), dt, dev)
    _need("alpha", alpha, (B, T, H), dt, dev)
    _need("beta", beta, (B, T, H), dt, dev)
    out = torch.empty((B, T, H, D), dtype=torch.float32, device=dev) if out is None else out
    _need("out", out, (B, T, H, D), torch.float32, dev)
    wv, wg = prefill_workspace(B, H, chunk, dev) if work is None else work
    treewy_prefill_chain(S, q, k, v, alpha, beta, B, T, H, chunk, out, wv, wg, _dtype_code(q),
                         stream)
    return out


def prefill(S, q, k, v, alpha, beta, stream=None, out=None):
    """One-launch prefill: the gated delta rule over the T tokens of q,k,v
    [B,T,H,128] and alpha, beta [B,T,H] from the state S [B,H,128,128]
    (updated in place).  Returns out [B,T,H,128] fp32.  No workspace."""
    import torch
    B, T, H, d = q.shape
    if d != D:
        raise ValueError(f"head dim {d}, expected {D}")
    dev, dt = q.device, q.dtype
    _need("S", S, (B, H, D, D), torch.float32, dev)
    for name, x in (("q", q), ("k", k), ("v", v)):
        _need(name, x, (B, T, H, D), dt, dev)
    _need("alpha", alpha, (B, T, H), dt, dev)
    _need("beta", beta, (B, T, H), dt, dev)
    out = torch.empty((B, T, H, D), dtype=torch.float32, device=dev) if out is None else out
    _need("out", out, (B, T, H, D), torch.float32, dev)
    treewy_prefill(S, q, k, v, alpha, beta, B, T, H, out, _dtype_code(q), stream)
    return out


def prefill_workspace(B, H, chunk, device):
    """Workspace of treewy_prefill_chain: two pseudo-value and two gate buffers."""
    import torch
    gm = (B * H * chunk + 3) // 4 * 4
    return (torch.empty(2 * B * H * chunk * D, dtype=torch.float32, device=device),
            torch.empty(2 * gm, dtype=torch.float32, device=device))


def store_all(S0, q, k, v, alpha, beta, parent, stream=None, out=None, snapshots=None):
    import torch
    B, N, H, dev = _check_tokens(S0, q, k, v, alpha, beta, parent)
    out = torch.empty((B, N, H, D), dtype=torch.float32, device=dev) if out is None else out
    if snapshots is None:
        snapshots = torch.empty((B, H, N + 1, D, D), dtype=torch.float32, device=dev)
    _need("out", out, (B, N, H, D), torch.float32, dev)
    _need("snapshots", snapshots, (B, H, N + 1, D, D), torch.float32, dev)
    treewy_store_all(S0, q, k, v, alpha, beta, parent, B, H, N, out, snapshots, _dtype_code(q),
                     stream)
    return out, snapshots


def store_all_select(snapshots, accepted, S_out=None, stream=None):
    import torch
    B, H, N1 = snapshots.shape[:3]
    dev = snapshots.device
    _need("snapshots", snapshots, (B, H, N1, D, D), torch.float32, dev)
    _need("accepted", accepted, (B,), torch.int32, dev)
    S_out = torch.empty((B, H, D, D), dtype=torch.float32, device=dev) if S_out is None else S_out
    _need("S_out", S_out, (B, H, D, D), torch.float32, dev)
    treewy_store_all_select(snapshots, accepted, B, H, N1 - 1, S_out, stream)
    return S_out
