"""Python wrapper of the CPU oracle (wi_oracle.c) and its brute-force twin.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code
with the HIP library. See wi_oracle.c for the reading of the RetroInfer pages
each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "wi_oracle.c")
# WIO_SANITIZE=1 selects a separate build instrumented with AddressSanitizer
# and UndefinedBehaviorSanitizer (load it with libasan preloaded).
SANITIZE = os.environ.get("WIO_SANITIZE") == "1"
_SO = os.path.join(_HERE, "libwi_oracle_san.so" if SANITIZE else "libwi_oracle.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g"]

F32, BF16 = 0, 1


def _host_has_fma() -> bool:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("flags"):
                    return " fma " in line + " "
    except OSError:
        pass
    return False


def gcc_command(src: str, out: str) -> list:
    """gcc line for the oracle: scalar code, no FMA contraction of separate
    multiplies and adds. The explicit fma()/fmaf() calls are correctly
    rounded either way; -mfma (where the host has it) only lets gcc emit the
    instruction instead of a libm call."""
    fma = ["-mfma"] if _host_has_fma() else []
    san = SANITIZE_FLAGS if SANITIZE else []
    return ["gcc", "-O2", "-std=gnu11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
            *fma, *san, "-fPIC", "-shared", src, "-o", out, "-lm"]


def _flags() -> str:
    return " ".join(a for a in gcc_command("SRC", "OUT") if a not in ("SRC", "OUT"))


def _built_for_this_host() -> bool:
    stamp = _SO + ".flags"
    return os.path.exists(stamp) and open(stamp).read() == _flags()


def compile_oracle(force: bool = False) -> str:
    """Compile the oracle with gcc (see gcc_command)."""
    if (force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC)
            or not _built_for_this_host()):
        tmp = _SO + f".tmp{os.getpid()}"
        subprocess.check_call(gcc_command(_SRC, tmp))
        os.replace(tmp, _SO)
        with open(_SO + ".flags", "w") as f:
            f.write(_flags())
    return _SO


class Desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("n_ctx", ctypes.c_int64), ("seg_len", ctypes.c_int32),
                ("clusters_per_seg", ctypes.c_int32), ("n_sink", ctypes.c_int32),
                ("n_local", ctypes.c_int32), ("n_iters", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("layer_id", ctypes.c_uint32),
                ("n_pending", ctypes.c_int64)]


class DDesc(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("k_retrieve", ctypes.c_int32),
                ("k_estimate", ctypes.c_int32), ("scale", ctypes.c_double)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(compile_oracle())
        u64, i32, i64 = ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64
        P = ctypes.c_void_p
        _lib.wio_mix64.restype = u64
        _lib.wio_mix64.argtypes = [u64]
        _lib.wio_key.restype = u64
        _lib.wio_key.argtypes = [u64] * 6
        _lib.wio_round_bf16.restype = ctypes.c_float
        _lib.wio_round_bf16.argtypes = [ctypes.c_float]
        _lib.wio_sizes.argtypes = [P, P, P, P, P]
        _lib.wio_kmeanspp.argtypes = [P, i32, i32, i32, u64, u64, u64, u64, u64, P]
        _lib.wio_assign.argtypes = [P, i32, i32, P, i32, P]
        _lib.wio_update.argtypes = [P, i32, i32, P, i32, i32, P, P]
        _lib.wio_build.argtypes = [P] * 15
        _lib.wio_decode.argtypes = [P] * 18 + [i64, P]
        _lib.wio_attend_sets.argtypes = [P] * 13 + [P, i32, P, i32, P]
        _lib.wio_append.argtypes = [P] * 7
        _lib.wio_extend.argtypes = [P] * 23
        _lib.wio_dense_attention.argtypes = [P] * 6
        _lib.wio_recall.argtypes = [P] * 8 + [i32, i32, P, P, P]
        _lib.wio_num_threads.restype = ctypes.c_int
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def make_desc(dtype, batch, n_kv_heads, n_ctx, seg_len=8192, clusters_per_seg=512,
              n_sink=4, n_local=64, n_iters=10, seed=0, layer_id=0, head_dim=128,
              n_pending=0):
    return Desc(F32 if dtype in ("f32", F32) else BF16, batch, n_kv_heads, head_dim,
                n_ctx, seg_len, clusters_per_seg, n_sink, n_local, n_iters, seed,
                layer_id, n_pending)


def sizes(desc):
    ns, c, cap = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    t = ctypes.c_int32()
    rc = lib().wio_sizes(ctypes.byref(desc), ctypes.byref(ns), ctypes.byref(c),
                         ctypes.byref(cap), ctypes.byref(t))
    if rc != 0:
        raise ValueError("invalid oracle sizes")
    return ns.value, c.value, cap.value, t.value


def mix64(z):
    return lib().wio_mix64(z)


def key(seed, b, l, h, s, r):
    return lib().wio_key(seed, b, l, h, s, r)


def round_bf16(x: float) -> float:
    return lib().wio_round_bf16(x)


def kmeanspp(X, k, seed=0, b=0, l=0, h=0, s=0):
    X = np.ascontiguousarray(X, dtype=np.float32)
    picks = np.empty(k, np.int32)
    lib().wio_kmeanspp(_p(X), X.shape[0], X.shape[1], k, seed, b, l, h, s, _p(picks))
    return picks


def assign(X, C):
    X = np.ascontiguousarray(X, dtype=np.float32)
    C = np.ascontiguousarray(C, dtype=np.float32)
    a = np.empty(X.shape[0], np.int32)
    lib().wio_assign(_p(X), X.shape[0], X.shape[1], _p(C), C.shape[0], _p(a))
    return a


def update(X, a, C, dtype):
    X = np.ascontiguousarray(X, dtype=np.float32)
    a = np.ascontiguousarray(a, dtype=np.int32)
    C = np.array(C, dtype=np.float32, copy=True)
    cnt = np.empty(C.shape[0], np.int32)
    lib().wio_update(_p(X), X.shape[0], X.shape[1], _p(a), C.shape[0],
                     F32 if dtype in ("f32", F32) else BF16, _p(C), _p(cnt))
    return C, cnt


def build(desc, K, V, init=None, units=None):
    """K, V: [B, H, N, d] float32. Returns a dict of index arrays.

    units: optional list of unit ids (b * H + h) to build; other units'
    outputs are left uninitialised."""
    ns, C, cap, T = sizes(desc)
    U = desc.batch * desc.n_kv_heads
    d = desc.head_dim
    n_idx = desc.n_ctx - desc.n_sink - desc.n_local
    nst = desc.n_sink + desc.n_local
    K = np.ascontiguousarray(K, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    assert K.shape == (desc.batch, desc.n_kv_heads, desc.n_ctx, d)
    if init is not None:
        init = np.ascontiguousarray(init, dtype=np.float32).reshape(U, C, d)
    mask = None
    if units is not None:
        mask = np.zeros(U, np.uint8)
        mask[list(units)] = 1
    out = dict(
        centroids=np.empty((U, C, d), np.float32), sizes=np.empty((U, C), np.int32),
        vsum=np.empty((U, C, d), np.float32), block_off=np.empty((U, C + 1), np.int32),
        kblk=np.empty((U, cap * T, d), np.float32), vblk=np.empty((U, cap * T, d), np.float32),
        slot_token=np.empty((U, cap * T), np.int32),
        steady_k=np.empty((U, nst, d), np.float32), steady_v=np.empty((U, nst, d), np.float32),
        assign=np.empty((U, n_idx), np.int32))
    rc = lib().wio_build(ctypes.byref(desc), _p(K), _p(V), _p(init),
                         _p(out["centroids"]), _p(out["sizes"]), _p(out["vsum"]),
                         _p(out["block_off"]), _p(out["kblk"]), _p(out["vblk"]),
                         _p(out["slot_token"]), _p(out["steady_k"]), _p(out["steady_v"]),
                         _p(out["assign"]), _p(mask))
    if rc != 0:
        raise ValueError("oracle build failed")
    return out


def _index_args(idx):
    return [_p(np.ascontiguousarray(idx[k])) for k in (
        "centroids", "sizes", "vsum", "block_off", "kblk", "vblk")]


def decode(desc, n_q_heads, k_retrieve, k_estimate, idx, q, scale=0.0,
           exec_cap=None):
    """Returns dict(out [B,Hq,d] f64, sel [U,M], exec_tokens, n_exec, gkey [U,C])."""
    ns, C, cap, T = sizes(desc)
    U = desc.batch * desc.n_kv_heads
    d = desc.head_dim
    k_e = min(k_estimate, C - k_retrieve)
    if exec_cap is None:
        exec_cap = desc.n_sink + desc.n_local + desc.n_pending + int(
            np.sort(idx["sizes"], axis=1)[:, ::-1][:, :k_retrieve].sum(axis=1).max(initial=0))
    q = np.ascontiguousarray(q, dtype=np.float32)
    res = dict(out=np.empty((desc.batch, n_q_heads, d), np.float64),
               sel=np.empty((U, k_retrieve + max(k_e, 0)), np.int32),
               exec_tokens=np.full((U, exec_cap), -7, np.int32),
               n_exec=np.empty(U, np.int32), gkey=np.empty((U, C), np.float64))
    dd = DDesc(n_q_heads, k_retrieve, k_estimate, scale)
    keep = [np.ascontiguousarray(idx[k]) for k in (
        "centroids", "sizes", "vsum", "block_off", "kblk", "vblk", "slot_token",
        "steady_k", "steady_v")] + _pending(desc, idx)
    rc = lib().wio_decode(ctypes.byref(desc), ctypes.byref(dd), *[_p(a) for a in keep],
                          _p(q), _p(res["out"]), _p(res["sel"]), _p(res["exec_tokens"]),
                          _p(res["n_exec"]), exec_cap, _p(res["gkey"]))
    if rc != 0:
        raise ValueError("oracle decode failed")
    return res


def attend_sets(desc, n_q_heads, idx, q, R, E, scale=0.0):
    U = desc.batch * desc.n_kv_heads
    d = desc.head_dim
    R = np.ascontiguousarray(R, dtype=np.int32).reshape(U, -1)
    E = np.ascontiguousarray(E, dtype=np.int32).reshape(U, -1)
    q = np.ascontiguousarray(q, dtype=np.float32)
    out = np.empty((desc.batch, n_q_heads, d), np.float64)
    dd = DDesc(n_q_heads, R.shape[1], E.shape[1], scale)
    keep = [np.ascontiguousarray(idx[k]) for k in (
        "centroids", "sizes", "vsum", "block_off", "kblk", "vblk", "steady_k", "steady_v")]
    keep += _pending(desc, idx)
    rc = lib().wio_attend_sets(ctypes.byref(desc), ctypes.byref(dd), *[_p(a) for a in keep],
                               _p(q), _p(R), R.shape[1], _p(E), E.shape[1], _p(out))
    if rc != 0:
        raise ValueError("oracle attend failed")
    return out


def _pending(desc, idx):
    """The pending rows [U, seg_len, d] (None when nothing is pending)."""
    if desc.n_pending == 0:
        return [None, None]
    return [np.ascontiguousarray(idx["pend_k"], dtype=np.float32),
            np.ascontiguousarray(idx["pend_v"], dtype=np.float32)]


def append(desc, idx, k_new, v_new):
    """One decode step's token per sequence (k_new, v_new [B, H, d]): slides
    the local window of idx in place and moves the token leaving it to the
    pending rows. Returns the descriptor of the grown index (n_ctx + 1,
    n_pending + 1)."""
    U = desc.batch * desc.n_kv_heads
    d = desc.head_dim
    for key in ("pend_k", "pend_v"):
        if key not in idx:
            idx[key] = np.zeros((U, desc.seg_len, d), np.float32)
    for key in ("steady_k", "steady_v", "pend_k", "pend_v"):
        idx[key] = np.ascontiguousarray(idx[key], dtype=np.float32)
    k_new = np.ascontiguousarray(k_new, dtype=np.float32)
    v_new = np.ascontiguousarray(v_new, dtype=np.float32)
    rc = lib().wio_append(ctypes.byref(desc), _p(idx["steady_k"]), _p(idx["steady_v"]),
                          _p(idx["pend_k"]), _p(idx["pend_v"]), _p(k_new), _p(v_new))
    if rc != 0:
        raise ValueError("oracle append failed (pending segment full?)")
    nd = Desc.from_buffer_copy(desc)
    nd.n_ctx += 1
    nd.n_pending += 1
    return nd


def extend(desc, idx):
    """Cluster the full pending segment and return (descriptor, index) of the
    grown index (n_pending = 0)."""
    nd = Desc.from_buffer_copy(desc)
    nd.n_pending = 0
    ns, C, cap, T = sizes(nd)
    U = desc.batch * desc.n_kv_heads
    d = desc.head_dim
    n_idx = desc.n_ctx - desc.n_sink - desc.n_local
    nst = desc.n_sink + desc.n_local
    out = dict(
        centroids=np.empty((U, C, d), np.float32), sizes=np.empty((U, C), np.int32),
        vsum=np.empty((U, C, d), np.float32), block_off=np.empty((U, C + 1), np.int32),
        kblk=np.empty((U, cap * T, d), np.float32), vblk=np.empty((U, cap * T, d), np.float32),
        slot_token=np.empty((U, cap * T), np.int32),
        steady_k=np.empty((U, nst, d), np.float32), steady_v=np.empty((U, nst, d), np.float32),
        assign=np.empty((U, n_idx), np.int32))
    ins = [np.ascontiguousarray(idx[k]) for k in (
        "centroids", "sizes", "vsum", "block_off", "kblk", "vblk", "slot_token",
        "steady_k", "steady_v", "assign")] + _pending(desc, idx)
    rc = lib().wio_extend(ctypes.byref(desc), *[_p(a) for a in ins],
                          *[_p(out[k]) for k in ("centroids", "sizes", "vsum", "block_off",
                                                 "kblk", "vblk", "slot_token", "steady_k",
                                                 "steady_v", "assign")])
    if rc != 0:
        raise ValueError("oracle extend failed (pending segment not full?)")
    return nd, out


def dense_attention(desc, n_q_heads, K, V, q, scale=0.0):
    """Full attention over all desc.n_ctx tokens (float64): K, V [B, H, N, d]."""
    K = np.ascontiguousarray(K, dtype=np.float32)
    V = np.ascontiguousarray(V, dtype=np.float32)
    q = np.ascontiguousarray(q, dtype=np.float32)
    assert K.shape == (desc.batch, desc.n_kv_heads, desc.n_ctx, desc.head_dim)
    out = np.empty((desc.batch, n_q_heads, desc.head_dim), np.float64)
    dd = DDesc(n_q_heads, 0, 0, scale)
    rc = lib().wio_dense_attention(ctypes.byref(desc), ctypes.byref(dd), _p(K), _p(V), _p(q),
                                   _p(out))
    if rc != 0:
        raise ValueError("oracle dense attention failed")
    return out


def recall(desc, n_q_heads, idx, q, R, k):
    """recall@k of the retrieval zone R [U, n_r]: dict(recall [B, Hq],
    top [B, Hq, k] positions, top_score [B, Hq, k])."""
    U = desc.batch * desc.n_kv_heads
    R = np.ascontiguousarray(R, dtype=np.int32).reshape(U, -1)
    q = np.ascontiguousarray(q, dtype=np.float32)
    res = dict(recall=np.empty((desc.batch, n_q_heads), np.float64),
               top=np.empty((desc.batch, n_q_heads, k), np.int32),
               top_score=np.empty((desc.batch, n_q_heads, k), np.float64))
    dd = DDesc(n_q_heads, 0, 0, 0.0)
    keep = [np.ascontiguousarray(idx[key]) for key in ("sizes", "block_off", "kblk",
                                                       "slot_token")]
    rc = lib().wio_recall(ctypes.byref(desc), ctypes.byref(dd), *[_p(a) for a in keep], _p(q),
                          _p(R), R.shape[1], k, _p(res["recall"]), _p(res["top"]),
                          _p(res["top_score"]))
    if rc != 0:
        raise ValueError("oracle recall failed (k outside [1, clustered tokens]?)")
    return res


def num_threads() -> int:
    return lib().wio_num_threads()
