"""Python access to the fp64 CPU oracle of the speculative-sampling verify step.

TEST INFRASTRUCTURE ONLY: the oracle is used by the test suite, the smoke
check and the benchmark's CPU-baseline leg.  The product path (the HIP
library and its binding) never imports this package.

The arithmetic lives in specverify_oracle.c (plain C, fp64, libm exp); this
file only builds it with gcc, loads it with ctypes and marshals numpy arrays.
Batched calls may split the sequences over host threads: ctypes releases the
GIL while the C code runs, and sequences are independent.

Every function here is pinned in tests/test_oracle_pins.py and
tests/test_philox_pin.py against facts fixed outside the oracle (closed
forms, exhaustive enumeration, chi-square tests, library routines).
"""
from __future__ import annotations

import concurrent.futures as _cf
import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "specverify_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

DTYPE_F32 = 0
DTYPE_BF16 = 1
DTYPE_F16 = 2
FLAG_ZERO_RESIDUAL = 1
FLAG_NO_CROSSING = 2
FLAG_BAD_INPUT = 4


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = [
            os.environ.get("CC", "gcc"), "-O2", "-std=c11", "-Wall", "-Wextra",
            "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
            "-o", _LIB_PATH + ".tmp", _SRC, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def build_sanitized(out: str) -> str:
    """The same oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
    (every report fatal), for a CPU test run under SPECVERIFY_ORACLE_LIB; the
    Python process needs libasan preloaded."""
    cmd = [
        os.environ.get("CC", "gcc"), "-O1", "-g", "-std=c11", "-Wall", "-Wextra",
        "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
        "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
        "-o", out, _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("SPECVERIFY_ORACLE_LIB")  # another build of the same source (sanitized)
    if not path:
        path = _LIB_PATH
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
    lib = C.CDLL(path)
    P = C.c_void_p
    lib.orc_decode.restype = C.c_double
    lib.orc_decode.argtypes = [P, C.c_int32, C.c_int64]
    lib.orc_philox4x32_10.restype = None
    lib.orc_philox4x32_10.argtypes = [P, P, P]
    lib.orc_uniform.restype = C.c_double
    lib.orc_uniform.argtypes = [C.c_uint64, C.c_uint32, C.c_uint32, C.c_uint32, C.c_uint32]
    lib.orc_row_probs.restype = C.c_int
    lib.orc_row_probs.argtypes = [P, C.c_int32, C.c_int64, C.c_double, C.c_int32, P, P]
    lib.orc_row_probs_p.restype = C.c_int
    lib.orc_row_probs_p.argtypes = [P, C.c_int32, C.c_int64, C.c_double, C.c_int32, C.c_double, P, P]
    lib.orc_row_argmax.restype = C.c_int64
    lib.orc_row_argmax.argtypes = [P, C.c_int32, C.c_int64]
    lib.orc_verify_seq_u.restype = C.c_int
    lib.orc_verify_seq_u.argtypes = [
        P, P, P, C.c_int32, C.c_int64, P, P, C.c_double, C.c_double,
        P, P, P, P, P, P, P, P, P, P,
    ]
    lib.orc_verify_seq_u_batch.restype = C.c_int
    lib.orc_verify_seq_u_batch.argtypes = [
        P, P, P, C.c_int32, C.c_int64, C.c_int64, P, P, P, P, P,
    ]
    lib.orc_verify_sample.restype = C.c_int
    lib.orc_verify_sample.argtypes = [
        C.c_int32, P, C.c_int64, C.c_int32, P, C.c_int64, P, C.c_int64, P,
        C.c_double, C.c_int32, C.c_double, C.c_uint64, C.c_uint32, C.c_double,
        C.c_int32, C.c_int32, P, P, P, P, P, P, P, P, P, P,
    ]
    lib.orc_verify_greedy.restype = C.c_int
    lib.orc_verify_greedy.argtypes = [
        C.c_int32, P, C.c_int64, C.c_int32, P, C.c_int64, P, C.c_int32, C.c_int32, P, P,
    ]
    lib.orc_verify_argmax.restype = C.c_int
    lib.orc_verify_argmax.argtypes = [
        C.c_int32, P, C.c_int64, C.c_int32, P, C.c_int64, P, C.c_int64, P,
        C.c_double, C.c_int32, C.c_double, C.c_uint64, C.c_uint32, C.c_int32, C.c_int32, P, P, P, P, P, P, P, P,
        P,
    ]
    lib.orc_draft_sample.restype = C.c_int
    lib.orc_draft_sample.argtypes = [
        C.c_int32, P, C.c_int64, C.c_int32, P, C.c_int64, C.c_double, C.c_int32, C.c_double, C.c_uint64,
        C.c_uint32, C.c_double, C.c_int32, C.c_int32, P, P, P, P, P, P,
    ]
    lib.orc_token_likelihood.restype = C.c_int
    lib.orc_token_likelihood.argtypes = [
        C.c_int32, P, C.c_int64, C.c_int32, P, C.c_int64, P, C.c_int64, C.c_double, C.c_int32, C.c_double, P,
        C.c_int32, C.c_int32, P, P, P, P, P,
    ]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _dtype_code(dtype: str) -> int:
    return {"f32": DTYPE_F32, "bf16": DTYPE_BF16, "f16": DTYPE_F16}[dtype]


def _as_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    want = np.float32 if dtype == "f32" else np.uint16
    return np.ascontiguousarray(a, dtype=want)


# --------------------------------------------------------------------------
# Philox and uniforms
# --------------------------------------------------------------------------
def philox4x32_10(counter: Sequence[int], key: Sequence[int]) -> np.ndarray:
    lib = _load()
    c = np.asarray(counter, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def uniform(seed: int, seq: int, pos: int, purpose: int, offset: int) -> float:
    return float(_load().orc_uniform(seed, seq, pos, purpose, offset))


# --------------------------------------------------------------------------
# Rows
# --------------------------------------------------------------------------
def row_probs(row: np.ndarray, dtype: str, temperature: float, top_k: int = 0, top_p: float = 1.0):
    """Temperature softmax of one logit row over its top-k kept set, then the
    top-p nucleus of that distribution (top_p < 1).

    Returns (prob[V] float64, dict(m, S, tau, kept, tau_p, margin)).
    """
    lib = _load()
    r = _as_storage(row, dtype)
    V = r.shape[0]
    prob = np.zeros(V, dtype=np.float64)
    st = np.zeros(6, dtype=np.float64)
    rc = lib.orc_row_probs_p(_ptr(r), _dtype_code(dtype), V, float(temperature), int(top_k), float(top_p),
                             _ptr(prob), _ptr(st))
    if rc == -2:
        raise MemoryError("oracle row_probs")
    return prob, dict(m=st[0], S=st[1], tau=st[2], kept=int(st[3]), tau_p=st[4], margin=st[5], ok=(rc == 0))


def row_argmax(row: np.ndarray, dtype: str) -> int:
    r = _as_storage(row, dtype)
    return int(_load().orc_row_argmax(_ptr(r), _dtype_code(dtype), r.shape[0]))


# --------------------------------------------------------------------------
# The verify core with explicit uniforms
# --------------------------------------------------------------------------
def verify_seq_u(P: np.ndarray, Q: np.ndarray, x: Sequence[int], u_acc, u_res, u_bonus: float,
                 eps: float = 1e-6) -> dict:
    """One sequence: P [K+1, V] target probs, Q [K, V] draft probs, x [K] ids."""
    lib = _load()
    P = np.ascontiguousarray(P, dtype=np.float64)
    K = P.shape[0] - 1
    V = P.shape[1]
    Q = np.ascontiguousarray(Q, dtype=np.float64).reshape(K, V) if K > 0 else np.zeros((1, V))
    x = np.ascontiguousarray(x, dtype=np.int32).reshape(K) if K > 0 else np.zeros(1, np.int32)
    ua = np.ascontiguousarray(u_acc, dtype=np.float64).reshape(-1) if K > 0 else np.zeros(1)
    ur = np.ascontiguousarray(u_res, dtype=np.float64).reshape(-1) if K > 0 else np.zeros(1)
    tokens = np.zeros(K + 1, np.int32)
    n = np.zeros(1, np.int32)
    p = np.zeros(max(K, 1))
    q = np.zeros(max(K, 1))
    z = np.zeros(1)
    dacc = np.zeros(max(K, 1))
    dfin = np.zeros(1)
    lo = np.zeros(1, np.int32)
    hi = np.zeros(1, np.int32)
    fl = np.zeros(1, np.int32)
    rc = lib.orc_verify_seq_u(_ptr(P), _ptr(Q), _ptr(x), K, V, _ptr(ua), _ptr(ur), float(u_bonus),
                              float(eps), _ptr(tokens), _ptr(n), _ptr(p), _ptr(q), _ptr(z),
                              _ptr(dacc), _ptr(dfin), _ptr(lo), _ptr(hi), _ptr(fl))
    return dict(rc=rc, tokens=tokens, n=int(n[0]), p=p[:K], q=q[:K], z=float(z[0]),
                d_acc=dacc[:K], d_fin=float(dfin[0]), tok_lo=int(lo[0]), tok_hi=int(hi[0]),
                flags=int(fl[0]))


def verify_seq_u_batch(P, Q, x, u_acc, u_res, u_bonus):
    """The core over many uniform sets; returns (tokens [T, K+1], n [T])."""
    lib = _load()
    P = np.ascontiguousarray(P, dtype=np.float64)
    K = P.shape[0] - 1
    V = P.shape[1]
    Q = np.ascontiguousarray(Q, dtype=np.float64)
    x = np.ascontiguousarray(x, dtype=np.int32)
    ub = np.ascontiguousarray(u_bonus, dtype=np.float64).reshape(-1)
    T = ub.shape[0]
    ua = np.ascontiguousarray(u_acc, dtype=np.float64).reshape(T * max(K, 0))
    ur = np.ascontiguousarray(u_res, dtype=np.float64).reshape(T * max(K, 0))
    if K == 0:
        ua = np.zeros(1)
        ur = np.zeros(1)
        Q = np.zeros((1, V))
        x = np.zeros(1, np.int32)
    tokens = np.zeros((T, K + 1), np.int32)
    n = np.zeros(T, np.int32)
    rc = lib.orc_verify_seq_u_batch(_ptr(P), _ptr(Q), _ptr(x), K, V, T, _ptr(ua), _ptr(ur),
                                    _ptr(ub), _ptr(tokens), _ptr(n))
    if rc != 0:
        raise ValueError("oracle batch core rejected its input")
    return tokens, n


# --------------------------------------------------------------------------
# Batched, seeded verify over a packed ragged batch
# --------------------------------------------------------------------------
def _ranges(B, seqs, threads):
    if seqs is not None:
        return [(int(b), int(b) + 1) for b in seqs]
    nthr = max(1, min(threads or 1, B))
    step = (B + nthr - 1) // nthr
    return [(s, min(B, s + step)) for s in range(0, B, step)]


def _run(fn, ranges, threads):
    if (threads or 1) <= 1 or len(ranges) <= 1:
        return [fn(r) for r in ranges]
    with _cf.ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, ranges))


def verify_sample(target, draft, draft_ids, cu_draft, vocab: int, dtype: str,
                  temperature: float, top_k: int, seed: int, offset: int,
                  eps: float = 1e-6, seqs: Optional[Sequence[int]] = None,
                  threads: Optional[int] = None, target_stride: Optional[int] = None,
                  draft_stride: Optional[int] = None, top_p: float = 1.0) -> dict:
    """Seeded speculative verify over a batch; mirrors the library's outputs.

    Returns tokens [R_t], num_accepted [B], probs [R_d, 2] (p, q of each
    draft id), residual_mass [B], plus diagnostics: d_acc [R_d] (distance
    of each evaluated accept draw to its threshold, inf if not evaluated),
    d_fin [B] (distance of the final draw to its interval edges), tok_lo /
    tok_hi [B] (ids whose interval meets the eps-window), flags [B] and
    p_margin [B] (the sequence's smallest top-p margin; inf without top-p).
    Sequences not listed in `seqs` keep sentinel values (-2 / nan).
    """
    lib = _load()
    cu = np.ascontiguousarray(cu_draft, dtype=np.int32)
    B = cu.shape[0] - 1
    R_d = int(cu[-1])
    R_t = R_d + B
    tgt = _as_storage(target, dtype)
    drf = _as_storage(draft, dtype) if R_d > 0 else np.zeros((1, vocab), tgt.dtype)
    ids = np.ascontiguousarray(draft_ids, dtype=np.int32) if R_d > 0 else np.zeros(1, np.int32)
    ts = int(target_stride or (tgt.shape[-1] if tgt.ndim == 2 else vocab))
    ds = int(draft_stride or (drf.shape[-1] if drf.ndim == 2 else vocab))
    out = dict(
        tokens=np.full(R_t, -2, np.int32),
        num_accepted=np.full(B, -2, np.int32),
        probs=np.full((max(R_d, 1), 2), np.nan),
        residual_mass=np.full(B, np.nan),
        d_acc=np.full(max(R_d, 1), np.inf),
        d_fin=np.full(B, np.nan),
        tok_lo=np.full(B, -2, np.int32),
        tok_hi=np.full(B, -2, np.int32),
        flags=np.zeros(B, np.int32),
        p_margin=np.full(B, np.nan),
    )
    o = out

    def fn(rng):
        return lib.orc_verify_sample(
            B, _ptr(cu), vocab, _dtype_code(dtype), _ptr(tgt), ts, _ptr(drf), ds, _ptr(ids),
            float(temperature), int(top_k), float(top_p), int(seed), int(offset), float(eps), rng[0], rng[1],
            _ptr(o["tokens"]), _ptr(o["num_accepted"]), _ptr(o["probs"]),
            _ptr(o["residual_mass"]), _ptr(o["d_acc"]), _ptr(o["d_fin"]), _ptr(o["tok_lo"]),
            _ptr(o["tok_hi"]), _ptr(o["flags"]), _ptr(o["p_margin"]))

    rcs = _run(fn, _ranges(B, seqs, threads), threads)
    if any(rc == -2 for rc in rcs):
        raise MemoryError("oracle verify_sample")
    out["probs"] = out["probs"][:R_d]
    out["d_acc"] = out["d_acc"][:R_d]
    out["rc"] = min(rcs) if rcs else 0
    return out


def verify_greedy(target, draft_ids, cu_draft, vocab: int, dtype: str,
                  seqs: Optional[Sequence[int]] = None, threads: Optional[int] = None,
                  target_stride: Optional[int] = None) -> dict:
    lib = _load()
    cu = np.ascontiguousarray(cu_draft, dtype=np.int32)
    B = cu.shape[0] - 1
    R_d = int(cu[-1])
    R_t = R_d + B
    tgt = _as_storage(target, dtype)
    ids = np.ascontiguousarray(draft_ids, dtype=np.int32) if R_d > 0 else np.zeros(1, np.int32)
    ts = int(target_stride or (tgt.shape[-1] if tgt.ndim == 2 else vocab))
    tokens = np.full(R_t, -2, np.int32)
    nacc = np.full(B, -2, np.int32)

    def fn(rng):
        return lib.orc_verify_greedy(B, _ptr(cu), vocab, _dtype_code(dtype), _ptr(tgt), ts,
                                     _ptr(ids), rng[0], rng[1], _ptr(tokens), _ptr(nacc))

    _run(fn, _ranges(B, seqs, threads), threads)
    return dict(tokens=tokens, num_accepted=nacc)


def verify_argmax(target, draft, draft_ids, cu_draft, vocab: int, dtype: str, temperature: float, top_k: int,
                  seed: int, offset: int, seqs: Optional[Sequence[int]] = None, threads: Optional[int] = None,
                  target_stride: Optional[int] = None, draft_stride: Optional[int] = None,
                  top_p: float = 1.0) -> dict:
    """The argmax-draw variant: the sampling variant's acceptance test, then
    the argmax of max(0, p_n - q_n) at a rejection or of p_K when all pass.

    Returns tokens, num_accepted, probs, residual_mass, d_acc and, per
    sequence, gap (relative margin of the final argmax over its runner-up),
    second (the runner-up's id) and flags.
    """
    lib = _load()
    cu = np.ascontiguousarray(cu_draft, dtype=np.int32)
    B = cu.shape[0] - 1
    R_d = int(cu[-1])
    R_t = R_d + B
    tgt = _as_storage(target, dtype)
    drf = _as_storage(draft, dtype) if R_d > 0 else np.zeros((1, vocab), tgt.dtype)
    ids = np.ascontiguousarray(draft_ids, dtype=np.int32) if R_d > 0 else np.zeros(1, np.int32)
    ts = int(target_stride or (tgt.shape[-1] if tgt.ndim == 2 else vocab))
    ds = int(draft_stride or (drf.shape[-1] if drf.ndim == 2 else vocab))
    o = dict(tokens=np.full(R_t, -2, np.int32), num_accepted=np.full(B, -2, np.int32),
             probs=np.full((max(R_d, 1), 2), np.nan), residual_mass=np.full(B, np.nan),
             d_acc=np.full(max(R_d, 1), np.inf), gap=np.full(B, np.nan), second=np.full(B, -2, np.int32),
             flags=np.zeros(B, np.int32), p_margin=np.full(B, np.nan))

    def fn(rng):
        return lib.orc_verify_argmax(
            B, _ptr(cu), vocab, _dtype_code(dtype), _ptr(tgt), ts, _ptr(drf), ds, _ptr(ids), float(temperature),
            int(top_k), float(top_p), int(seed), int(offset), rng[0], rng[1], _ptr(o["tokens"]),
            _ptr(o["num_accepted"]), _ptr(o["probs"]), _ptr(o["residual_mass"]), _ptr(o["d_acc"]), _ptr(o["gap"]),
            _ptr(o["second"]), _ptr(o["flags"]), _ptr(o["p_margin"]))

    rcs = _run(fn, _ranges(B, seqs, threads), threads)
    if any(rc == -2 for rc in rcs):
        raise MemoryError("oracle verify_argmax")
    o["probs"] = o["probs"][:R_d]
    o["d_acc"] = o["d_acc"][:R_d]
    o["rc"] = min(rcs) if rcs else 0
    return o


def draft_sample(draft, cu_draft, vocab: int, dtype: str, temperature: float, top_k: int, seed: int, offset: int,
                 eps: float = 1e-6, seqs: Optional[Sequence[int]] = None, threads: Optional[int] = None,
                 draft_stride: Optional[int] = None, top_p: float = 1.0) -> dict:
    """Seeded draft-side sampling: x(b, k) ~ q_k by the inverse CDF with U(b, k, 3).

    Returns ids [R_d] and, per draft row, dist (distance of u to the chosen
    id's interval edges), tok_lo / tok_hi (ids whose interval meets the
    eps-window) and flags.  Rows of sequences not listed in `seqs` keep -2.
    """
    lib = _load()
    cu = np.ascontiguousarray(cu_draft, dtype=np.int32)
    B = cu.shape[0] - 1
    R_d = int(cu[-1])
    n = max(R_d, 1)
    drf = _as_storage(draft, dtype) if R_d > 0 else np.zeros((1, vocab), np.float32 if dtype == "f32" else np.uint16)
    ds = int(draft_stride or (drf.shape[-1] if drf.ndim == 2 else vocab))
    out = dict(ids=np.full(n, -2, np.int32), dist=np.full(n, np.nan), tok_lo=np.full(n, -2, np.int32),
               tok_hi=np.full(n, -2, np.int32), flags=np.zeros(n, np.int32), p_margin=np.full(n, np.nan))
    o = out

    def fn(rng):
        return lib.orc_draft_sample(B, _ptr(cu), vocab, _dtype_code(dtype), _ptr(drf), ds, float(temperature),
                                    int(top_k), float(top_p), int(seed), int(offset), float(eps), rng[0], rng[1],
                                    _ptr(o["ids"]), _ptr(o["dist"]), _ptr(o["tok_lo"]), _ptr(o["tok_hi"]),
                                    _ptr(o["flags"]), _ptr(o["p_margin"]))

    rcs = _run(fn, _ranges(B, seqs, threads), threads)
    if any(rc == -2 for rc in rcs):
        raise MemoryError("oracle draft_sample")
    for k in out:
        out[k] = out[k][:R_d]
    out["rc"] = min(rcs) if rcs else 0
    return out


def token_likelihood(target, draft, tokens, cu_draft, vocab: int, dtype: str, temperature: float, top_k: int,
                     seqs: Optional[Sequence[int]] = None, threads: Optional[int] = None,
                     target_stride: Optional[int] = None, draft_stride: Optional[int] = None,
                     top_p: float = 1.0) -> dict:
    """Per-token speculative likelihood of tokens[r] at row r of both tensors
    (position (b, k) is row cu_draft[b] + k).

    Returns accept [R] = q(y) min(1, p(y)/q(y)), reject [R] = (1 - beta) p'(y),
    p [R] = p(y), beta [R] = sum_v min(p, q), and per sequence nll [B] =
    -sum_k log(accept + reject) and flags.
    """
    lib = _load()
    cu = np.ascontiguousarray(cu_draft, dtype=np.int32)
    B = cu.shape[0] - 1
    R = int(cu[-1])
    n = max(R, 1)
    empty = np.zeros((1, vocab), np.float32 if dtype == "f32" else np.uint16)
    tgt = _as_storage(target, dtype) if R > 0 else empty
    drf = _as_storage(draft, dtype) if R > 0 else empty
    tok = np.ascontiguousarray(tokens, dtype=np.int32) if R > 0 else np.zeros(1, np.int32)
    ts = int(target_stride or (tgt.shape[-1] if tgt.ndim == 2 else vocab))
    ds = int(draft_stride or (drf.shape[-1] if drf.ndim == 2 else vocab))
    terms = np.full((n, 3), np.nan)
    beta = np.full(n, np.nan)
    nll = np.full(B, np.nan)
    flags = np.zeros(B, np.int32)
    pm = np.full(n, np.nan)

    def fn(rng):
        return lib.orc_token_likelihood(B, _ptr(cu), vocab, _dtype_code(dtype), _ptr(tgt), ts, _ptr(drf), ds,
                                        float(temperature), int(top_k), float(top_p), _ptr(tok), rng[0], rng[1],
                                        _ptr(terms), _ptr(beta), _ptr(nll), _ptr(flags), _ptr(pm))

    rcs = _run(fn, _ranges(B, seqs, threads), threads)
    if any(rc == -2 for rc in rcs):
        raise MemoryError("oracle token_likelihood")
    return dict(accept=terms[:R, 0], reject=terms[:R, 1], p=terms[:R, 2], beta=beta[:R], nll=nll, flags=flags,
                p_margin=pm[:R], rc=min(rcs) if rcs else 0)


def verify_workload(w, mode: str = "sample", **kw) -> dict:
    """Convenience: run the oracle on a workloads.Workload.

    mode: "sample", "greedy", "argmax" (argmax draws), "draft" (draft-side sampling) or
    "likelihood" (per-token speculative likelihood of the guesses, rows from w.likelihood_rows())."""
    if mode == "likelihood":
        tgt, drf, tok = w.likelihood_rows()
        return token_likelihood(tgt, drf, tok, w.cu_draft, w.vocab, w.dtype, w.temperature, w.top_k,
                                top_p=w.top_p, **kw)
    if mode == "draft":
        return draft_sample(w.draft, w.cu_draft, w.vocab, w.dtype, w.temperature, w.top_k, w.seed, w.offset,
                            top_p=w.top_p, **kw)
    if mode == "argmax":
        return verify_argmax(w.target, w.draft, w.draft_ids, w.cu_draft, w.vocab, w.dtype, w.temperature, w.top_k,
                             w.seed, w.offset, top_p=w.top_p, **kw)
    if mode == "greedy":
        return verify_greedy(w.target, w.draft_ids, w.cu_draft, w.vocab, w.dtype, **kw)
    return verify_sample(w.target, w.draft, w.draft_ids, w.cu_draft, w.vocab, w.dtype,
                         w.temperature, w.top_k, w.seed, w.offset, top_p=w.top_p, **kw)
