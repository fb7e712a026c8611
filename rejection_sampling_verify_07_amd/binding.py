"""ctypes binding of libspecverify (the C ABI in include/specverify.h).

Argument marshalling only: torch supplies device memory and the stream;
every step of the verify path runs in the HIP kernels of the library.  There
is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_OK = 0
SV_ERR_INVALID_ARGUMENT = 1
SV_ERR_UNSUPPORTED = 2
SV_ERR_WORKSPACE_TOO_SMALL = 3
SV_ERR_HIP = 4
SV_DTYPE_F32 = 0
SV_DTYPE_BF16 = 1
SV_DTYPE_F16 = 2
MAX_VOCAB = 1 << 20
MAX_DRAFT = 128


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


class ProfileEventsT(C.Structure):
    """sv_profile_events_t (specverify_profile.h): two raw HIP events."""
    _fields_ = [("start", C.c_void_p), ("stop", C.c_void_p)]


class ShapeT(C.Structure):
    _fields_ = [
        ("batch", C.c_int32),
        ("max_draft", C.c_int32),
        ("total_draft", C.c_int32),
        ("vocab", C.c_int32),
        ("dtype", C.c_int32),
        ("target_row_stride", C.c_int64),
        ("draft_row_stride", C.c_int64),
        ("cu_draft", C.c_void_p),
    ]


_lib = None


def load_library(path: Optional[str] = None):
    """Load libspecverify.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("SPECVERIFY_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"{p} is missing: build the HIP library first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = C.CDLL(p)
    VP = C.c_void_p
    lib.spec_verify_sample.restype = C.c_int
    lib.spec_verify_sample.argtypes = [
        C.POINTER(ShapeT), VP, VP, VP, C.c_float, C.c_int32, C.c_float, C.c_uint64, C.c_uint32,
        VP, VP, VP, VP, VP, C.POINTER(C.c_size_t), VP,
    ]
    lib.spec_verify_argmax.restype = C.c_int
    lib.spec_verify_argmax.argtypes = lib.spec_verify_sample.argtypes
    lib.spec_verify_sample_noalloc.restype = C.c_int
    lib.spec_verify_sample_noalloc.argtypes = [
        C.POINTER(ShapeT), VP, VP, VP, C.c_float, C.c_int32, C.c_float, C.c_uint64, C.c_uint32, VP, VP, VP, VP, VP,
    ]
    lib.spec_verify_greedy.restype = C.c_int
    lib.spec_verify_greedy.argtypes = [C.POINTER(ShapeT), VP, VP, VP, VP, VP, C.POINTER(C.c_size_t), VP]
    lib.spec_draft_sample.restype = C.c_int
    lib.spec_draft_sample.argtypes = [
        C.POINTER(ShapeT), VP, C.c_float, C.c_int32, C.c_float, C.c_uint64, C.c_uint32, VP, VP,
        C.POINTER(C.c_size_t), VP,
    ]
    lib.spec_token_likelihood.restype = C.c_int
    lib.spec_token_likelihood.argtypes = [
        C.POINTER(ShapeT), VP, VP, VP, C.c_float, C.c_int32, C.c_float, VP, VP, VP, VP, C.POINTER(C.c_size_t),
        VP,
    ]
    lib.spec_profile_stream_read.restype = C.c_int
    lib.spec_profile_stream_read.argtypes = [C.POINTER(ProfileEventsT), VP, C.c_size_t, VP, VP]
    lib.spec_verify_status_string.restype = C.c_char_p
    lib.spec_verify_status_string.argtypes = [C.c_int]
    # benchmark entry points: the same calls with a leading events argument
    for name in ("spec_verify_sample", "spec_verify_argmax", "spec_verify_greedy", "spec_draft_sample",
                 "spec_token_likelihood"):
        f = getattr(lib, name + "_profiled")
        f.restype = C.c_int
        f.argtypes = [C.POINTER(ProfileEventsT)] + list(getattr(lib, name).argtypes)
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().spec_verify_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != SV_OK:
        raise SpecVerifyError(status, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SV_DTYPE_BF16
    if t.dtype == torch.float16:
        return SV_DTYPE_F16
    raise TypeError(f"logits must be float32, bfloat16 or float16, got {t.dtype}")


def _rows(t: torch.Tensor, name: str):
    if t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if t.numel() == 0:
        return t.shape[1]  # no element is read; an empty tensor may report stride 0
    if t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return t.stride(0)


def make_shape(target: torch.Tensor, draft: Optional[torch.Tensor], batch: int, max_draft: int,
               total_draft: int, cu_draft: Optional[torch.Tensor], target_rows: int,
               draft_rows: int = 0) -> ShapeT:
    """The C shape of a call.  target_rows / draft_rows: the rows the call
    reads from each tensor (the kernels index rows by the geometry, so a tensor
    that is shorter, or of another element type or width than the other, would
    be read past its end)."""
    if target.dim() != 2:
        raise ValueError("target_logits must be a 2-D tensor with unit column stride")
    vocab = target.shape[1]
    if target.shape[0] < target_rows:
        raise ValueError(f"target_logits has {target.shape[0]} rows; the batch needs {target_rows}")
    other = draft is not None and draft is not target
    if other:
        if draft.dtype != target.dtype:
            raise ValueError(f"draft_logits is {draft.dtype} but target_logits is {target.dtype}")
        if draft.dim() != 2 or draft.shape[1] != vocab:
            raise ValueError(f"draft_logits must have {vocab} columns, like target_logits")
        if draft.shape[0] < draft_rows:
            raise ValueError(f"draft_logits has {draft.shape[0]} rows; the batch needs {draft_rows}")
    ts = _rows(target, "target_logits")
    if draft is target:  # draft-side sampling: the draft rows are the one tensor
        ds = ts
    else:
        ds = _rows(draft, "draft_logits") if (other and draft.numel() > 0) else vocab
    return ShapeT(
        batch=batch, max_draft=max_draft, total_draft=total_draft, vocab=vocab, dtype=_dtype_code(target),
        target_row_stride=ts, draft_row_stride=ds,
        cu_draft=(cu_draft.data_ptr() if cu_draft is not None else None),
    )


def _batch_geometry(target, draft_ids, cu_draft, max_draft):
    total = draft_ids.numel()
    if cu_draft is None:
        batch = target.shape[0] - total  # rows_t = sum(K_b) + B
        if batch <= 0 or total % batch != 0:
            raise ValueError("target rows must be B*(K+1) for B*K draft ids; pass cu_draft for ragged K")
        k = total // batch
        if max_draft is not None and max_draft != k:
            raise ValueError("max_draft does not match the uniform draft length")
        return batch, k, total
    if cu_draft.dtype != torch.int32 or cu_draft.dim() != 1:
        raise ValueError("cu_draft must be a 1-D int32 tensor")
    batch = cu_draft.numel() - 1
    if batch < 1:
        raise ValueError("cu_draft needs B + 1 >= 2 entries")
    if target.shape[0] < total + batch:
        raise ValueError(f"target_logits has {target.shape[0]} rows; {batch} sequences with {total} draft ids "
                         f"need {total + batch}")
    if max_draft is None:
        max_draft = int((cu_draft[1:] - cu_draft[:-1]).max().item()) if batch > 0 else 0
    return batch, max_draft, total


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def verify_sample(target_logits: torch.Tensor, draft_logits: torch.Tensor, draft_ids: torch.Tensor,
                  cu_draft: Optional[torch.Tensor] = None, temperature: float = 1.0, top_k: int = 0,
                  seed: int = 0, offset: int = 0, max_draft: Optional[int] = None, return_probs: bool = True,
                  workspace: Optional[torch.Tensor] = None, out: Optional[dict] = None, stream=None,
                  argmax: bool = False, top_p: float = 1.0) -> dict:
    """Speculative-sampling verify on the GPU (spec_verify_sample, or
    spec_verify_argmax with argmax=True: argmax draws).

    target_logits [sum(K_b+1), V] and draft_logits [sum(K_b), V], float32,
    bfloat16 or float16, rows packed as in include/specverify.h; draft_ids int32
    [sum(K_b)]; cu_draft int32 [B+1] prefix sums or None (uniform K).
    Returns tokens [sum(K_b+1)], num_accepted [B], probs [sum(K_b), 2] and
    residual_mass [B] (the last two when return_probs).
    """
    lib = load_library()
    fn = lib.spec_verify_argmax if argmax else lib.spec_verify_sample
    name = "spec_verify_argmax" if argmax else "spec_verify_sample"
    batch, kmax, total = _batch_geometry(target_logits, draft_ids, cu_draft, max_draft)
    if draft_ids.dtype != torch.int32:
        raise TypeError("draft_ids must be int32")
    shape = make_shape(target_logits, draft_logits, batch, kmax, total, cu_draft, total + batch, total)
    dev = target_logits.device
    need = C.c_size_t(0)
    _check(fn(C.byref(shape), None, None, None, float(temperature), int(top_k), float(top_p), int(seed),
              int(offset), None, None, None, None, None, C.byref(need), None), name + "(workspace query)")
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = dict(
            tokens=torch.empty(total + batch, dtype=torch.int32, device=dev),
            num_accepted=torch.empty(batch, dtype=torch.int32, device=dev),
        )
        if return_probs:
            out["probs"] = torch.empty((max(total, 1), 2), dtype=torch.float32, device=dev)[:total]
            out["residual_mass"] = torch.empty(batch, dtype=torch.float32, device=dev)
    have = C.c_size_t(workspace.numel())
    st = fn(
        C.byref(shape), target_logits.data_ptr(), draft_logits.data_ptr() if draft_logits.numel() else None,
        draft_ids.data_ptr() if draft_ids.numel() else None, float(temperature), int(top_k), float(top_p), int(seed),
        int(offset),
        out["tokens"].data_ptr(), out["num_accepted"].data_ptr(),
        out["probs"].data_ptr() if out.get("probs") is not None and total > 0 else None,
        out["residual_mass"].data_ptr() if out.get("residual_mass") is not None else None,
        workspace.data_ptr(), C.byref(have), C.c_void_p(_stream_handle(stream)))
    _check(st, name)
    return out


def verify_sample_noalloc(target_logits: torch.Tensor, draft_logits: torch.Tensor, draft_ids: torch.Tensor,
                          cu_draft: Optional[torch.Tensor] = None, temperature: float = 1.0, top_k: int = 0,
                          seed: int = 0, offset: int = 0, max_draft: Optional[int] = None, out: Optional[dict] = None,
                          stream=None, top_p: float = 1.0) -> dict:
    """spec_verify_sample_noalloc: verify_sample with the library's own
    per-device scratch instead of a workspace (the library allocates nothing;
    calls that overlap on one GPU race).  `out` (tokens, num_accepted, probs,
    residual_mass) may be preallocated; otherwise it is allocated here."""
    lib = load_library()
    batch, kmax, total = _batch_geometry(target_logits, draft_ids, cu_draft, max_draft)
    if draft_ids.dtype != torch.int32:
        raise TypeError("draft_ids must be int32")
    shape = make_shape(target_logits, draft_logits, batch, kmax, total, cu_draft, total + batch, total)
    dev = target_logits.device
    if out is None:
        out = dict(tokens=torch.empty(total + batch, dtype=torch.int32, device=dev),
                   num_accepted=torch.empty(batch, dtype=torch.int32, device=dev),
                   probs=torch.empty((max(total, 1), 2), dtype=torch.float32, device=dev)[:total],
                   residual_mass=torch.empty(batch, dtype=torch.float32, device=dev))
    st = lib.spec_verify_sample_noalloc(
        C.byref(shape), target_logits.data_ptr(), draft_logits.data_ptr() if draft_logits.numel() else None,
        draft_ids.data_ptr() if draft_ids.numel() else None, float(temperature), int(top_k), float(top_p), int(seed),
        int(offset), out["tokens"].data_ptr(), out["num_accepted"].data_ptr(),
        out["probs"].data_ptr() if out.get("probs") is not None and total > 0 else None,
        out["residual_mass"].data_ptr() if out.get("residual_mass") is not None else None,
        C.c_void_p(_stream_handle(stream)))
    _check(st, "spec_verify_sample_noalloc")
    return out


def verify_argmax(*args, **kw) -> dict:
    """spec_verify_argmax: verify_sample's acceptance test, argmax draws."""
    return verify_sample(*args, argmax=True, **kw)


def verify_greedy(target_logits: torch.Tensor, draft_ids: torch.Tensor, cu_draft: Optional[torch.Tensor] = None,
                  max_draft: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                  out: Optional[dict] = None, stream=None) -> dict:
    """Greedy argmax-compare verify on the GPU (spec_verify_greedy)."""
    lib = load_library()
    batch, kmax, total = _batch_geometry(target_logits, draft_ids, cu_draft, max_draft)
    if draft_ids.dtype != torch.int32:
        raise TypeError("draft_ids must be int32")
    shape = make_shape(target_logits, None, batch, kmax, total, cu_draft, total + batch)
    dev = target_logits.device
    need = C.c_size_t(0)
    _check(lib.spec_verify_greedy(C.byref(shape), None, None, None, None, None, C.byref(need), None),
           "spec_verify_greedy(workspace query)")
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = dict(
            tokens=torch.empty(total + batch, dtype=torch.int32, device=dev),
            num_accepted=torch.empty(batch, dtype=torch.int32, device=dev),
        )
    have = C.c_size_t(workspace.numel())
    st = lib.spec_verify_greedy(C.byref(shape), target_logits.data_ptr(),
                                draft_ids.data_ptr() if draft_ids.numel() else None, out["tokens"].data_ptr(),
                                out["num_accepted"].data_ptr(), workspace.data_ptr(), C.byref(have),
                                C.c_void_p(_stream_handle(stream)))
    _check(st, "spec_verify_greedy")
    return out


def _draft_geometry(draft_logits, cu_draft, batch, max_draft):
    total = draft_logits.shape[0]
    if cu_draft is None:
        if batch is None or batch <= 0 or total % batch != 0:
            raise ValueError("pass batch (rows = batch * K) or cu_draft for ragged K")
        k = total // batch
        if max_draft is not None and max_draft != k:
            raise ValueError("max_draft does not match the uniform draft length")
        return batch, k, total
    if cu_draft.dtype != torch.int32 or cu_draft.dim() != 1:
        raise ValueError("cu_draft must be a 1-D int32 tensor")
    b = cu_draft.numel() - 1
    if max_draft is None:
        max_draft = int((cu_draft[1:] - cu_draft[:-1]).max().item()) if b > 0 else 0
    return b, max_draft, total


def draft_sample(draft_logits: torch.Tensor, cu_draft: Optional[torch.Tensor] = None, batch: Optional[int] = None,
                 temperature: float = 1.0, top_k: int = 0, seed: int = 0, offset: int = 0,
                 max_draft: Optional[int] = None, workspace: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None, stream=None, top_p: float = 1.0) -> torch.Tensor:
    """Draft-side sampling on the GPU (spec_draft_sample): x(b, k) ~ q_k.

    draft_logits [sum(K_b), V] float32, bfloat16 or float16, rows packed as for the
    verify; cu_draft int32 [B+1] or None with `batch` (uniform K).  Returns
    the int32 ids [sum(K_b)].
    """
    lib = load_library()
    b, kmax, total = _draft_geometry(draft_logits, cu_draft, batch, max_draft)
    shape = make_shape(draft_logits, draft_logits, b, kmax, total, cu_draft, total)
    dev = draft_logits.device
    need = C.c_size_t(0)
    _check(lib.spec_draft_sample(C.byref(shape), None, float(temperature), int(top_k), float(top_p), int(seed),
                                 int(offset), None, None, C.byref(need), None), "spec_draft_sample(workspace query)")
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty(max(total, 1), dtype=torch.int32, device=dev)[:total]
    have = C.c_size_t(workspace.numel())
    st = lib.spec_draft_sample(C.byref(shape), draft_logits.data_ptr() if total else None, float(temperature),
                               int(top_k), float(top_p), int(seed), int(offset), out.data_ptr() if total else None,
                               workspace.data_ptr(), C.byref(have), C.c_void_p(_stream_handle(stream)))
    _check(st, "spec_draft_sample")
    return out


def _likelihood_outputs(total, batch, dev, terms, beta, nll):
    out = {}
    if terms:
        out["terms"] = torch.empty((max(total, 1), 2), dtype=torch.float32, device=dev)[:total]
    if beta:
        out["beta"] = torch.empty(max(total, 1), dtype=torch.float32, device=dev)[:total]
    if nll:
        out["nll"] = torch.empty(batch, dtype=torch.float64, device=dev)
    if not out:
        raise ValueError("ask for at least one of terms, beta, nll")
    return out


def _ptr_or_none(out, key):
    t = out.get(key)
    return t.data_ptr() if t is not None and t.numel() > 0 else None


def token_likelihood(target_logits: torch.Tensor, draft_logits: torch.Tensor, tokens: torch.Tensor,
                     cu_draft: Optional[torch.Tensor] = None, batch: Optional[int] = None, temperature: float = 1.0,
                     top_k: int = 0, max_draft: Optional[int] = None, terms: bool = True, beta: bool = True,
                     nll: bool = True, workspace: Optional[torch.Tensor] = None, stream=None,
                     top_p: float = 1.0) -> dict:
    """Per-token speculative likelihood on the GPU (spec_token_likelihood).

    target_logits and draft_logits [sum(K_b), V] (float32, bfloat16 or
    float16; position (b, k) is row cu_draft[b] + k of both), tokens int32
    [sum(K_b)]; cu_draft int32 [B+1] or None with `batch` (uniform K).
    Returns terms [sum(K_b), 2] (accept part, reject part), beta [sum(K_b)]
    and nll [B] (float64), each when asked for.
    """
    lib = load_library()
    if tokens.dtype != torch.int32:
        raise TypeError("tokens must be int32")
    if target_logits.shape[0] != draft_logits.shape[0] or target_logits.shape[0] != tokens.numel():
        raise ValueError("target_logits, draft_logits and tokens need one row per position")
    b, kmax, total = _draft_geometry(draft_logits, cu_draft, batch, max_draft)
    shape = make_shape(target_logits, draft_logits, b, kmax, total, cu_draft, total, total)
    dev = target_logits.device
    need = C.c_size_t(0)
    _check(lib.spec_token_likelihood(C.byref(shape), None, None, None, float(temperature), int(top_k), float(top_p),
                                     None, None, None, None, C.byref(need), None),
           "spec_token_likelihood(workspace query)")
    if workspace is None or workspace.numel() < need.value:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
    out = _likelihood_outputs(total, b, dev, terms, beta, nll)
    have = C.c_size_t(workspace.numel())
    st = lib.spec_token_likelihood(
        C.byref(shape), target_logits.data_ptr() if total else None, draft_logits.data_ptr() if total else None,
        tokens.data_ptr() if total else None, float(temperature), int(top_k), float(top_p), _ptr_or_none(out, "terms"),
        _ptr_or_none(out, "beta"), _ptr_or_none(out, "nll"), workspace.data_ptr(), C.byref(have),
        C.c_void_p(_stream_handle(stream)))
    _check(st, "spec_token_likelihood")
    return out


def workspace_bytes(target_logits, draft_logits, draft_ids, cu_draft=None, top_k=0, max_draft=None,
                    greedy=False) -> int:
    lib = load_library()
    batch, kmax, total = _batch_geometry(target_logits, draft_ids, cu_draft, max_draft)
    shape = make_shape(target_logits, None if greedy else draft_logits, batch, kmax, total, cu_draft, total + batch,
                       0 if greedy else total)
    need = C.c_size_t(0)
    if greedy:
        st = lib.spec_verify_greedy(C.byref(shape), None, None, None, None, None, C.byref(need), None)
    else:
        st = lib.spec_verify_sample(C.byref(shape), None, None, None, 1.0, int(top_k), 1.0, 0, 0, None, None, None,
                                    None, None, C.byref(need), None)
    _check(st, "workspace query")
    return need.value


class HipEvents:
    """n pairs of raw HIP events (created eagerly), passed one pair per call
    to the *_profiled entry points, which record them around the streaming
    kernel of that call."""

    def __init__(self, n: int):
        self._hip = C.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self._hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.n = n
        self.pairs = (ProfileEventsT * n)()
        for i in range(n):
            for field in ("start", "stop"):
                h = C.c_void_p()
                if self._hip.hipEventCreate(C.byref(h)) != 0:
                    raise RuntimeError("hipEventCreate failed")
                setattr(self.pairs[i], field, h.value)

    def pair(self, i: int):
        """A pointer to pair i, the leading argument of a *_profiled call."""
        return C.pointer(self.pairs[i])

    def elapsed_ms(self):
        """Per-call durations (ms) of the streaming kernel; call after a device sync."""
        out = []
        for i in range(self.n):
            ms = C.c_float(0)
            if self._hip.hipEventElapsedTime(C.byref(ms), self.pairs[i].start, self.pairs[i].stop) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(ms.value)
        return out

    def close(self):
        for i in range(self.n):
            self._hip.hipEventDestroy(self.pairs[i].start)
            self._hip.hipEventDestroy(self.pairs[i].stop)
        self.n = 0


class StreamReadPlan:
    """spec_profile_stream_read over one device buffer (benchmark only): a
    plain read of its bytes with the streaming passes' loads and tiles."""

    def __init__(self, buf: torch.Tensor, stream=None):
        self.lib = load_library()
        self.buf = buf
        self.nbytes = buf.numel() * buf.element_size() // 16 * 16
        self.sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
        self.args = (C.c_void_p(buf.data_ptr()), C.c_size_t(self.nbytes), C.c_void_p(self.sink.data_ptr()),
                     C.c_void_p(_stream_handle(stream)))

    def profiled(self, events):
        _check(self.lib.spec_profile_stream_read(events, *self.args), "spec_profile_stream_read")


class _Plan:
    """A call with every argument marshalled once (for tight loops).  __call__
    enqueues it; profiled(events) enqueues the *_profiled form with a pointer
    from HipEvents.pair()."""

    name = ""

    def __call__(self):
        st = self.fn(*self.args)
        if st != SV_OK:
            raise SpecVerifyError(st, self.name)
        return self.out

    def profiled(self, events):
        st = self.fn_profiled(events, *self.args)
        if st != SV_OK:
            raise SpecVerifyError(st, self.name + "_profiled")
        return self.out


class SamplePlan(_Plan):
    """spec_verify_sample with every argument marshalled once (for tight loops).

    Holds references to the tensors it was built from; __call__ enqueues one
    verify on `stream` (default: the current stream at construction).
    """

    def __init__(self, target_logits, draft_logits, draft_ids, cu_draft=None, temperature=1.0, top_k=0, seed=0,
                 offset=0, max_draft=None, out=None, workspace=None, stream=None, probs=True, argmax=False,
                 top_p=1.0):
        self.lib = load_library()
        batch, kmax, total = _batch_geometry(target_logits, draft_ids, cu_draft, max_draft)
        self.shape = make_shape(target_logits, draft_logits, batch, kmax, total, cu_draft, total + batch, total)
        dev = target_logits.device
        need = C.c_size_t(0)
        _check(self.lib.spec_verify_sample(C.byref(self.shape), None, None, None, float(temperature), int(top_k),
                                           float(top_p), int(seed), int(offset), None, None, None, None, None,
                                           C.byref(need), None), "workspace query")
        self.workspace = workspace if workspace is not None and workspace.numel() >= need.value else \
            torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
        self.out = out or dict(tokens=torch.empty(total + batch, dtype=torch.int32, device=dev),
                               num_accepted=torch.empty(batch, dtype=torch.int32, device=dev),
                               probs=torch.empty((max(total, 1), 2), dtype=torch.float32, device=dev),
                               residual_mass=torch.empty(batch, dtype=torch.float32, device=dev))
        self.have = C.c_size_t(self.workspace.numel())
        self._keep = (target_logits, draft_logits, draft_ids, cu_draft)
        self.args = (C.byref(self.shape), C.c_void_p(target_logits.data_ptr()),
                     C.c_void_p(draft_logits.data_ptr() if draft_logits.numel() else None),
                     C.c_void_p(draft_ids.data_ptr() if draft_ids.numel() else None), C.c_float(temperature),
                     C.c_int32(top_k), C.c_float(top_p), C.c_uint64(seed), C.c_uint32(offset),
                     C.c_void_p(self.out["tokens"].data_ptr()), C.c_void_p(self.out["num_accepted"].data_ptr()),
                     C.c_void_p(self.out["probs"].data_ptr() if (probs and total > 0) else None),
                     C.c_void_p(self.out["residual_mass"].data_ptr() if probs else None),
                     C.c_void_p(self.workspace.data_ptr()), C.byref(self.have),
                     C.c_void_p(_stream_handle(stream)))
        self.name = "spec_verify_argmax" if argmax else "spec_verify_sample"
        self.fn = getattr(self.lib, self.name)
        self.fn_profiled = getattr(self.lib, self.name + "_profiled")



class GreedyPlan(_Plan):
    """spec_verify_greedy with every argument marshalled once."""

    def __init__(self, target_logits, draft_ids, cu_draft=None, max_draft=None, out=None, workspace=None,
                 stream=None):
        self.lib = load_library()
        batch, kmax, total = _batch_geometry(target_logits, draft_ids, cu_draft, max_draft)
        self.shape = make_shape(target_logits, None, batch, kmax, total, cu_draft, total + batch)
        dev = target_logits.device
        need = C.c_size_t(0)
        _check(self.lib.spec_verify_greedy(C.byref(self.shape), None, None, None, None, None, C.byref(need), None),
               "workspace query")
        self.workspace = workspace if workspace is not None and workspace.numel() >= need.value else \
            torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
        self.out = out or dict(tokens=torch.empty(total + batch, dtype=torch.int32, device=dev),
                               num_accepted=torch.empty(batch, dtype=torch.int32, device=dev))
        self.have = C.c_size_t(self.workspace.numel())
        self._keep = (target_logits, draft_ids, cu_draft)
        self.args = (C.byref(self.shape), C.c_void_p(target_logits.data_ptr()),
                     C.c_void_p(draft_ids.data_ptr() if draft_ids.numel() else None),
                     C.c_void_p(self.out["tokens"].data_ptr()), C.c_void_p(self.out["num_accepted"].data_ptr()),
                     C.c_void_p(self.workspace.data_ptr()), C.byref(self.have), C.c_void_p(_stream_handle(stream)))
        self.name = "spec_verify_greedy"
        self.fn = getattr(self.lib, self.name)
        self.fn_profiled = getattr(self.lib, self.name + "_profiled")



class LikelihoodPlan(_Plan):
    """spec_token_likelihood with every argument marshalled once."""

    def __init__(self, target_logits, draft_logits, tokens, cu_draft=None, batch=None, temperature=1.0, top_k=0,
                 max_draft=None, terms=True, beta=True, nll=True, workspace=None, stream=None, top_p=1.0):
        self.lib = load_library()
        b, kmax, total = _draft_geometry(draft_logits, cu_draft, batch, max_draft)
        self.shape = make_shape(target_logits, draft_logits, b, kmax, total, cu_draft, total, total)
        dev = target_logits.device
        need = C.c_size_t(0)
        _check(self.lib.spec_token_likelihood(C.byref(self.shape), None, None, None, float(temperature), int(top_k),
                                              float(top_p), None, None, None, None, C.byref(need), None),
               "workspace query")
        self.workspace = workspace if workspace is not None and workspace.numel() >= need.value else \
            torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
        self.out = _likelihood_outputs(total, b, dev, terms, beta, nll)
        self.have = C.c_size_t(self.workspace.numel())
        self._keep = (target_logits, draft_logits, tokens, cu_draft)
        self.args = (C.byref(self.shape), C.c_void_p(target_logits.data_ptr()), C.c_void_p(draft_logits.data_ptr()),
                     C.c_void_p(tokens.data_ptr()), C.c_float(temperature), C.c_int32(top_k), C.c_float(top_p),
                     C.c_void_p(_ptr_or_none(self.out, "terms")), C.c_void_p(_ptr_or_none(self.out, "beta")),
                     C.c_void_p(_ptr_or_none(self.out, "nll")), C.c_void_p(self.workspace.data_ptr()),
                     C.byref(self.have), C.c_void_p(_stream_handle(stream)))
        self.name = "spec_token_likelihood"
        self.fn = getattr(self.lib, self.name)
        self.fn_profiled = getattr(self.lib, self.name + "_profiled")



class DraftPlan(_Plan):
    """spec_draft_sample with every argument marshalled once."""

    def __init__(self, draft_logits, cu_draft=None, batch=None, temperature=1.0, top_k=0, seed=0, offset=0,
                 max_draft=None, out=None, workspace=None, stream=None, top_p=1.0):
        self.lib = load_library()
        b, kmax, total = _draft_geometry(draft_logits, cu_draft, batch, max_draft)
        self.shape = make_shape(draft_logits, draft_logits, b, kmax, total, cu_draft, total)
        dev = draft_logits.device
        need = C.c_size_t(0)
        _check(self.lib.spec_draft_sample(C.byref(self.shape), None, float(temperature), int(top_k), float(top_p),
                                          int(seed), int(offset), None, None, C.byref(need), None), "workspace query")
        self.workspace = workspace if workspace is not None and workspace.numel() >= need.value else \
            torch.empty(max(need.value, 1), dtype=torch.uint8, device=dev)
        self.out = out if out is not None else torch.empty(max(total, 1), dtype=torch.int32, device=dev)
        self.have = C.c_size_t(self.workspace.numel())
        self._keep = (draft_logits, cu_draft)
        self.args = (C.byref(self.shape), C.c_void_p(draft_logits.data_ptr()), C.c_float(temperature),
                     C.c_int32(top_k), C.c_float(top_p), C.c_uint64(seed), C.c_uint32(offset),
                     C.c_void_p(self.out.data_ptr()),
                     C.c_void_p(self.workspace.data_ptr()), C.byref(self.have), C.c_void_p(_stream_handle(stream)))
        self.name = "spec_draft_sample"
        self.fn = getattr(self.lib, self.name)
        self.fn_profiled = getattr(self.lib, self.name + "_profiled")

