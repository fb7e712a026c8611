"""Seeded synthetic inputs for the speculative-sampling verify step.

This module only draws inputs: target and draft logit rows, per-sequence
draft lengths and draft token ids.  It holds none of the verify arithmetic
(no softmax, no acceptance test, no residual, no inverse CDF), and it imports
neither the GPU binding nor the oracle, so both sides can be fed from it.

The draft ids must be distributed as the draft distribution q that the
verifier itself forms (the exactness argument of the speculative-sampling
proof on "CS3602_FINAL_SpeDec", section 2, assumes the guess is drawn from
q).  They are drawn with the Gumbel-max trick: x = argmax_v (l_v / T + G_v)
over the draft row's top-k kept set (all ids whose logit is >= the k-th
largest when top-k is on), with G_v i.i.d. standard Gumbel.  This is a
different route from anything the verifier computes.

The five named workloads imitate language-model logits of the sizes the
pages use (Pythia's 50304-token vocabulary, gamma = K = 4 draft tokens) plus
two larger-vocabulary batches.  Every sequence is drawn from its own child
generator (numpy SeedSequence.spawn), so the first b sequences of a batch
are identical whatever batch size is asked for.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "make_config",
    "make_workload",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "f32_to_f16_bits",
    "f16_bits_to_f32",
    "decode_f32",
]


# --------------------------------------------------------------------------
# bf16 encoding (round-to-nearest-even on the top 16 bits of an IEEE fp32)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint32)
    b = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


# IEEE binary16: numpy's own conversion (round to nearest, ties to even)
def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16; return the bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of binary16 bits to float32."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def decode_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Stored logits (float32 values, or 16-bit patterns) widened to float32."""
    if dtype == "f32":
        return x
    return bf16_bits_to_f32(x) if dtype == "bf16" else f16_bits_to_f32(x)


# --------------------------------------------------------------------------
# Workload container
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Workload:
    """One batch of verify inputs, host resident.

    Layout (packed, ragged): sequence b owns draft rows
    cu_draft[b] .. cu_draft[b+1]-1 and target rows cu_draft[b]+b ..
    cu_draft[b+1]+b (K_b + 1 rows, the last one is the bonus position).
    Logits are row-major [rows, vocab]; dtype "f32" holds float32 values,
    dtype "bf16" and "f16" hold the raw bfloat16 / IEEE binary16 bit patterns
    as uint16.
    """

    name: str
    batch: int
    k_max: int
    vocab: int
    dtype: str
    temperature: float
    top_k: int
    seed: int
    offset: int
    ragged: bool
    modes: tuple
    draft_lens: np.ndarray  # int32 [B]
    cu_draft: np.ndarray  # int32 [B+1]
    target: np.ndarray  # [R_t, V] float32 or uint16
    draft: np.ndarray  # [R_d, V] float32 or uint16
    draft_ids: np.ndarray  # int32 [R_d]
    info: dict = dataclasses.field(default_factory=dict)
    top_p: float = 1.0  # nucleus filter after top-k; 1 keeps everything

    @property
    def rows_target(self) -> int:
        return int(self.cu_draft[-1]) + self.batch

    @property
    def rows_draft(self) -> int:
        return int(self.cu_draft[-1])

    @property
    def elem_size(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def algorithmic_bytes(self, mode: str = "sample") -> int:
        """Bytes the method must read once: every logit of every row it uses
        (sample, argmax: target and draft rows; greedy: target rows; draft: draft rows;
        likelihood: the draft rows and as many target rows)."""
        if mode == "draft":
            rows = self.rows_draft
        elif mode == "likelihood":
            rows = 2 * self.rows_draft
        else:
            rows = self.rows_target + (self.rows_draft if mode in ("sample", "argmax") else 0)
        return rows * self.vocab * self.elem_size

    def positions(self) -> int:
        """Verified positions per call: sum over sequences of K_b + 1."""
        return self.rows_target

    def likelihood_rows(self):
        """The rows in the likelihood layout, where position (b, k), k < K_b, is
        row cu_draft[b] + k of both tensors: target rows k < K_b of every
        sequence, the draft rows, and the guesses as the scored tokens."""
        keep = [np.arange(int(self.cu_draft[b]) + b, int(self.cu_draft[b + 1]) + b) for b in range(self.batch)]
        keep = np.concatenate(keep + [np.zeros(0, np.int64)]).astype(np.int64)
        return np.ascontiguousarray(self.target[keep]), self.draft, self.draft_ids

    def target_f32(self) -> np.ndarray:
        return decode_f32(self.target, self.dtype)

    def draft_f32(self) -> np.ndarray:
        return decode_f32(self.draft, self.dtype)


# --------------------------------------------------------------------------
# The five named workloads
# --------------------------------------------------------------------------
WORKLOADS = {
    1: dict(
        name="tiny_b1_k4_v1000_f32",
        batch=1, k=4, vocab=1000, dtype="f32", temperature=1.0, top_k=0,
        kind="iid", target_sigma=2.0, draft_sigma=1.0, ragged=False,
        modes=("sample", "greedy"),
    ),
    2: dict(
        name="pythia_b1_k4_v50304_f32",
        batch=1, k=4, vocab=50304, dtype="f32", temperature=1.0, top_k=0,
        kind="peaks", target_sigma=3.0, draft_sigma=1.5, ragged=False,
        modes=("sample",),
    ),
    3: dict(
        name="batched_b64_k4_v50304_bf16",
        batch=64, k=4, vocab=50304, dtype="bf16", temperature=0.8, top_k=0,
        kind="peaks", target_sigma=3.0, draft_sigma=(0.5, 3.0), ragged=False,
        modes=("sample",),
    ),
    4: dict(
        name="deep_b256_k8_v128256_bf16",
        batch=256, k=8, vocab=128256, dtype="bf16", temperature=1.0, top_k=0,
        kind="zipf", target_sigma=2.0, draft_sigma=1.0, ragged=False,
        modes=("sample", "greedy"),
    ),
    5: dict(
        name="ragged_b32_k1to8_v151936_bf16_top50",
        batch=32, k=8, vocab=151936, dtype="bf16", temperature=0.7, top_k=50,
        kind="zipf", target_sigma=2.0, draft_sigma=1.0, ragged=True,
        modes=("sample",),
    ),
}

_PEAK_IDS = 20  # ids per row boosted in the "peaks" recipe
_PEAK_BOOST = 8.0
_ZIPF_S = 1.1


def _target_rows(rng, kind, n_rows, vocab, sigma):
    if n_rows == 0:
        return np.zeros((0, vocab), np.float32)
    noise = rng.standard_normal((n_rows, vocab), dtype=np.float32)
    if kind == "iid":
        return noise * np.float32(sigma)
    if kind == "peaks":
        rows = noise * np.float32(sigma)
        for r in range(n_rows):
            ids = rng.choice(vocab, size=min(_PEAK_IDS, vocab), replace=False)
            rows[r, ids] += np.float32(_PEAK_BOOST)
        return rows
    if kind == "zipf":
        prior = (-_ZIPF_S * np.log(np.arange(1, vocab + 1, dtype=np.float64))).astype(np.float32)
        return noise * np.float32(sigma) + prior[None, :]
    if kind == "flat":
        return np.zeros((n_rows, vocab), np.float32)
    raise ValueError(kind)


def _encode(x, dtype):
    if dtype == "f32":
        return x.astype(np.float32)
    return f32_to_bf16_bits(x) if dtype == "bf16" else f32_to_f16_bits(x)


def _decode(x, dtype):
    return decode_f32(x, dtype)


def _gumbel_draw(rng, logits_f32, temperature, top_k):
    """x ~ softmax(l / T) restricted to the top-k kept set, by Gumbel-max."""
    l = logits_f32.astype(np.float64)
    v = l.shape[0]
    keep = l > -np.inf
    if 0 < top_k < v:
        kth = np.partition(l, v - top_k)[v - top_k]
        keep &= l >= kth
    g = -np.log(-np.log(rng.random(v)))
    score = np.where(keep, l / temperature + g, -np.inf)
    return int(np.argmax(score))


def _gen_sequence(seq_rng, spec, k_b, vocab, dtype):
    """Draw one sequence's K_b+1 target rows, K_b draft rows and K_b ids."""
    kind = spec["kind"]
    sigma_d = spec["draft_sigma"]
    if isinstance(sigma_d, tuple):
        sigma_d = float(seq_rng.uniform(sigma_d[0], sigma_d[1]))
    tgt = _target_rows(seq_rng, kind, k_b + 1, vocab, spec["target_sigma"])
    if k_b > 0:
        noise = seq_rng.standard_normal((k_b, vocab), dtype=np.float32)
        drf = tgt[:k_b] + noise * np.float32(sigma_d)
    else:
        drf = np.zeros((0, vocab), np.float32)
    tgt_e = _encode(tgt, dtype)
    drf_e = _encode(drf, dtype)
    drf_dec = _decode(drf_e, dtype)
    ids = np.array(
        [_gumbel_draw(seq_rng, drf_dec[k], spec["temperature"], spec["top_k"]) for k in range(k_b)],
        dtype=np.int32,
    )
    return tgt_e, drf_e, ids, sigma_d


def make_workload(
    spec: dict,
    gen_seed: int,
    batch: Optional[int] = None,
    draft_lens: Optional[Sequence[int]] = None,
    threads: Optional[int] = None,
) -> Workload:
    """Build a workload from a spec dict (see WORKLOADS for the keys).

    batch overrides spec["batch"] (the first `batch` sequences are the same
    as in the full batch).  draft_lens, when given, fixes K_b per sequence.
    """
    spec = dict(spec)
    B = int(batch if batch is not None else spec["batch"])
    vocab = int(spec["vocab"])
    dtype = spec["dtype"]
    ss = np.random.SeedSequence(int(gen_seed))
    children = ss.spawn(B)
    seq_rngs = [np.random.Generator(np.random.PCG64(c)) for c in children]
    if draft_lens is not None:
        ks = np.asarray(draft_lens, dtype=np.int32)
        assert ks.shape == (B,)
    elif spec.get("ragged"):
        # K_b ~ U{1..k}: the first draw of each sequence's own generator
        ks = np.array([int(r.integers(1, spec["k"] + 1)) for r in seq_rngs], dtype=np.int32)
    else:
        ks = np.full(B, int(spec["k"]), dtype=np.int32)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ks)
    R_d = int(cu[-1])
    R_t = R_d + B
    store = np.float32 if dtype == "f32" else np.uint16
    target = np.empty((R_t, vocab), dtype=store)
    draft = np.empty((R_d, vocab), dtype=store)
    ids = np.empty(R_d, dtype=np.int32)
    sigmas = np.zeros(B)

    def work(b):
        tgt, drf, xb, sd = _gen_sequence(seq_rngs[b], spec, int(ks[b]), vocab, dtype)
        t0 = int(cu[b]) + b
        target[t0:t0 + ks[b] + 1] = tgt
        draft[cu[b]:cu[b + 1]] = drf
        ids[cu[b]:cu[b + 1]] = xb
        sigmas[b] = sd

    nthr = threads or min(16, os.cpu_count() or 1)
    if B == 1 or nthr == 1:
        for b in range(B):
            work(b)
    else:
        with _cf.ThreadPoolExecutor(nthr) as ex:
            list(ex.map(work, range(B)))

    return Workload(
        name=spec.get("name", "custom"),
        batch=B,
        k_max=int(max(spec["k"], ks.max() if B else 0)),
        vocab=vocab,
        dtype=dtype,
        temperature=float(spec["temperature"]),
        top_k=int(spec.get("top_k", 0)),
        seed=int(spec.get("seed", 0)),
        offset=int(spec.get("offset", 0)),
        ragged=bool(spec.get("ragged", False) or draft_lens is not None),
        modes=tuple(spec.get("modes", ("sample",))),
        draft_lens=ks,
        cu_draft=cu,
        target=target,
        draft=draft,
        draft_ids=ids,
        info=dict(draft_sigma=sigmas, gen_seed=int(gen_seed)),
        top_p=float(spec.get("top_p", 1.0)),
    )


def make_config(n: int, batch: Optional[int] = None, gen_seed: Optional[int] = None, **kw) -> Workload:
    """Workload n (1..5); the generator seed defaults to n."""
    return make_workload(WORKLOADS[n], gen_seed if gen_seed is not None else n, batch=batch, **kw)
