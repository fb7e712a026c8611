"""GPU parity of top-k calls with many rows (64 sequences of 4 guesses: 320
target and 256 draft rows, so that every call -- sampling, draft sampling,
likelihood -- spans hundreds of rows), over edge-case rows.

The policy is the one of the other top-k tests: counts and ids bit-exact
outside boundary draws, probabilities and residual mass within the dtype's
tolerance.  Rows sorted by logit put every candidate of a chunk above the
chunk's bound; long runs of ties and constant rows overflow the candidate
slots and take the exact select path; a row with fewer finite logits than
top_k has tau = -inf.
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (compare_draft, compare_likelihood, compare_sample, gpu_draft, gpu_likelihood, gpu_sample,
                      note)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_07_amd as sv

    sv.load_library()


def _spec(**kw):
    # 64 sequences of 4 guesses: 320 target and 256 draft rows
    d = dict(name="topk_rows", batch=64, k=4, vocab=5000, dtype="bf16", temperature=0.8, top_k=50, kind="iid",
             target_sigma=2.0, draft_sigma=1.0, ragged=False, modes=("sample",))
    d.update(kw)
    return d


def _encode(x, dtype):
    if dtype == "f32":
        return x.astype(np.float32)
    return W.f32_to_bf16_bits(x) if dtype == "bf16" else W.f32_to_f16_bits(x)


def _with_rows(w, f):
    """The same workload with f applied to every row (guesses unchanged: still valid ids)."""
    return dataclasses.replace(w, target=_encode(f(w.target_f32().copy()), w.dtype),
                               draft=_encode(f(w.draft_f32().copy()), w.dtype))


def _ties(x):
    return np.round(x * 2) / 2


def _constant(x):
    return np.zeros_like(x) + np.float32(0.25)


def _ascending(x):
    return np.sort(x, axis=1)


def _descending(x):
    return -np.sort(-x, axis=1)


def _masked(x):
    x[:, ::7] = -np.inf
    x[:, x.shape[1] // 2:] = -np.inf
    return x


def _wave0_peaks(vec):
    """100 peaks in the first tile of every row, one element in each of the
    blocks (load 0 or 1, thread 0..49), all other logits near -5.  The peaks
    take four levels 5 + k/32 (exact in bf16), and thread 0 has both of its
    peaks at the lowest one, which is then the tile bound: all 100 peak blocks,
    every one in wave 0, reach it, so the staged candidate compaction takes its
    second round, and the kept set has ties at tau.  vec: logits per 16-byte
    block."""

    def f(x):
        y = x * np.float32(0.2) - np.float32(5.0)
        rows = np.arange(y.shape[0])[:, None]
        tid = np.arange(50)
        for i in (0, 1):
            cols = (i * 256 + tid) * vec + (tid * 3 + i) % vec
            level = np.where(tid > 0, (rows * 7 + tid * 3 + i * 5) % 4, 0)
            y[:, cols] = np.float32(5.0) + np.float32(1.0 / 32.0) * level
        return y

    return f


def _wave0_blocks_at_bound(x, vec, top_k, loads=6):
    """Blocks of wave 0 in the first tile of row x whose maximum reaches the
    tile bound (the top_k-th largest lane maximum, cut to its top 16 key bits;
    the values here are positive)."""
    bmax = x[: 256 * loads * vec].reshape(loads, 256, vec).max(axis=2)
    b = np.float32(np.sort(bmax.max(axis=0))[::-1][top_k - 1])
    bound = (np.array([b]).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)[0]
    assert bound > 0
    return int((bmax[:, :64] >= bound).sum())


def _few_finite(x):
    # 10 finite logits per row: fewer than top_k, so tau = -inf
    y = np.full_like(x, -np.inf)
    y[:, 3:13] = x[:, 3:13]
    return y


CASES = {
    "bf16_v5000_top50": (_spec(), None),
    "bf16_v1001_misaligned": (_spec(vocab=1001), None),
    "bf16_v7": (_spec(vocab=7, top_k=3), None),
    "bf16_v1": (_spec(vocab=1, top_k=1), None),
    "f32_v5000_top50": (_spec(dtype="f32"), None),
    "f32_v1001_misaligned": (_spec(dtype="f32", vocab=1001), None),
    "f16_v5000_top50": (_spec(dtype="f16"), None),
    "bf16_top1": (_spec(top_k=1), None),
    "bf16_top240": (_spec(top_k=240, vocab=20000), None),
    "f32_top240": (_spec(top_k=240, vocab=20000, dtype="f32"), None),
    "bf16_top256": (_spec(top_k=256, vocab=20000), None),
    "bf16_top400": (_spec(top_k=400, vocab=20000), None),  # the two-key pass's limit: tiles cut to their top_k
    "bf16_top600_ties": (_spec(top_k=600, vocab=20000), _ties),  # exact path: staged bucket, ties at tau
    # top_k above the candidate pass: the exact select over full rows
    "bf16_top300_ties": (_spec(top_k=300, vocab=20000), _ties),  # staged bucket, ties at tau
    "bf16_top300_constant_rows": (_spec(top_k=300, vocab=20000), _constant),  # bucket too large for LDS
    "f32_top1000": (_spec(top_k=1000, vocab=20000, dtype="f32"), None),  # list filled by a separate walk
    "bf16_top2000": (_spec(top_k=2000, vocab=20000), None),  # more kept ids than a list holds
    "bf16_zipf_ragged": (_spec(kind="zipf", k=8, ragged=True, vocab=60000, temperature=0.7), None),
    "bf16_ties": (_spec(vocab=9000), _ties),
    "bf16_constant_rows": (_spec(vocab=3000), _constant),
    "bf16_ascending_rows": (_spec(vocab=20000), _ascending),
    "f32_ascending_rows": (_spec(vocab=20000, dtype="f32"), _ascending),
    "bf16_descending_rows": (_spec(vocab=20000), _descending),
    "bf16_neg_inf_masks": (_spec(vocab=6000), _masked),
    "f16_neg_inf_masks": (_spec(vocab=6000, dtype="f16"), _masked),
    "bf16_fewer_finite_than_top_k": (_spec(vocab=4000), _few_finite),
    "bf16_wave0_peaks_two_rounds": (_spec(vocab=20000), _wave0_peaks(8)),
    "f32_wave0_peaks_two_rounds": (_spec(vocab=20000, dtype="f32"), _wave0_peaks(4)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_topk_many_rows(name):
    spec, f = CASES[name]
    w = W.make_workload(dict(spec, name=name), gen_seed=zlib.crc32(name.encode()) % 1000)
    if f is not None:
        w = _with_rows(w, f)
    assert w.rows_draft >= 256 and w.rows_target + w.rows_draft >= 256
    if "wave0_peaks" in name:
        nb = _wave0_blocks_at_bound(w.target_f32()[0], 4 if w.dtype == "f32" else 8, w.top_k)
        assert 64 < nb <= 128, nb
    note(f"top-k rows {name}: B={w.batch} rows_t={w.rows_target} rows_d={w.rows_draft} V={w.vocab} "
         f"{w.dtype} top_k={w.top_k}")
    rep = compare_sample(w, gpu_sample(w), oracle.verify_workload(w, "sample", threads=16))
    note(f"{name} sample: {rep}")
    rows, nb = compare_draft(gpu_draft(w), oracle.verify_workload(w, "draft", threads=16))
    note(f"{name} draft: {rows} rows, {nb} boundary draws")
    rep = compare_likelihood(w, gpu_likelihood(w), oracle.verify_workload(w, "likelihood", threads=16))
    note(f"{name} likelihood: {rep}")


def test_topk_rows_full_size_workload():
    """The 151936-vocabulary top-50 workload at 64 sequences (bf16)."""
    w = W.make_workload(dict(W.WORKLOADS[5], batch=64, name="topk_rows_v151936"), gen_seed=91)
    note(f"top-k rows full size: rows_t={w.rows_target} rows_d={w.rows_draft}")
    rep = compare_sample(w, gpu_sample(w), oracle.verify_workload(w, "sample", threads=16))
    note(f"full size sample: {rep}")
    rows, nb = compare_draft(gpu_draft(w), oracle.verify_workload(w, "draft", threads=16))
    note(f"full size draft: {rows} rows, {nb} boundary draws")
