"""GPU parity with IEEE binary16 logits (SV_DTYPE_F16), the precision the
pages' models ran in ("CS3602_FINAL_SpeDec", problem analysis, item 1).

Every call widens fp16 exactly to fp32 and forms no probability in 16 bits,
so the policy is the bf16 one: counts and ids bit-exact outside boundary
draws, p(x), q(x) and the residual mass within 2e-3 relative, greedy
bit-exact.  The fp16-specific parts are the decode, the out-of-row fill
patterns of the streaming passes and the 16-bit select keys.
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import (compare_argmax, compare_draft, compare_greedy, compare_sample, gpu_argmax, gpu_draft,
                      gpu_greedy, gpu_sample, note)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_07_amd as sv

    sv.load_library()


def _oracle(w, mode="sample"):
    return oracle.verify_workload(w, mode, threads=16)


def _f16_config(n):
    spec = dict(W.WORKLOADS[n])
    spec["dtype"] = "f16"
    spec["name"] = spec["name"].replace("bf16", "f16")
    return W.make_workload(spec, gen_seed=n)


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_f16_workload_sample(cfg):
    w = _f16_config(cfg)
    note(f"f16 workload {cfg} {w.name}: rows_t={w.rows_target} V={w.vocab} top_k={w.top_k}")
    rep = compare_sample(w, gpu_sample(w), _oracle(w))
    note(f"f16 workload {cfg}: {rep}")


def test_f16_workload_greedy():
    w = _f16_config(4)
    note(f"f16 greedy {w.name}")
    compare_greedy(w, gpu_greedy(w), _oracle(w, "greedy"))


@pytest.mark.parametrize("cfg", [3, 5])
def test_f16_workload_argmax_and_draft(cfg):
    w = _f16_config(cfg)
    note(f"f16 argmax {w.name}")
    rep = compare_argmax(w, gpu_argmax(w), _oracle(w, "argmax"))
    note(f"f16 argmax {cfg}: {rep}")
    note(f"f16 draft {w.name}")
    rows, nb = compare_draft(gpu_draft(w), _oracle(w, "draft"))
    note(f"f16 draft {cfg}: {rows} rows, {nb} boundary draws")


def _spec(**kw):
    d = dict(name="f16_edge", batch=4, k=3, vocab=1001, dtype="f16", temperature=1.0, top_k=0, kind="iid",
             target_sigma=2.0, draft_sigma=1.0, ragged=False, modes=("sample",))
    d.update(kw)
    return d


def _with_rows(w, f):
    tf, df = f(w.target_f32().copy()), f(w.draft_f32().copy())
    return dataclasses.replace(w, target=W.f32_to_f16_bits(tf), draft=W.f32_to_f16_bits(df))


def _scaled(s):
    return lambda x: x * np.float32(s)


# name: (spec, row transform or None, extra make_workload kwargs)
EDGE = {
    "vocab1": (_spec(vocab=1, batch=3), None, {}),
    "vocab7": (_spec(vocab=7, batch=5, k=2), None, {}),
    "vocab1001_misaligned_rows": (_spec(), None, {}),
    "ragged_with_zero_lengths": (_spec(batch=6, k=8, vocab=5000), None, dict(draft_lens=[0, 3, 0, 1, 8, 2])),
    "top_k_1": (_spec(top_k=1, vocab=4000, batch=6), None, {}),
    "top_k_160_one_key_limit": (_spec(top_k=160, vocab=20000), None, {}),
    "top_k_240_two_keys": (_spec(top_k=240, vocab=20000), None, {}),
    "top_k_256_two_keys": (_spec(top_k=256, vocab=20000), None, {}),
    "top_k_300_two_keys": (_spec(top_k=300, vocab=20000), None, {}),
    "top_k_600_exact_path": (_spec(top_k=600, vocab=20000), None, {}),
    "zipf_top50_ragged": (_spec(kind="zipf", top_k=50, vocab=60000, batch=12, k=8, ragged=True, temperature=0.7),
                          None, {}),
    "ties_top50": (_spec(vocab=9000, batch=8, k=4, top_k=50), lambda x: np.round(x * 2) / 2, {}),
    "ties_full_rows": (_spec(vocab=9000, batch=8, k=4), lambda x: np.round(x * 2) / 2, {}),
    # logits of tens of thousands (binary16 ends at 65504), softened by T
    "wide_range_T2000": (_spec(vocab=7000, batch=6, temperature=2000.0), _scaled(4000.0), {}),
    "wide_range_top50": (_spec(vocab=7000, batch=6, temperature=2000.0, top_k=50), _scaled(4000.0), {}),
    # logits in binary16's subnormal range (below 2^-14), sharpened by T
    "subnormal_logits": (_spec(vocab=3000, batch=6, temperature=2e-6), _scaled(2e-6), {}),
    "subnormal_top20": (_spec(vocab=3000, batch=6, temperature=2e-6, top_k=20), _scaled(2e-6), {}),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_f16_edge_shapes(name):
    spec, f, kw = EDGE[name]
    w = W.make_workload(spec, gen_seed=zlib.crc32(name.encode()) % 1000, **kw)
    if f is not None:
        w = _with_rows(w, f)  # the guesses stay those drawn before the transform: still valid ids
    note(f"f16 edge {name}: B={w.batch} K={w.draft_lens.tolist()} V={w.vocab} T={w.temperature} top_k={w.top_k}")
    rep = compare_sample(w, gpu_sample(w), _oracle(w))
    note(f"f16 edge {name}: {rep}")
    compare_greedy(w, gpu_greedy(w), _oracle(w, "greedy"))
    compare_argmax(w, gpu_argmax(w), _oracle(w, "argmax"))
    compare_draft(gpu_draft(w), _oracle(w, "draft"))


@pytest.mark.parametrize("top_k", [0, 50])
def test_f16_negative_infinity_masks(top_k):
    w = W.make_workload(_spec(vocab=6000, batch=8, k=4, top_k=top_k), gen_seed=11)

    def mask(x):
        x[:, 3000:] = -np.inf
        x[:, ::7] = -np.inf
        return x

    w = _with_rows(w, mask)
    note(f"f16 -inf masks top_k={top_k}")
    rep = compare_sample(w, gpu_sample(w), _oracle(w))
    note(f"f16 -inf: {rep}")
    compare_greedy(w, gpu_greedy(w), _oracle(w, "greedy"))
    compare_draft(gpu_draft(w), _oracle(w, "draft"))
