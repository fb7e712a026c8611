"""spec_verify_argmax (probabilistic acceptance, argmax of the residual or of
the last target position) on the GPU against the oracle's argmax variant."""
import zlib

import pytest

import oracle
import workloads as W
from gpu_util import compare_argmax, gpu_argmax, note

pytestmark = pytest.mark.gpu


def _oracle(w):
    return oracle.verify_workload(w, "argmax", threads=16)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_argmax_full_size(cfg):
    w = W.make_config(cfg)
    note(f"argmax config {cfg} {w.name}")
    rep = compare_argmax(w, gpu_argmax(w), _oracle(w))
    note(f"argmax config {cfg}: {rep}")


def _spec(**kw):
    d = dict(name="argmax_edge", batch=6, k=3, vocab=1001, dtype="bf16", temperature=1.0, top_k=0, kind="iid",
             target_sigma=2.0, draft_sigma=1.0, ragged=False, modes=("sample",))
    d.update(kw)
    return d


EDGE = {
    "vocab1": _spec(vocab=1),
    "vocab7_f32": _spec(vocab=7, dtype="f32"),
    "misaligned_rows": _spec(),
    "top_k_1": _spec(top_k=1, vocab=4000),
    "top_k_300_two_keys": _spec(top_k=300, vocab=20000, batch=4),
    "top_k_600_exact_path": _spec(top_k=600, vocab=20000, batch=4),
    "zipf_top50_ragged": _spec(kind="zipf", top_k=50, vocab=60000, batch=12, k=8, ragged=True, temperature=0.7),
    "peaks_f32_wide": _spec(kind="peaks", target_sigma=3.0, draft_sigma=1.5, vocab=70001, dtype="f32", batch=3),
    "draft_close_to_target": _spec(draft_sigma=0.05, vocab=5000, batch=16, k=4),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_argmax_edge_shapes(name):
    w = W.make_workload(EDGE[name], gen_seed=zlib.crc32(name.encode()) % 1000)
    note(f"argmax edge {name}")
    rep = compare_argmax(w, gpu_argmax(w), _oracle(w))
    note(f"argmax edge {name}: {rep}")
