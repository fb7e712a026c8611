"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Policy (the stated bar): accepted counts and token ids bit-exact, except
sequences where a draw the oracle evaluated lies within 1e-6 of its
threshold or CDF edge (counted and reported; their output must still be
well formed and, for a final-draw boundary, lie in the oracle's eps-window);
p(x), q(x) and the residual mass within 1e-5 relative (fp32 inputs) or
2e-3 (bf16 inputs); greedy bit-exact.
"""
import dataclasses
import zlib

import numpy as np
import pytest
import torch
from scipy import special, stats

import oracle
import workloads as W
from gpu_util import compare_greedy, compare_sample, gpu_greedy, gpu_sample, note, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rejection_sampling_verify_07_amd as sv

    sv.load_library()


def _oracle(w, mode="sample"):
    return oracle.verify_workload(w, mode, threads=16)


# --------------------------------------------------------------------------
# the five workloads at their full sizes
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_config_sample_full_size(cfg):
    w = W.make_config(cfg)
    note(f"config {cfg} {w.name}: B={w.batch} rows_t={w.rows_target} "
         f"V={w.vocab} {w.dtype} T={w.temperature} top_k={w.top_k}")
    g = gpu_sample(w)
    o = _oracle(w)
    rep = compare_sample(w, g, o)
    note(f"config {cfg}: {rep}")


@pytest.mark.parametrize("cfg", [1, 4])
def test_config_greedy_full_size(cfg):
    w = W.make_config(cfg)
    note(f"greedy config {cfg}")
    g = gpu_greedy(w)
    compare_greedy(w, g, _oracle(w, "greedy"))
    # plant argmaxes so sequences run long and some accept everything
    tf = w.target_f32()
    ids = w.draft_ids.copy()
    for b in range(w.batch):
        K = w.draft_lens[b]
        for k in range(K):
            if b % 3 != 2 or k < K // 2:
                ids[w.cu_draft[b] + k] = int(np.argmax(tf[w.cu_draft[b] + b + k]))
    w2 = dataclasses.replace(w, draft_ids=ids)
    g2 = gpu_greedy(w2)
    o2 = _oracle(w2, "greedy")
    compare_greedy(w2, g2, o2)
    assert np.any(o2["num_accepted"] == w.draft_lens)


# --------------------------------------------------------------------------
# edge shapes and degenerate cases
# --------------------------------------------------------------------------
def _spec(**kw):
    d = dict(name="edge", batch=4, k=3, vocab=1001, dtype="bf16", temperature=1.0, top_k=0, kind="iid",
             target_sigma=2.0, draft_sigma=1.0, ragged=False, modes=("sample",))
    d.update(kw)
    return d


EDGE = {
    "vocab1": (_spec(vocab=1, batch=3), {}),
    "vocab7_f32": (_spec(vocab=7, dtype="f32", batch=5, k=2), {}),
    "vocab1001_bf16_misaligned_rows": (_spec(), {}),
    "vocab1001_f32": (_spec(dtype="f32"), {}),
    "ragged_with_zero_lengths": (_spec(batch=6, k=8, vocab=5000), dict(draft_lens=[0, 3, 0, 1, 8, 2])),
    "batch1_k1": (_spec(batch=1, k=1, vocab=3000), {}),
    "top_k_1": (_spec(top_k=1, vocab=4000, batch=6), {}),
    "top_k_v_minus_1": (_spec(top_k=1000, batch=3), {}),
    "top_k_v": (_spec(top_k=1001, batch=3), {}),
    "top_k_160_one_key_limit": (_spec(top_k=160, vocab=20000, batch=4), {}),
    "top_k_161_two_keys": (_spec(top_k=161, vocab=20000, batch=4), {}),
    "top_k_240_two_keys": (_spec(top_k=240, vocab=20000, batch=4), {}),
    "top_k_256_two_keys": (_spec(top_k=256, vocab=20000, batch=4), {}),
    "top_k_300_two_keys": (_spec(top_k=300, vocab=20000, batch=4), {}),
    "top_k_400_two_keys_limit": (_spec(top_k=400, vocab=20000, batch=4), {}),
    "top_k_600_exact_path": (_spec(top_k=600, vocab=20000, batch=4), {}),
    "temperature_0.05": (_spec(temperature=0.05, vocab=8000, batch=8), {}),
    "temperature_5": (_spec(temperature=5.0, vocab=8000, batch=8), {}),
    "k128": (_spec(k=128, batch=2, vocab=300, dtype="f32"), {}),
    "zipf_top50_ragged": (_spec(kind="zipf", top_k=50, vocab=60000, batch=12, k=8, ragged=True,
                                temperature=0.7), {}),
    "peaks_f32_wide": (_spec(kind="peaks", target_sigma=3.0, draft_sigma=1.5, vocab=70001, dtype="f32", batch=3,
                             k=4), {}),
}


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_shapes(name):
    spec, kw = EDGE[name]
    w = W.make_workload(spec, gen_seed=zlib.crc32(name.encode()) % 1000, **kw)
    note(f"edge {name}: B={w.batch} K={w.draft_lens.tolist()} V={w.vocab} {w.dtype} top_k={w.top_k}")
    g = gpu_sample(w)
    rep = compare_sample(w, g, _oracle(w))
    note(f"edge {name}: {rep}")
    gg = gpu_greedy(w)
    compare_greedy(w, gg, _oracle(w, "greedy"))


def _with_rows(w, f):
    """A copy of w with target/draft float rows transformed by f (then re-encoded)."""
    tf, df = f(w.target_f32().copy()), f(w.draft_f32().copy())
    enc = {"f32": lambda x: x.astype(np.float32), "bf16": W.f32_to_bf16_bits, "f16": W.f32_to_f16_bits}[w.dtype]
    return dataclasses.replace(w, target=enc(tf), draft=enc(df))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("top_k", [0, 50])
def test_ties(dtype, top_k):
    w = W.make_workload(_spec(dtype=dtype, vocab=9000, batch=8, k=4, top_k=top_k), gen_seed=5)
    w = _with_rows(w, lambda x: np.round(x * 2) / 2)  # many equal logits, ties at tau and at the max
    note(f"ties {dtype} top_k={top_k}")
    rep = compare_sample(w, gpu_sample(w), _oracle(w))
    note(f"ties: {rep}")
    compare_greedy(w, gpu_greedy(w), _oracle(w, "greedy"))


@pytest.mark.parametrize("top_k", [0, 50])
def test_negative_infinity_masks(top_k):
    w = W.make_workload(_spec(vocab=6000, batch=8, k=4, top_k=top_k), gen_seed=11)

    def mask(x):
        x[:, 3000:] = -np.inf
        x[:, ::7] = -np.inf
        return x

    w = _with_rows(w, mask)
    note(f"-inf masks top_k={top_k}")
    rep = compare_sample(w, gpu_sample(w), _oracle(w))
    note(f"-inf: {rep}")
    compare_greedy(w, gpu_greedy(w), _oracle(w, "greedy"))


def test_constant_rows_take_the_full_row_path():
    # every logit ties, so the top-50 kept set is the whole row (larger than a kept list)
    w = W.make_workload(_spec(vocab=5000, batch=4, k=3, top_k=50, kind="flat"), gen_seed=2)
    note("constant rows, top_k=50")
    rep = compare_sample(w, gpu_sample(w), _oracle(w))
    note(f"constant rows: {rep}")


def test_tied_head_takes_the_chunk_list_select():
    # 200 logits tied at the row maximum, one at the start of each of the first
    # 200 16-byte blocks (rows are 16-byte aligned here): 200 lanes of the first
    # tile reach the maximum, so the tile's bound is that maximum and its 200
    # ties are its candidates -- more than the speculative select loads per
    # chunk (128), fewer than a chunk holds (256).  The kept set is the 200
    # ties, more than one per lane of a wave.
    w = W.make_workload(_spec(vocab=20000, batch=3, k=3, top_k=50, kind="zipf"), gen_seed=21)

    def tie_head(x):
        x = np.minimum(x, 8.0)
        x[:, 0:1600:8] = 9.0
        return x

    w = _with_rows(w, tie_head)
    note("tied head: 200 ties at the max in the first chunk, top_k=50")
    g = gpu_sample(w)
    rep = compare_sample(w, g, _oracle(w))
    note(f"tied head: {rep}")
    compare_greedy(w, gpu_greedy(w), _oracle(w, "greedy"))


def test_many_chunks_bypass_the_speculative_select():
    # V = 300000 bf16 is 19 chunks per row, more than the speculative select covers
    w = W.make_workload(_spec(vocab=300000, batch=2, k=2, top_k=50, kind="zipf", temperature=0.7), gen_seed=22)
    note("V=300000 bf16 top_k=50 (19 chunks per row)")
    rep = compare_sample(w, gpu_sample(w), _oracle(w))
    note(f"many chunks: {rep}")


def test_candidate_overflow_takes_the_exact_path():
    # heavy ties inside one chunk overflow its candidate slots
    w = W.make_workload(_spec(vocab=30000, batch=3, k=3, top_k=50, kind="zipf"), gen_seed=3)

    def flat_head(x):
        x[:, :2000] = np.round(x[:, :2000])
        x[:, :600] = 4.0
        return x

    w = _with_rows(w, flat_head)
    note("candidate overflow")
    rep = compare_sample(w, gpu_sample(w), _oracle(w))
    note(f"overflow: {rep}")


def test_draft_equals_target_accepts_all():
    w = W.make_workload(_spec(vocab=3000, batch=16, k=5), gen_seed=4)
    tgt_rows = np.concatenate([w.target[w.cu_draft[b] + b: w.cu_draft[b] + b + 5] for b in range(w.batch)])
    w = dataclasses.replace(w, draft=tgt_rows)
    g = gpu_sample(w)
    assert np.all(g["num_accepted"] == 5)
    compare_sample(w, g, _oracle(w))


@pytest.mark.parametrize("top_k", [0, 50])
def test_accept_ratio_near_the_uniform(top_k):
    """Guesses whose p/q lies just above or below its accept uniform.

    The kernel decides the accept test in fp32 unless u lies within 2^-12
    (relative) of the fp32 ratio, and in fp64 there; these guesses put the
    ratio at u * (1 + rel) for rel from -3e-3 to 3e-3, on both sides of that
    margin.  Each sequence has one guess.  In the sequences whose u lies in
    [0.2, 0.95] the draft row is random with the guess on top, and the target
    row equals it except at the guess, whose logit is solved (by bisection on
    the oracle's own probabilities) so that the ratio lands on its mark; the
    other sequences keep their random rows.  Every placed decision must be
    the one its offset fixes (accept above u, reject below), on the GPU and
    in the oracle."""
    rels = [-3e-3, -4e-4, -2e-4, -5e-5, -1e-5, 1e-5, 5e-5, 2e-4, 4e-4, 3e-3]
    B, V, T = 96, 3000, 0.5
    w = W.make_workload(_spec(vocab=V, batch=B, k=1, dtype="f32", temperature=T, top_k=top_k), gen_seed=21)
    rng = np.random.default_rng(5)
    target, draft, ids = w.target.copy(), w.draft.copy(), w.draft_ids.copy()
    want = {}
    for b in range(B):
        u = oracle.uniform(w.seed, b, 0, 0, w.offset)
        if not 0.2 <= u <= 0.95:
            continue
        mark = u * (1.0 + rels[len(want) % len(rels)])
        want[b] = int(u < mark)
        d = rng.normal(0.0, 1.0, V).astype(np.float32)
        x = int(rng.integers(V))
        d[x] = np.float32(d.max() + 1.0)  # the guess tops the draft row (kept by any top-k)
        q = oracle.row_probs(d, "f32", T, top_k)[0][x]

        def ratio(delta):
            t = d.copy()
            t[x] = np.float32(d[x] + delta)
            return oracle.row_probs(t, "f32", T, top_k)[0][x] / q, t

        lo, hi = -2.0, 1.0
        assert ratio(lo)[0] < mark < ratio(hi)[0]
        for _ in range(60):
            mid = 0.5 * (lo + hi)
            if ratio(mid)[0] < mark:
                lo = mid
            else:
                hi = mid
        (rl, tl), (rh, th) = ratio(lo), ratio(hi)
        r, t = (rl, tl) if abs(rl - mark) < abs(rh - mark) else (rh, th)
        assert abs(r / mark - 1.0) < 2e-6
        target[int(w.cu_draft[b]) + b] = t
        draft[int(w.cu_draft[b])] = d
        ids[int(w.cu_draft[b])] = x
    assert len(want) >= 3 * len(rels)
    w = dataclasses.replace(w, target=target, draft=draft, draft_ids=ids)
    o = _oracle(w)
    g = gpu_sample(w)
    for b, a in want.items():
        assert int(o["num_accepted"][b]) == a, f"oracle, sequence {b}"
        assert int(g["num_accepted"][b]) == a, f"GPU, sequence {b}"
    rep = compare_sample(w, g, o)
    note(f"accept near the uniform (top_k {top_k}, {len(want)} placed): {rep}")


def test_guess_outside_both_supports_is_rejected():
    """A guess whose target logit is -inf in a row with fewer finite logits
    than top_k (so tau = -inf keeps it, with p = 0) and which the draft's
    top-k drops (q = 0): the ratio is 0 and the guess must be rejected.  The
    accept test's fp32 shortcut must not read "kept by the filter" as p > 0."""
    V, K, B = 64, 2, 8
    w = W.make_workload(_spec(vocab=V, batch=B, k=K, dtype="f32", temperature=1.0, top_k=50), gen_seed=31)
    rng = np.random.default_rng(9)
    target, draft, ids = w.target.copy(), w.draft.copy(), w.draft_ids.copy()
    for b in range(B):
        t0, d0 = int(w.cu_draft[b]) + b, int(w.cu_draft[b])
        for k in range(K):
            row_t = np.full(V, -np.inf, np.float32)
            live = rng.choice(V, size=10, replace=False)
            row_t[live] = rng.normal(0.0, 1.0, 10).astype(np.float32)  # 10 finite: tau = -inf
            row_d = rng.normal(0.0, 1.0, V).astype(np.float32)
            dead = [v for v in range(V) if v not in set(live.tolist())]
            x = int(dead[b % len(dead)])
            row_d[x] = np.float32(row_d.min() - 5.0)  # outside the draft's top 50: q(x) = 0
            target[t0 + k], draft[d0 + k], ids[d0 + k] = row_t, row_d, x
        target[t0 + K] = rng.normal(0.0, 1.0, V).astype(np.float32)
    w = dataclasses.replace(w, target=target, draft=draft, draft_ids=ids)
    o = _oracle(w)
    g = gpu_sample(w)
    assert np.all(o["num_accepted"] == 0)
    assert np.all(g["num_accepted"] == 0)
    compare_sample(w, g, o)


def test_strided_and_offset_rows():
    """Rows with a padded stride and a start offset (not 16-byte aligned)."""
    w = W.make_workload(_spec(vocab=2000, batch=5, k=3, dtype="bf16", top_k=40), gen_seed=8)
    dev = "cuda:0"
    pad, off = 5, 1

    def place(a):
        buf = np.zeros((a.shape[0], a.shape[1] + pad), dtype=np.uint16)
        buf[:, off:off + a.shape[1]] = a
        t = torch.from_numpy(buf.view(np.int16)).to(dev).view(torch.bfloat16)
        return t[:, off:off + a.shape[1]]

    tgt, drf = place(w.target), place(w.draft)
    assert tgt.stride(0) == 2000 + pad
    ids = torch.from_numpy(w.draft_ids).to(dev)
    g = gpu_sample(w, tensors=(tgt, drf, ids, None))
    rep = compare_sample(w, g, _oracle(w))
    note(f"strided: {rep}")
    gg = gpu_greedy(w, tensors=(tgt, drf, ids, None))
    compare_greedy(w, gg, _oracle(w, "greedy"))


def test_out_of_range_ids_and_bad_offsets_are_reported():
    w = W.make_workload(_spec(vocab=1000, batch=4, k=3, ragged=True), gen_seed=6,
                        draft_lens=[3, 3, 3, 3])
    ids = w.draft_ids.copy()
    ids[4] = 1000  # sequence 1
    ids[9] = -3  # sequence 3
    w2 = dataclasses.replace(w, draft_ids=ids)
    g = gpu_sample(w2)
    assert g["num_accepted"][1] == -1 and g["num_accepted"][3] == -1
    o = _oracle(w)
    compare_sample(w2, g, o, seqs=[0, 2])
    gg = gpu_greedy(w2)
    # sequence 1's bad id sits at position 1, past a possible first mismatch:
    # every id is checked, as in the sampling verify
    assert gg["num_accepted"][1] == -1 and gg["num_accepted"][3] == -1
    og = oracle.verify_greedy(w2.target, w2.draft_ids, w2.cu_draft, w2.vocab, w2.dtype)
    assert og["num_accepted"][1] == -1 and og["num_accepted"][3] == -1
    for b in (0, 2):
        assert gg["num_accepted"][b] == og["num_accepted"][b]
    # a prefix array that points past the draft rows
    tgt, drf, idt, cu = to_device(w)
    cu_bad = cu.clone()
    cu_bad[4] = 13  # total is 12
    import rejection_sampling_verify_07_amd as sv

    out = sv.verify_sample(tgt, drf, idt, cu_draft=cu_bad, max_draft=3, temperature=1.0)
    torch.cuda.synchronize()
    assert out["num_accepted"].cpu().numpy()[3] == -1


# --------------------------------------------------------------------------
# determinism and distribution
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg", [3, 5])
def test_bitwise_determinism(cfg):
    w = W.make_config(cfg)
    t = to_device(w)
    a = gpu_sample(w, tensors=t)
    for _ in range(3):
        b = gpu_sample(w, tensors=t)
        for k in a:
            assert np.array_equal(a[k], b[k], equal_nan=True), k


def test_seed_and_offset_change_the_draws():
    w = W.make_config(3)
    t = to_device(w)
    a = gpu_sample(w, tensors=t)
    b = gpu_sample(dataclasses.replace(w, offset=1), tensors=t)
    assert not np.array_equal(a["tokens"], b["tokens"])
    o = _oracle(dataclasses.replace(w, offset=1))
    compare_sample(w, b, o)


def test_chi_square_on_gpu_million_sequences():
    """10^6 sequences in one call, x ~ q per sequence: first token ~ p_0."""
    rng = np.random.default_rng(77)
    V, T, B = 8, 0.9, 10**6
    lt = (rng.standard_normal((2, V)) * 1.5).astype(np.float32)
    ld = (lt[:1] + rng.standard_normal((1, V))).astype(np.float32)
    p = special.softmax(lt[0].astype(np.float64) / T)
    q = special.softmax(ld[0].astype(np.float64) / T)
    x = rng.choice(V, B, p=q).astype(np.int32)
    dev = "cuda:0"
    tgt = torch.from_numpy(lt).to(dev).repeat(B, 1)
    drf = torch.from_numpy(ld).to(dev).repeat(B, 1)
    ids = torch.from_numpy(x).to(dev)
    import rejection_sampling_verify_07_amd as sv

    out = sv.verify_sample(tgt, drf, ids, temperature=T, seed=123, offset=0)
    torch.cuda.synchronize()
    first = out["tokens"].view(B, 2)[:, 0].cpu().numpy()
    obs = np.bincount(first, minlength=V)
    pv = stats.chisquare(obs, p * B).pvalue
    note(f"chi-square p-value {pv:.3g}")
    assert pv > 1e-3
