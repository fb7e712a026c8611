"""Pins of the CPU oracle against facts fixed outside it.

Each test names what it checks the oracle against:
  * library routines (torch's bf16 widening, scipy's softmax / logsumexp,
    torch.topk, numpy.argmax),
  * closed forms from the speculative-sampling proof on "CS3602_FINAL_SpeDec"
    (section 2): the residual normaliser is 1 - beta with
    beta = sum_x min(p(x), q(x)), and accept-or-resample emits x with
    probability exactly p(x),
  * exhaustive enumeration of every 24-bit uniform on tiny vocabularies,
  * chi-square tests over 10^5..10^6 seeded trials,
  * special cases with known answers.
A plausible slip in the oracle (p and q swapped, a dropped temperature, an
off-by-one row, <= instead of <, a missing normaliser) fails at least one.
"""
import numpy as np
import pytest
import torch
from scipy import special, stats

import workloads as W

GRID = 2**24


def _softmax(l, T, top_k=0):
    """Independent reference: scipy softmax over the top-k kept set (ties kept)."""
    l = np.asarray(l, dtype=np.float64)
    keep = np.ones_like(l, dtype=bool)
    if 0 < top_k < l.shape[-1]:
        kth = np.sort(l)[::-1][top_k - 1]
        keep = l >= kth
    z = np.where(keep, l / T, -np.inf)
    return special.softmax(z)


def _probs_rows(rows, T, top_k=0):
    return np.stack([_softmax(r, T, top_k) for r in rows])


# --------------------------------------------------------------------------
# decoding, row statistics, argmax
# --------------------------------------------------------------------------
def test_bf16_decode_matches_torch(orc):
    bits = np.arange(65536, dtype=np.uint16)
    f = W.bf16_bits_to_f32(bits)
    keep = ~np.isnan(f)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    for i in np.flatnonzero(keep)[::97]:
        assert orc._load().orc_decode(bits[i:i + 1].ctypes.data, 1, 0) == ref[i]
    # generator-side RNE cast agrees with torch's float -> bf16 rounding
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    mine = W.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, theirs)


def test_f16_decode_matches_numpy(orc):
    # every binary16 pattern: zeros, subnormals, normals, infinities, NaNs
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    dec = orc._load().orc_decode
    got = np.array([dec(bits[i:i + 1].ctypes.data, 2, 0) for i in range(65536)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # generator-side cast agrees with torch's float -> float16 rounding
    x = np.random.default_rng(1).standard_normal(100000).astype(np.float32) * 7
    theirs = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.f32_to_f16_bits(x), theirs)


@pytest.mark.parametrize("T", [0.05, 0.7, 1.0, 5.0])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_row_probs_vs_scipy(orc, T, dtype):
    rng = np.random.default_rng(7)
    l = (rng.standard_normal(3001) * 3).astype(np.float32)
    row = l if dtype == "f32" else W.f32_to_bf16_bits(l) if dtype == "bf16" else W.f32_to_f16_bits(l)
    lf = W.decode_f32(row, dtype)
    prob, st = orc.row_probs(row, dtype, T)
    lse = special.logsumexp(lf.astype(np.float64) / T)
    assert st["m"] == lf.max()
    assert abs((st["m"] / T + np.log(st["S"])) - lse) < 1e-12 * max(1, abs(lse))
    np.testing.assert_allclose(prob, special.softmax(lf.astype(np.float64) / T), rtol=1e-12, atol=1e-300)
    assert abs(prob.sum() - 1) < 1e-12


@pytest.mark.parametrize("k", [1, 5, 50, 3000])
def test_top_k_threshold_vs_torch_topk(orc, k):
    rng = np.random.default_rng(k)
    l = rng.integers(-40, 40, 3001).astype(np.float32) / 4  # many ties
    prob, st = orc.row_probs(l, "f32", 0.7, k)
    tau = torch.topk(torch.from_numpy(l).double(), k).values[k - 1].item()
    assert st["tau"] == tau
    assert st["kept"] == int((l >= tau).sum()) >= k
    assert np.all(prob[l < tau] == 0) and np.all(prob[l >= tau] > 0)
    np.testing.assert_allclose(prob, _softmax(l, 0.7, k), rtol=1e-12, atol=1e-300)


def test_top_k_at_or_above_vocab_is_off(orc):
    l = np.random.default_rng(3).standard_normal(64).astype(np.float32)
    p0, _ = orc.row_probs(l, "f32", 1.0, 0)
    p1, st = orc.row_probs(l, "f32", 1.0, 64)
    assert np.array_equal(p0, p1) and st["kept"] == 64


def test_argmax_first_index_vs_numpy(orc):
    rng = np.random.default_rng(11)
    for _ in range(50):
        l = rng.integers(-5, 5, 257).astype(np.float32)  # ties at the max
        assert orc.row_argmax(l, "f32") == int(np.argmax(l))
    l = np.full(9, -np.inf, np.float32)
    l[[3, 6]] = 2.0
    assert orc.row_argmax(l, "f32") == 3


# --------------------------------------------------------------------------
# beta identity (residual normaliser = 1 - beta) on every workload shape
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,batch", [(1, 1), (2, 1), (3, 6), (4, 2), (5, 4)])
def test_residual_mass_is_one_minus_beta(orc, cfg, batch):
    w = W.make_config(cfg, batch=batch)
    r = orc.verify_workload(w, threads=4)
    T = w.temperature
    tf, df = w.target_f32(), w.draft_f32()
    checked = 0
    for b in range(w.batch):
        n = r["num_accepted"][b]
        K = w.draft_lens[b]
        assert 0 <= n <= K
        if n == K:
            assert r["residual_mass"][b] == 0
            continue
        p = _softmax(tf[w.cu_draft[b] + b + n], T, w.top_k)
        q = _softmax(df[w.cu_draft[b] + n], T, w.top_k)
        beta = np.minimum(p, q).sum()
        assert abs(r["residual_mass"][b] - (1 - beta)) < 1e-12
        checked += 1
    # per-position p(x), q(x) against scipy
    for b in range(w.batch):
        for k in range(w.draft_lens[b]):
            x = w.draft_ids[w.cu_draft[b] + k]
            p = _softmax(tf[w.cu_draft[b] + b + k], T, w.top_k)[x]
            q = _softmax(df[w.cu_draft[b] + k], T, w.top_k)[x]
            np.testing.assert_allclose(r["probs"][w.cu_draft[b] + k], [p, q], rtol=1e-10)
    assert checked > 0 or cfg == 1


# --------------------------------------------------------------------------
# Exhaustive enumeration of the 2^24 uniforms on a tiny vocabulary
# --------------------------------------------------------------------------
def _enumerate_core(orc, P, Q, x, which):
    """Run the oracle core once per 24-bit uniform value of one draw.

    which = "acc": u_acc over the grid (u_res = 0); "res": u_acc forced to
    reject (u = 1 - 2^-24 rejects unless the ratio is 1), u_res over the
    grid; "bonus": u_acc = 0, u_bonus over the grid.
    Returns the emitted token at position 0 (K = 1) or at K, per grid value.
    """
    K = P.shape[0] - 1
    out = []
    step = 2**22
    for s in range(0, GRID, step):
        u = (np.arange(s, s + step, dtype=np.float64)) / GRID
        if which == "acc":
            ua = np.repeat(u[:, None], K, 1)
            ur = np.zeros((step, K))
            ub = np.zeros(step)
        elif which == "res":
            ua = np.full((step, K), 1 - 1 / GRID)
            ur = np.repeat(u[:, None], K, 1)
            ub = np.zeros(step)
        else:
            ua = np.zeros((step, K))
            ur = np.zeros((step, K))
            ub = u
        tok, n = orc.verify_seq_u_batch(P, Q, x, ua, ur, ub)
        out.append((tok, n))
    tok = np.concatenate([t for t, _ in out])
    n = np.concatenate([m for _, m in out])
    return tok, n


@pytest.mark.slow
def test_exact_law_by_exhaustive_enumeration(orc):
    """P(emitted = v) = min(p, q)(v) + (1 - beta) p'(v) = p(v), to within V * 2^-24."""
    V = 4
    lt = np.array([0.3, -1.2, 1.1, 0.0])
    ld = np.array([-0.4, 0.9, 0.2, 0.5])
    T = 0.9
    p = _softmax(lt, T)
    q = _softmax(ld, T)
    P = np.stack([p, _softmax(np.array([1.0, 0.0, -1.0, 2.0]), T)])
    Q = q[None, :]
    # the residual law does not depend on which guess was rejected: enumerate once
    x_rej = int(np.argmax(q / p))  # a guess with q > p, so the forced reject is real
    tok_r, n_r = _enumerate_core(orc, P, Q, np.array([x_rej]), "res")
    assert np.all(n_r == 0)
    law_res = np.bincount(tok_r[:, 0], minlength=V) / GRID
    resid = np.maximum(p - q, 0)
    np.testing.assert_allclose(law_res, resid / resid.sum(), atol=V / GRID)
    law = np.zeros(V)
    for x in range(V):
        tok_a, n_a = _enumerate_core(orc, P, Q, np.array([x]), "acc")
        acc = np.mean(n_a == 1)
        # accept fraction on the 2^24 grid = ceil(min(1, p/q) * 2^24) / 2^24
        assert acc == np.ceil(min(1.0, p[x] / q[x]) * GRID) / GRID
        assert np.all(tok_a[n_a == 1, 0] == x)
        law += q[x] * (acc * np.eye(V)[x] + (1 - acc) * law_res)
    np.testing.assert_allclose(law, p, atol=2 * V / GRID)
    # bonus: all accepted -> emitted token at position K follows p_K
    x_acc = int(np.argmax(p / q))
    tok_b, n_b = _enumerate_core(orc, P, Q, np.array([x_acc]), "bonus")
    assert np.all(n_b == 1)
    law_b = np.bincount(tok_b[:, 1], minlength=V) / GRID
    np.testing.assert_allclose(law_b, P[1], atol=V / GRID)


# --------------------------------------------------------------------------
# Seeded, end-to-end statistical checks
# --------------------------------------------------------------------------
def _replicated_batch(lt_rows, ld_rows, ids_per_seq, dtype="f32"):
    """B identical sequences (different uniforms through b) with given ids."""
    B, K = ids_per_seq.shape
    V = lt_rows.shape[1]
    tgt = np.tile(lt_rows.astype(np.float32), (B, 1))
    drf = np.tile(ld_rows.astype(np.float32), (B, 1)) if K else np.zeros((0, V), np.float32)
    cu = np.arange(B + 1, dtype=np.int32) * K
    return tgt, drf, ids_per_seq.reshape(-1).astype(np.int32), cu


@pytest.mark.slow
def test_chi_square_first_token_is_p(orc):
    """10^6 trials, x ~ q drawn per trial: the first emitted token follows p_0,
    and the bonus token (all accepted) follows p_K."""
    rng = np.random.default_rng(2024)
    V, K, T = 8, 2, 0.8
    lt = rng.standard_normal((K + 1, V)) * 1.5
    ld = lt[:K] + rng.standard_normal((K, V))
    lt32, ld32 = lt.astype(np.float32), ld.astype(np.float32)
    P = _probs_rows(lt32, T)
    Q = _probs_rows(ld32, T)
    B = 10**6
    ids = np.stack([rng.choice(V, B, p=Q[k]) for k in range(K)], 1)
    tgt, drf, x, cu = _replicated_batch(lt32, ld32, ids)
    r = orc.verify_sample(tgt, drf, x, cu, V, "f32", T, 0, seed=99, offset=5, threads=8)
    tok = r["tokens"].reshape(B, K + 1)
    first = tok[:, 0]
    assert np.all(first >= 0)
    obs = np.bincount(first, minlength=V)
    assert stats.chisquare(obs, P[0] * B).pvalue > 1e-3
    allacc = r["num_accepted"] == K
    obs_b = np.bincount(tok[allacc, K], minlength=V)
    assert stats.chisquare(obs_b, P[K] * allacc.sum()).pvalue > 1e-3
    # averaged over x ~ q the acceptance rate of position 0 is beta_0
    beta0 = np.minimum(P[0], Q[0]).sum()
    acc0 = np.mean(r["num_accepted"] >= 1)
    assert abs(acc0 - beta0) < 5 * np.sqrt(beta0 * (1 - beta0) / B)


@pytest.mark.slow
def test_accept_count_law(orc):
    """Fixed inputs: P(n >= j) = prod_{k<j} min(1, p_k(x_k)/q_k(x_k))."""
    rng = np.random.default_rng(5)
    V, K, T = 6, 4, 1.0
    lt = (rng.standard_normal((K + 1, V)) * 1.2).astype(np.float32)
    ld = (lt[:K] + rng.standard_normal((K, V)) * 0.8).astype(np.float32)
    P, Q = _probs_rows(lt, T), _probs_rows(ld, T)
    x = np.array([int(np.argmax(Q[k])) for k in range(K)])
    B = 10**5
    tgt, drf, ids, cu = _replicated_batch(lt, ld, np.tile(x, (B, 1)))
    r = orc.verify_sample(tgt, drf, ids, cu, V, "f32", T, 0, seed=7, offset=0, threads=8)
    ratio = np.minimum(1, P[np.arange(K), x] / Q[np.arange(K), x])
    law = np.array([np.prod(ratio[:j]) * (1 - ratio[j]) for j in range(K)] + [np.prod(ratio)])
    obs = np.bincount(r["num_accepted"], minlength=K + 1)
    keep = law * B > 5
    exp_ = law[keep] * B
    obs_k = obs[keep]
    assert obs[~keep].sum() <= max(10, 10 * law[~keep].sum() * B)
    assert stats.chisquare(obs_k, exp_ * obs_k.sum() / exp_.sum()).pvalue > 1e-3


# --------------------------------------------------------------------------
# Greedy: target argmax at every emitted position
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cfg,batch", [(1, 1), (4, 3), (5, 5)])
def test_greedy_is_target_argmax(orc, cfg, batch):
    w = W.make_config(cfg, batch=batch)
    ids = w.draft_ids.copy()
    tf = w.target_f32()
    # make some sequences fully accepted and some partially, by planting argmaxes
    for b in range(w.batch):
        for k in range(w.draft_lens[b]):
            if b % 2 == 0 or k < w.draft_lens[b] // 2:
                ids[w.cu_draft[b] + k] = int(np.argmax(tf[w.cu_draft[b] + b + k]))
    r = orc.verify_greedy(w.target, ids, w.cu_draft, w.vocab, w.dtype)
    for b in range(w.batch):
        K = w.draft_lens[b]
        a = [int(np.argmax(tf[w.cu_draft[b] + b + k])) for k in range(K + 1)]
        x = ids[w.cu_draft[b]:w.cu_draft[b + 1]]
        n = next((k for k in range(K) if x[k] != a[k]), K)
        want = list(x[:n]) + [a[n]] + [-1] * (K - n)
        got = r["tokens"][w.cu_draft[b] + b: w.cu_draft[b] + b + K + 1]
        assert r["num_accepted"][b] == n
        assert list(got) == want


# --------------------------------------------------------------------------
# Special cases with known answers
# --------------------------------------------------------------------------
def test_draft_equals_target_accepts_everything(orc):
    rng = np.random.default_rng(1)
    B, K, V = 200, 5, 33
    lt = (rng.standard_normal((K + 1, V)) * 2).astype(np.float32)
    ids = np.stack([rng.integers(0, V, K) for _ in range(B)])
    tgt, drf, x, cu = _replicated_batch(lt, lt[:K], ids)
    r = orc.verify_sample(tgt, drf, x, cu, V, "f32", 0.9, 0, seed=3, offset=1)
    assert np.all(r["num_accepted"] == K)
    assert np.all(r["residual_mass"] == 0)
    tok = r["tokens"].reshape(B, K + 1)
    assert np.array_equal(tok[:, :K], ids)


def test_disjoint_top_k_supports_reject_at_zero(orc):
    V, K = 20, 3
    lt = np.zeros((K + 1, V), np.float32)
    ld = np.zeros((K, V), np.float32)
    lt[:, :5] = np.arange(5, 0, -1)  # target keeps ids 0..4 (top-5)
    ld[:, 10:15] = np.arange(5, 0, -1)  # draft keeps ids 10..14
    ids = np.array([[10, 11, 12]])
    tgt, drf, x, cu = _replicated_batch(lt, ld, ids)
    r = orc.verify_sample(tgt, drf, x, cu, V, "f32", 1.0, 5, seed=0, offset=0)
    assert r["num_accepted"][0] == 0
    assert r["probs"][0, 0] == 0 and r["probs"][0, 1] > 0
    assert abs(r["residual_mass"][0] - 1.0) < 1e-15  # residual is p_0 itself
    assert 0 <= r["tokens"][0] < 5
    assert list(r["tokens"][1:]) == [-1, -1, -1]


def test_vocab_of_one(orc):
    B, K = 10, 4
    tgt, drf, x, cu = _replicated_batch(np.zeros((K + 1, 1)), np.ones((K, 1)), np.zeros((B, K), int))
    r = orc.verify_sample(tgt, drf, x, cu, 1, "f32", 1.0, 0, seed=1, offset=0)
    assert np.all(r["num_accepted"] == K) and np.all(r["tokens"] == 0)


def test_point_mass_draft(orc):
    """q = delta_x: accept probability p(x), residual p with x removed, Z = 1 - p(x)."""
    rng = np.random.default_rng(9)
    V, K, T = 12, 1, 1.0
    lt = rng.standard_normal((K + 1, V)).astype(np.float32)
    ld = np.full((K, V), -np.inf, np.float32)
    ld[0, 4] = 0.0
    p = _softmax(lt[0], T)
    B = 200000
    tgt, drf, ids, cu = _replicated_batch(lt, ld, np.full((B, 1), 4))
    r = orc.verify_sample(tgt, drf, ids, cu, V, "f32", T, 0, seed=12, offset=0, threads=8)
    rej = r["num_accepted"] == 0
    assert abs(np.mean(~rej) - p[4]) < 5 * np.sqrt(p[4] * (1 - p[4]) / B)
    np.testing.assert_allclose(r["residual_mass"][rej], 1 - p[4], rtol=1e-12)
    first = r["tokens"].reshape(B, 2)[rej, 0]
    assert not np.any(first == 4)
    want = np.where(np.arange(V) == 4, 0, p) / (1 - p[4])
    obs = np.bincount(first, minlength=V)
    m = want > 0
    assert stats.chisquare(obs[m], want[m] * rej.sum()).pvalue > 1e-3


def test_zero_residual_falls_back_to_p(orc):
    """A guess outside both top-k sets has p = q = 0 and is rejected; with equal
    rows the residual has no mass and the token is drawn from p_n."""
    V = 10
    l = np.arange(V, dtype=np.float32)[::-1].copy()
    tgt, drf, ids, cu = _replicated_batch(np.stack([l, l]), l[None], np.array([[9]]))
    r = orc.verify_sample(tgt, drf, ids, cu, V, "f32", 1.0, 3, seed=0, offset=0)
    assert r["num_accepted"][0] == 0
    assert r["flags"][0] & orc.FLAG_ZERO_RESIDUAL
    assert r["residual_mass"][0] == 0
    assert 0 <= r["tokens"][0] < 3


def test_hand_worked_example(orc):
    """V = 3, T = 1, p = (0.5, 0.3, 0.2), q = (0.2, 0.5, 0.3), guess x = 1.
    Ratio p/q = 0.6: u = 0.59 accepts, u = 0.6 rejects (strict <).  The
    residual max(0, p - q) = (0.3, 0, 0) has mass 0.3 = 1 - beta
    (beta = 0.2 + 0.3 + 0.2 = 0.7), so a rejection always emits id 0.
    Bonus row p_1 = (1/8, 5/8, 1/4) (edges 0.125 and 0.75 are exact in
    binary): u = 0.05 -> 0, 0.125 -> 1 (the running mass must exceed u),
    0.74 -> 1, 0.75 -> 2."""
    P = np.array([[0.5, 0.3, 0.2], [0.125, 0.625, 0.25]])
    Q = np.array([[0.2, 0.5, 0.3]])
    r = orc.verify_seq_u(P, Q, [1], [0.59], [0.0], 0.05)
    assert r["n"] == 1 and list(r["tokens"]) == [1, 0]
    assert abs(r["d_acc"][0] - 0.01) < 1e-12
    r = orc.verify_seq_u(P, Q, [1], [0.6], [0.999], 0.05)
    assert r["n"] == 0 and list(r["tokens"]) == [0, -1]
    assert abs(r["z"] - 0.3) < 1e-15
    for ub, want in [(0.05, 0), (0.125, 1), (0.74, 1), (0.75, 2), (0.999, 2)]:
        r = orc.verify_seq_u(P, Q, [1], [0.0], [0.0], ub)
        assert r["tokens"][1] == want, (ub, r)
    # the eps-window around a CDF edge spans both neighbours
    r = orc.verify_seq_u(P, Q, [1], [0.0], [0.0], 0.75 - 1e-8, eps=1e-6)
    assert (r["tok_lo"], r["tok_hi"]) == (1, 2) and r["d_fin"] < 1e-6


# --------------------------------------------------------------------------
# draft-side sampling (the guesses x ~ q that the proof assumes)
# --------------------------------------------------------------------------
def _one_row_per_sequence(row, B, dtype="f32"):
    rows = np.repeat(np.asarray(row, np.float32)[None, :], B, axis=0)
    return (rows if dtype == "f32" else W.f32_to_bf16_bits(rows)), np.arange(B + 1, dtype=np.int32)


@pytest.mark.parametrize("top_k", [0, 5])
def test_draft_sample_law_chi_square(orc, top_k):
    """2*10^5 independent draws (one per sequence, distinct counters) follow
    q = softmax(l / T) over the top-k kept set, by a chi-square test against
    scipy's softmax."""
    rng = np.random.default_rng(31)
    V, T, B = 8, 0.8, 200000
    row = (rng.standard_normal(V) * 1.5).astype(np.float32)
    rows, cu = _one_row_per_sequence(row, B)
    r = orc.draft_sample(rows, cu, V, "f32", T, top_k, seed=7, offset=3, threads=8)
    q = _softmax(row, T, top_k)
    obs = np.bincount(r["ids"], minlength=V)
    assert obs[q == 0].sum() == 0
    keep = q > 0
    assert stats.chisquare(obs[keep], q[keep] * B).pvalue > 1e-3


def test_draft_sample_top_k_1_is_argmax(orc):
    # distinct logits: top_k = 1 keeps only the maximum, so the draw is numpy's argmax
    rng = np.random.default_rng(5)
    rows = (rng.standard_normal((64, 500)) * 3).astype(np.float32)
    cu = np.array([0, 10, 10, 40, 64], np.int32)
    r = orc.draft_sample(rows, cu, 500, "f32", 0.9, 1, seed=1, offset=0)
    assert np.array_equal(r["ids"], np.argmax(rows, axis=1))
    # a tied maximum is kept whole (ties at tau are kept): every draw is one of the tied ids
    tied = rng.integers(-20, 20, (64, 500)).astype(np.float32) / 2
    r = orc.draft_sample(tied, cu, 500, "f32", 0.9, 1, seed=1, offset=0)
    assert np.all(tied[np.arange(64), r["ids"]] == tied.max(axis=1))


def test_draft_sample_single_finite_logit(orc):
    rows = np.full((6, 40), -np.inf, np.float32)
    for i in range(6):
        rows[i, (7 * i) % 40] = 0.5 * i
    r = orc.draft_sample(rows, np.array([0, 6], np.int32), 40, "f32", 1.0, 0, seed=4, offset=9)
    assert np.array_equal(r["ids"], (7 * np.arange(6)) % 40)


def test_draft_sample_seed_and_offset_move_the_draws(orc):
    rng = np.random.default_rng(8)
    rows = (rng.standard_normal((200, 50)) * 0.3).astype(np.float32)  # flat: draws spread out
    cu = np.array([0, 200], np.int32)
    a = orc.draft_sample(rows, cu, 50, "f32", 1.0, 0, seed=1, offset=0)["ids"]
    b = orc.draft_sample(rows, cu, 50, "f32", 1.0, 0, seed=2, offset=0)["ids"]
    c = orc.draft_sample(rows, cu, 50, "f32", 1.0, 0, seed=1, offset=1)["ids"]
    assert (a != b).mean() > 0.5 and (a != c).mean() > 0.5


# --------------------------------------------------------------------------
# the argmax-draw variant (OpenVINO notebook's steps 3-4)
# --------------------------------------------------------------------------
def test_argmax_variant_residual_and_extra_token_vs_numpy(orc):
    """At a rejection the token is numpy's argmax of max(0, p_n - q_n) with p
    and q from scipy's softmax; when every guess passes it is numpy's argmax
    of p_K.  Acceptance counts equal the sampling variant's (same uniforms)."""
    w = W.make_workload(dict(W.WORKLOADS[2], name="argmax_pin"), gen_seed=3, batch=24)
    a = orc.verify_workload(w, "argmax", threads=8)
    s = orc.verify_workload(w, "sample", threads=8)
    assert np.array_equal(a["num_accepted"], s["num_accepted"])
    tf, df = w.target_f32(), w.draft_f32()
    seen_reject = seen_bonus = 0
    for b in range(w.batch):
        k0, k1 = w.cu_draft[b], w.cu_draft[b + 1]
        n = a["num_accepted"][b]
        tok = a["tokens"][k0 + b + n]
        if n < k1 - k0:
            p = _softmax(tf[k0 + b + n], w.temperature, w.top_k)
            q = _softmax(df[k0 + n], w.temperature, w.top_k)
            r = np.maximum(p - q, 0.0)
            assert tok == int(np.argmax(r))
            seen_reject += 1
        else:
            assert tok == int(np.argmax(tf[k0 + b + n]))
            seen_bonus += 1
    assert seen_reject > 0


def _best_and_runner_up(wt):
    """numpy reference for the argmax draw: the lowest id of the largest
    positive weight; the runner-up is the lowest id of the largest positive
    weight among the other ids (-1 when there is none); gap = (best -
    runner-up) / best, 1 with no runner-up."""
    pos = np.flatnonzero(wt > 0)
    if pos.size == 0:
        return -1, -1, 0.0
    order = pos[np.lexsort((pos, -wt[pos]))]  # descending weight, ascending id among equals
    best = int(order[0])
    if order.size == 1:
        return best, -1, 1.0
    sec = int(order[1])
    return best, sec, float((wt[best] - wt[sec]) / wt[best])


def test_argmax_variant_gap_and_runner_up_vs_numpy(orc):
    """The argmax variant also reports, per sequence, the runner-up id of its
    final argmax and the relative gap to it (the GPU test accepts either id
    when the gap is small).  Against numpy on max(0, p_n - q_n) (or p_K) from
    scipy's softmax: the runner-up is the best other id, the gap its margin."""
    w = W.make_workload(dict(W.WORKLOADS[2], name="argmax_gap_pin"), gen_seed=3, batch=24)
    a = orc.verify_workload(w, "argmax", threads=8)
    tf, df = w.target_f32(), w.draft_f32()
    for b in range(w.batch):
        k0, k1 = w.cu_draft[b], w.cu_draft[b + 1]
        n = a["num_accepted"][b]
        p = _softmax(tf[k0 + b + n], w.temperature, w.top_k)
        wt = np.maximum(p - _softmax(df[k0 + n], w.temperature, w.top_k), 0.0) if n < k1 - k0 else p
        best, sec, gap = _best_and_runner_up(wt)
        assert a["tokens"][k0 + b + n] == best
        assert a["second"][b] == sec
        assert abs(a["gap"][b] - gap) <= 1e-9 * max(1.0, gap)


# Hand-built rows (V = 4, T = 1, fp32): (target row 0, target row 1, draft row
# 0, guess) -> (token, runner-up, gap).  A draft equal to target row 0 accepts
# its guess (p = q), so the token is the argmax of p_1; a point-mass draft
# (q = 1 at the guess, where p is about e^-33) rejects it, and the residual is
# p_0 on the other ids.
_NEG = -np.inf
ARGMAX_CASES = {
    "extra_tie_at_max": ([0, 0, 0, 0], [0, 3, 3, 1], None, 0, (1, 2, 0.0)),
    "extra_tie_at_runner_up": ([0, 0, 0, 0], [5, 1, 3, 3], None, 0, (0, 2, 1 - np.exp(-2.0))),
    "extra_max_after_runner_up": ([0, 0, 0, 0], [1, 3, 5, 0], None, 0, (2, 1, 1 - np.exp(-2.0))),
    "extra_single_positive": ([0, 0, 0, 0], [0, _NEG, _NEG, _NEG], None, 0, (0, -1, 1.0)),
    "residual_tie_at_max": ([3, 3, 1, -30], [0, 0, 0, 0], [_NEG, _NEG, _NEG, 0], 3, (0, 1, 0.0)),
    "residual_runner_up_after_max": ([1, 4, 2, -30], [0, 0, 0, 0], [_NEG, _NEG, _NEG, 0], 3,
                                     (1, 2, 1 - np.exp(-2.0))),
    "residual_single_positive": ([2, _NEG, _NEG, -30], [0, 0, 0, 0], [_NEG, _NEG, _NEG, 0], 3, (0, -1, 1.0)),
}


@pytest.mark.parametrize("name", sorted(ARGMAX_CASES))
def test_argmax_variant_gap_and_runner_up_hand_cases(orc, name):
    t0, t1, d0, x, (tok, sec, gap) = ARGMAX_CASES[name]
    tgt = np.array([t0, t1], np.float32)
    drf = np.array([d0 if d0 is not None else t0], np.float32)
    a = orc.verify_argmax(tgt, drf, np.array([x], np.int32), np.array([0, 1], np.int32), 4, "f32", 1.0, 0, 0, 0)
    n = 1 if d0 is None else 0
    assert a["num_accepted"][0] == n
    assert a["tokens"][n] == tok
    assert a["second"][0] == sec
    assert a["gap"][0] == pytest.approx(gap, rel=1e-12, abs=1e-15)


def test_argmax_variant_draft_equals_target(orc):
    w = W.make_workload(dict(W.WORKLOADS[1], name="argmax_eq", batch=6), gen_seed=4)
    a = orc.verify_argmax(w.target, w.target[np.concatenate([np.arange(w.cu_draft[b] + b, w.cu_draft[b + 1] + b)
                                                            for b in range(w.batch)])],
                          w.draft_ids, w.cu_draft, w.vocab, w.dtype, w.temperature, 0, 0, 0)
    K = w.k_max
    assert np.all(a["num_accepted"] == K)
    tf = w.target_f32()
    for b in range(w.batch):
        assert a["tokens"][b * (K + 1) + K] == int(np.argmax(tf[b * (K + 1) + K]))


# --------------------------------------------------------------------------
# per-token speculative likelihood (the perplexity check of
# "CS3602_FINAL_SpeDec": accept part + reject part of an observed token)
# --------------------------------------------------------------------------
def _lik_rows(seed, R, V, dtype, scale=2.0):
    rng = np.random.default_rng(seed)
    t = (rng.standard_normal((R, V)) * scale).astype(np.float32)
    d = (t + rng.standard_normal((R, V)).astype(np.float32)).astype(np.float32)
    enc = {"f32": lambda x: x, "bf16": W.f32_to_bf16_bits, "f16": W.f32_to_f16_bits}[dtype]
    return enc(t), enc(d)


@pytest.mark.parametrize("dtype,top_k,T", [("f32", 0, 1.0), ("bf16", 0, 0.7), ("bf16", 20, 1.3), ("f16", 5, 0.5)])
def test_likelihood_terms_vs_scipy(orc, dtype, top_k, T):
    """Against scipy's softmax: the accept part is min(p, q)(y); the reject part
    is max(0, p - q)(y) (the proof's identity (1 - beta) p'(y) = p(y) - min);
    their sum is p(y), the proof's claim that accept-or-resample emits y with
    probability p(y); beta = 1 - sum max(0, p - q); and the sequence's NLL
    equals the target's own, -sum log p(y) from scipy's log_softmax."""
    R, V = 12, 400
    tgt, drf = _lik_rows(3, R, V, dtype)
    cu = np.array([0, 5, 5, 12], np.int32)   # three sequences, one empty
    rng = np.random.default_rng(4)
    tf, df = W.decode_f32(tgt, dtype), W.decode_f32(drf, dtype)
    P, Q = _probs_rows(tf, T, top_k), _probs_rows(df, T, top_k)
    # tokens inside the target's support (else p(y) = 0 and the NLL is infinite)
    tok = np.array([rng.choice(np.flatnonzero(P[r] > 0)) for r in range(R)], np.int32)
    o = orc.token_likelihood(tgt, drf, tok, cu, V, dtype, T, top_k)
    py, qy = P[np.arange(R), tok], Q[np.arange(R), tok]
    np.testing.assert_allclose(o["p"], py, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(o["accept"], np.minimum(py, qy), rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(o["reject"], np.maximum(py - qy, 0), rtol=1e-9, atol=1e-15)
    np.testing.assert_allclose(o["accept"] + o["reject"], py, rtol=1e-12, atol=1e-300)
    np.testing.assert_allclose(o["beta"], 1 - np.maximum(P - Q, 0).sum(axis=1), rtol=0, atol=1e-13)
    assert np.all(o["flags"] == 0)
    for b in range(3):
        ks = slice(cu[b], cu[b + 1])
        lsm = np.array([special.log_softmax(np.where(P[r] > 0, tf[r].astype(np.float64) / T, -np.inf))[tok[r]]
                        for r in range(cu[b], cu[b + 1])])
        want = -lsm.sum() if lsm.size else 0.0
        assert abs(o["nll"][b] - want) <= 1e-11 * max(1.0, abs(want)), (b, o["nll"][b], want)
        assert np.all(np.isfinite(o["accept"][ks]))


def test_likelihood_hand_worked_example(orc):
    """V = 4, T = 1, p = (1/2, 1/4, 1/8, 1/8), q = (1/4, 1/4, 1/4, 1/4):
    beta = 1/4 + 1/4 + 1/8 + 1/8 = 3/4 and the residual max(0, p - q) =
    (1/4, 0, 0, 0) has mass 1/4 = 1 - beta.  y = 0: accepted with 1/4,
    emitted after a rejection with (1 - 3/4) * 1 = 1/4, total 1/2 = p(0).
    y = 1: 1/4 + 0.  y = 2: 1/8 + 0.  NLL of (0, 1, 2) = ln 2 + ln 4 + ln 8."""
    p = np.array([0.5, 0.25, 0.125, 0.125])
    q = np.full(4, 0.25)
    tgt = np.log(np.repeat(p[None], 3, 0)).astype(np.float32)
    drf = np.log(np.repeat(q[None], 3, 0)).astype(np.float32)
    o = orc.token_likelihood(tgt, drf, np.array([0, 1, 2], np.int32), np.array([0, 3], np.int32), 4, "f32",
                             1.0, 0)
    np.testing.assert_allclose(o["beta"], 0.75, atol=1e-7)
    np.testing.assert_allclose(o["accept"], [0.25, 0.25, 0.125], atol=1e-7)
    np.testing.assert_allclose(o["reject"], [0.25, 0.0, 0.0], atol=1e-7)
    assert abs(o["nll"][0] - np.log(64.0)) < 1e-6


def test_likelihood_beta_is_the_acceptance_rate(orc):
    """beta is the probability that a guess x ~ q passes the acceptance test:
    sum_x q(x) min(1, p(x)/q(x)).  The oracle's own verify step, run over
    20000 sequences with the same row pair, guesses drawn from q with
    numpy and a different Philox stream per sequence, accepts the first
    guess at a rate within 4.5 binomial sigma of the likelihood's beta."""
    V, N, T = 40, 20000, 0.9
    rng = np.random.default_rng(9)
    lt = (rng.standard_normal(V) * 1.5).astype(np.float32)
    ld = (lt + rng.standard_normal(V) * 1.2).astype(np.float32)
    lik = orc.token_likelihood(lt[None], ld[None], np.zeros(1, np.int32), np.array([0, 1], np.int32), V, "f32",
                               T, 0)
    beta = float(lik["beta"][0])
    q = _softmax(ld, T)
    x = rng.choice(V, size=N, p=q).astype(np.int32)
    tgt = np.repeat(np.stack([lt, lt])[None], N, 0).reshape(2 * N, V)  # target rows k = 0, 1 per sequence
    drf = np.repeat(ld[None], N, 0)
    cu = np.arange(N + 1, dtype=np.int32)
    o = orc.verify_sample(tgt, drf, x, cu, V, "f32", T, 0, 1234, 0, threads=8)
    rate = float(np.mean(o["num_accepted"] >= 1))
    sigma = np.sqrt(beta * (1 - beta) / N)
    assert abs(rate - beta) < 4.5 * sigma, (rate, beta, sigma)


def test_likelihood_special_cases(orc):
    V = 300
    tgt, drf = _lik_rows(5, 4, V, "f32")
    tok = np.array([3, 7, 11, 299], np.int32)
    cu = np.array([0, 4], np.int32)
    # draft = target: every guess is accepted, nothing comes from the residual
    o = orc.token_likelihood(tgt, tgt, tok, cu, V, "f32", 1.0, 0)
    np.testing.assert_allclose(o["beta"], 1.0, atol=1e-13)
    assert np.all(o["reject"] == 0) and np.allclose(o["accept"], o["p"], rtol=1e-15)
    # disjoint top-k supports: beta = 0, every emitted token comes from the residual
    t2 = np.full((1, 10), -5.0, np.float32)
    d2 = np.full((1, 10), -5.0, np.float32)
    t2[0, :3] = [3.0, 2.0, 1.0]
    d2[0, 5:8] = [3.0, 2.0, 1.0]
    o = orc.token_likelihood(t2, d2, np.array([1], np.int32), np.array([0, 1], np.int32), 10, "f32", 1.0, 3)
    assert o["beta"][0] == 0.0 and o["accept"][0] == 0.0
    assert abs(o["reject"][0] - _softmax(t2[0], 1.0, 3)[1]) < 1e-15
    # V = 1: p = q = 1, NLL 0
    o = orc.token_likelihood(np.zeros((2, 1), np.float32), np.ones((2, 1), np.float32), np.zeros(2, np.int32),
                             np.array([0, 2], np.int32), 1, "f32", 1.0, 0)
    assert np.all(o["beta"] == 1.0) and np.all(o["accept"] == 1.0) and o["nll"][0] == 0.0
    # a token outside the vocabulary flags its sequence and leaves NaN
    o = orc.token_likelihood(tgt, drf, np.array([3, V, 1, 2], np.int32), np.array([0, 2, 4], np.int32), V, "f32",
                             1.0, 0)
    assert o["flags"][0] != 0 and np.isnan(o["nll"][0]) and np.isnan(o["accept"][1])
    assert o["flags"][1] == 0 and np.isfinite(o["nll"][1])
    # a token outside the target's top-k kept set has likelihood 0
    o = orc.token_likelihood(t2, d2, np.array([9], np.int32), np.array([0, 1], np.int32), 10, "f32", 1.0, 3)
    assert o["accept"][0] == 0.0 and o["reject"][0] == 0.0 and o["nll"][0] == np.inf


# --------------------------------------------------------------------------
# top-p (nucleus) filter after top-k
# --------------------------------------------------------------------------
def test_top_p_one_is_no_filter(orc):
    rng = np.random.default_rng(12)
    l = (rng.standard_normal(500) * 2).astype(np.float32)
    for top_k in (0, 40):
        a, _ = orc.row_probs(l, "f32", 0.8, top_k)
        b, st = orc.row_probs(l, "f32", 0.8, top_k, top_p=1.0)
        assert np.array_equal(a, b) and st["margin"] == np.inf


def test_top_p_tiny_keeps_the_maxima(orc):
    # any top_p below the largest probability keeps exactly the tied maxima
    l = np.array([1.0, 3.0, -2.0, 3.0, 0.5, 3.0], np.float32)
    prob, st = orc.row_probs(l, "f32", 1.0, 0, top_p=1e-9)
    np.testing.assert_allclose(prob, [0, 1 / 3, 0, 1 / 3, 0, 1 / 3], atol=1e-15)
    assert st["tau_p"] == 3.0


def test_top_p_hand_worked_example(orc):
    """p = (1/2, 1/4, 1/8, 1/8) (logits ln p, T = 1).  top_p = 0.6: {0} holds
    0.5 < 0.6, {0, 1} holds 0.75, so the nucleus is {0, 1} renormalised to
    (2/3, 1/3).  top_p = 0.8: ids 2 and 3 tie at 1/8; 0.75 < 0.8, and adding
    the tied pair reaches 1, so both are kept (no arbitrary half of a tie)."""
    l = np.log(np.array([0.5, 0.25, 0.125, 0.125])).astype(np.float32)
    prob, st = orc.row_probs(l, "f32", 1.0, 0, top_p=0.6)
    np.testing.assert_allclose(prob, [2 / 3, 1 / 3, 0, 0], atol=1e-7)
    assert abs(st["margin"] - 0.1) < 1e-6   # 0.6 - 0.5 = 0.1 and 0.75 - 0.6 = 0.15: the smaller
    prob, st = orc.row_probs(l, "f32", 1.0, 0, top_p=0.8)
    np.testing.assert_allclose(prob, [0.5, 0.25, 0.125, 0.125], atol=1e-7)
    assert st["kept"] == 4
    # "reaches": a top_p equal to the mass of the two largest keeps exactly those two
    p1, _ = orc.row_probs(l, "f32", 1.0, 0)
    prob, st = orc.row_probs(l, "f32", 1.0, 0, top_p=float(p1[0] + p1[1]))
    assert st["kept"] == 2 and st["margin"] == 0.0


@pytest.mark.parametrize("top_k,top_p,T", [(0, 0.9, 1.0), (0, 0.5, 0.7), (50, 0.8, 1.0), (20, 0.95, 1.5),
                                           (0, 0.3, 2.0)])
def test_top_p_is_the_smallest_high_logit_set(orc, top_k, top_p, T):
    """Against scipy's softmax of the top-k set: the kept set is upward closed
    in the logit (every id above a kept one is kept), it holds at least top_p
    of the mass, dropping its lowest logit value takes it below top_p (so it
    is the smallest such set, ties kept whole), and the result is that
    softmax renormalised on the set.  Nested as top_p grows."""
    rng = np.random.default_rng(int(top_p * 100) + top_k)
    l = np.round(rng.standard_normal(3000) * 4, 1).astype(np.float32)   # many ties
    base = _softmax(l, T, top_k)
    prob, st = orc.row_probs(l, "f32", T, top_k, top_p=top_p)
    kept = prob > 0
    lo = l[kept].min()
    assert np.array_equal(kept, (base > 0) & (l >= lo))               # upward closed, ties whole
    assert base[kept].sum() >= top_p - 1e-12
    assert base[kept & (l > lo)].sum() < top_p + 1e-12                 # minimal
    np.testing.assert_allclose(prob[kept], base[kept] / base[kept].sum(), rtol=1e-12)
    assert st["tau_p"] == lo
    above = kept & (l > lo)
    m = min(base[kept].sum() - top_p, top_p - base[above].sum() if above.any() else np.inf)
    assert abs(st["margin"] - m) < 1e-12
    bigger, _ = orc.row_probs(l, "f32", T, top_k, top_p=min(1.0, top_p + 0.05))
    assert np.all(bigger[kept] > 0)


def test_draft_sample_law_with_top_p(orc):
    """Draws from the nucleus distribution: chi-square of 10^6 draft-side
    samples against the renormalised nucleus of scipy's softmax."""
    V, T, top_p = 60, 0.9, 0.85
    rng = np.random.default_rng(17)
    l = (rng.standard_normal(V) * 1.5).astype(np.float32)
    base = _softmax(l, T)
    order = np.argsort(-l, kind="stable")
    cum = np.cumsum(base[order])
    cut = l[order][np.searchsorted(cum, top_p)]        # logit at which the mass reaches top_p
    keep = l >= cut
    want = np.where(keep, base, 0) / base[keep].sum()
    N = 1_000_000
    rows, cu = _one_row_per_sequence(l, N)
    o = orc.draft_sample(rows, cu, V, "f32", T, 0, 0, 0, threads=8, top_p=top_p)
    assert np.all(keep[o["ids"]])
    counts = np.bincount(o["ids"], minlength=V)[keep]
    chi = stats.chisquare(counts, want[keep] * N)
    assert chi.pvalue > 1e-4, chi
