"""Pins for the CPU oracle against what the pages and the mathematics fix, independent of the
oracle's own code: closed forms, invariants, exhaustive search, exact rational arithmetic, library
routines for the special cases, and a hand-derived worked case (tests/golden/tiny_layer_L3.json).
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def harmonic(n):
    return sum(1.0 / m for m in range(1, n + 1))


# -- worked case -----------------------------------------------------------------------------------

def test_golden_tiny_layer():
    g = json.load(open(os.path.join(GOLDEN, "tiny_layer_L3.json")))
    i = g["inputs"]
    col = lambda v: np.array(v, dtype=np.float64).reshape(i["L"], 1, 1)
    out = oracle.layer(col(i["Q"]), col(i["K"]), col(i["V"]), col(i["X"]), i["tau"], i["q"])
    ex = g["expected"]
    np.testing.assert_allclose(out["s_h"][0], ex["s_h"], rtol=1e-14)
    np.testing.assert_allclose(out["s_l"], ex["s_l"], rtol=1e-14)
    assert (out["k"], out["Lp"]) == (ex["k"], ex["Lp"])
    assert out["idx"][0].tolist() == ex["idx"]
    np.testing.assert_allclose(out["Oh"][0, :, 0], ex["O_hat"], rtol=1e-14)
    np.testing.assert_allclose(out["Y"][:, 0, 0], ex["Y"], rtol=1e-14)


# -- scoring --------------------------------------------------------------------------------------

@pytest.mark.parametrize("L,q", [(1, 1), (7, 3), (64, 16), (200, 16), (300, 64)])
def test_score_zero_keys_closed_form(L, q):
    """K = 0: every visible logit is 0, so query p spreads 1/(p+1) over keys 0..p and
    s_h[t] = H_L - H_max(t, L-q) (harmonic numbers)."""
    Hq, Hkv, d = 4, 2, 8
    Q = rnd((L, Hq, d), 1)
    s = oracle.head_scores(Q, np.zeros((L, Hkv, d)), q)
    H = [harmonic(n) for n in range(L + 1)]
    want = np.array([H[L] - H[max(t, L - q)] for t in range(L)])
    for h in range(Hq):
        np.testing.assert_allclose(s[h], want, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("seed", range(4))
def test_score_rows_are_distributions(seed):
    L, Hq, Hkv, d, q = 97, 6, 3, 16, 11
    s = oracle.head_scores(rnd((L, Hq, d), seed, 2.0), rnd((L, Hkv, d), seed + 10, 2.0), q)
    np.testing.assert_allclose(s.sum(axis=1), q, rtol=1e-13)
    assert (s > 0).all()
    # the last q-1 keys are invisible to the earlier recent queries: key L-1 only to the last one
    assert (s[:, -1] <= 1.0 + 1e-15).all()


@pytest.mark.parametrize("seed", range(3))
def test_score_matches_library_attention_weights(seed):
    """With V = identity, scaled_dot_product_attention returns the attention weights themselves, so
    its column sums over the recent queries are s_h; the library applies its own scale 1/sqrt(d)."""
    L, Hq, Hkv, d, q = 40, 4, 2, 8, 5
    Q, K = rnd((L, Hq, d), seed), rnd((L, Hkv, d), seed + 100)
    s = oracle.head_scores(Q, K, q)
    G = Hq // Hkv
    recent = torch.arange(L - q, L)
    mask = torch.arange(L)[None, :] <= recent[:, None]
    for h in range(Hq):
        qt = torch.from_numpy(Q[L - q:, h, :])[None, None]
        kt = torch.from_numpy(K[:, h // G, :])[None, None]
        w = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, torch.eye(L, dtype=torch.float64)[None, None], attn_mask=mask[None, None])
        np.testing.assert_allclose(s[h], w[0, 0].sum(0).numpy(), rtol=1e-12)


def test_layer_score_normalised_and_equal_heads():
    L, d, q = 50, 8, 7
    Q1 = rnd((L, 1, d), 3)
    Q = np.repeat(Q1, 4, axis=1)
    K = rnd((L, 1, d), 4)
    s_h = oracle.head_scores(Q, K, q)
    s_l = oracle.layer_score(s_h)
    assert abs(s_l.sum() - 1) < 1e-14
    np.testing.assert_allclose(s_l, s_h[0] / q, rtol=1e-12)


def test_layer_score_hand_case():
    """Heads that disagree: column sums (1, 2, 5) over a total of 8, a head's zero kept as zero."""
    s_h = np.array([[1.0, 0.0, 3.0], [0.0, 2.0, 2.0]])
    assert oracle.layer_score(s_h).tolist() == [0.125, 0.25, 0.625]


# -- budget ---------------------------------------------------------------------------------------

def brute_budget(vals, tau):
    """k = min { j : min over j-subsets of the exact sum >= tau }, in exact rationals."""
    fv = [Fraction(v) for v in vals]
    ft = Fraction(tau)
    for j in range(len(fv) + 1):
        c = min(sum(c_, Fraction(0)) for c_ in itertools.combinations(fv, j)) if j else Fraction(0)
        if c >= ft:
            return j
    return len(fv)


@pytest.mark.parametrize("seed", range(12))
def test_budget_exhaustive_exact(seed):
    """Dyadic values (multiples of 2^-20) keep every partial sum exact in fp64, so thresholds can sit
    exactly on a partial sum and test >= against > (the notes' inequality)."""
    r = np.random.default_rng(seed)
    L = int(r.integers(1, 9))
    v = r.integers(1, 2000, size=L).astype(np.float64)
    if seed % 3 == 0:
        v = np.round(v / 500) * 500 + 1          # ties
    v = v * 2.0 ** -20
    srt = np.sort(v)
    taus = [0.0, 1e-9, float(srt[0]), float(srt[: max(1, L // 2)].sum()),
            float(srt[: max(1, L // 2)].sum()) + 2.0 ** -21, float(v.sum()), float(v.sum()) * 2]
    for tau in taus:
        assert oracle.budget(v, tau)[0] == brute_budget(v, tau), (L, tau)


@pytest.mark.parametrize("seed", range(5))
def test_budget_coverage_invariant_and_monotone(seed):
    r = np.random.default_rng(seed)
    L = 2000
    v = r.gamma(0.5, size=L)
    v /= v.sum()
    srt = [Fraction(x) for x in np.sort(v)]
    prev = 0
    for tau in np.linspace(0, 0.98, 25):
        k, Lp = oracle.budget(v, tau)
        assert k + Lp == L and k >= prev
        prev = k
        ft = Fraction(float(tau))
        assert sum(srt[:k], Fraction(0)) >= ft                     # covers tau
        if k > 0:
            assert sum(srt[: k - 1], Fraction(0)) < ft             # and is minimal
    assert oracle.budget(v, 0.0) == (0, L)
    assert oracle.budget(v, 2.0) == (L, 0)


# -- selection ------------------------------------------------------------------------------------

def brute_select(scores, Lp):
    """Max-sum subset of size L'; among equal sums the lexicographically smallest index tuple."""
    best = None
    for c in itertools.combinations(range(len(scores)), Lp):
        key = (-sum(scores[i] for i in c), c)
        if best is None or key < best:
            best = key
    return list(best[1])


@pytest.mark.parametrize("seed", range(10))
def test_select_exhaustive_with_ties(seed):
    r = np.random.default_rng(seed)
    L = int(r.integers(2, 11))
    s = r.integers(0, 4, size=(3, L)).astype(np.float64)        # many exact ties
    for Lp in range(L + 1):
        idx = oracle.select(s, Lp)
        for h in range(3):
            assert idx[h].tolist() == brute_select(s[h].tolist(), Lp)


def test_select_nested_and_ascending():
    s = rnd((5, 300), 7) ** 2
    prev = [set() for _ in range(5)]
    for Lp in range(0, 301, 17):
        idx = oracle.select(s, Lp)
        for h in range(5):
            assert (np.diff(idx[h]) > 0).all()
            assert prev[h] <= set(idx[h].tolist())
            prev[h] = set(idx[h].tolist())


def test_select_zero_keys_keeps_the_prefix():
    """K = 0 makes tokens 0..L-q exactly tied at the top and later tokens strictly smaller, so the
    lower-index tie-break keeps exactly the first L' tokens."""
    L, q = 120, 16
    s = oracle.head_scores(rnd((L, 2, 8), 1), np.zeros((L, 2, 8)), q)
    for Lp in (1, 50, L - q + 1, L - 3, L):
        idx = oracle.select(s, Lp)
        assert (idx == np.arange(Lp)[None, :]).all()


# -- attention ------------------------------------------------------------------------------------

def sdpa_causal(q, k, v):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)[0, 0].numpy()


@pytest.mark.parametrize("seed", range(3))
def test_dense_attention_matches_library(seed):
    L, Hq, Hkv, d = 70, 4, 2, 16
    Q, K, V = rnd((L, Hq, d), seed, 1.5), rnd((L, Hkv, d), seed + 1, 1.5), rnd((L, Hkv, d), seed + 2)
    for h in range(Hq):
        np.testing.assert_allclose(oracle.dense_attention_rows(Q, K, V, h),
                                   sdpa_causal(Q[:, h], K[:, h // 2], V[:, h // 2]), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("seed", range(3))
def test_compressed_attention_mask_by_position(seed):
    """With ascending, unique positions, masking by original position equals the causal mask in the
    compressed index (checked against the library's causal attention)."""
    r = np.random.default_rng(seed)
    n, d = 60, 8
    pos = np.sort(r.choice(500, n, replace=False))
    q, k, v = rnd((n, d), seed), rnd((n, d), seed + 1), rnd((n, d), seed + 2)
    np.testing.assert_allclose(oracle.attention_rows(q, k, v, pos), sdpa_causal(q, k, v),
                               rtol=1e-12, atol=1e-13)
    # a row subset is the same rows of the full result
    rows = [0, 5, 59]
    np.testing.assert_allclose(oracle.attention_rows(q, k, v, pos, rows),
                               oracle.attention_rows(q, k, v, pos)[rows], rtol=1e-14)


def test_attention_closed_forms():
    n, d = 50, 8
    pos = np.arange(n) * 3
    v = rnd((n, d), 2)
    # zero keys: uniform weights over the visible prefix
    out = oracle.attention_rows(rnd((n, d), 1), np.zeros((n, d)), v, pos)
    want = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    np.testing.assert_allclose(out, want, rtol=1e-13)
    # constant values: the output is that constant
    c = np.tile(rnd((1, d), 5), (n, 1))
    np.testing.assert_allclose(oracle.attention_rows(rnd((n, d), 3), rnd((n, d), 4), c, pos), c,
                               rtol=1e-13)
    # row 0 sees only itself: exactly V[0]
    assert (oracle.attention_rows(rnd((n, d), 6), rnd((n, d), 7), v, pos)[0] == v[0]).all()


# -- decompress / residual / whole layer ----------------------------------------------------------

def test_decompress_compress_roundtrip_and_zero_rows():
    L, Hq, d = 40, 3, 4
    M = rnd((L, Hq, d), 1)
    idx = oracle.select(rnd((Hq, L), 2) ** 2, 17)
    Mh = np.stack([M[idx[h], h] for h in range(Hq)])
    O = oracle.decompress(Mh, idx, L)
    for h in range(Hq):
        keep = np.zeros(L, bool)
        keep[idx[h]] = True
        assert (O[keep, h] == M[keep, h]).all()
        assert (O[~keep, h] == 0).all() and not np.signbit(O[~keep, h]).any()
    X = rnd((L, Hq, d), 3)
    Y = oracle.residual(X, O)
    for h in range(Hq):
        un = np.setdiff1d(np.arange(L), idx[h])
        assert (Y[un, h] == X[un, h]).all()


@pytest.mark.parametrize("seed", range(2))
def test_tau_zero_layer_is_dense_attention_plus_residual(seed):
    L, Hq, Hkv, d, q = 64, 4, 2, 8, 8
    Q, K, V, X = (rnd((L, Hq, d), seed), rnd((L, Hkv, d), seed + 1), rnd((L, Hkv, d), seed + 2),
                  rnd((L, Hq, d), seed + 3))
    out = oracle.layer(Q, K, V, X, 0.0, q)
    assert out["Lp"] == L
    np.testing.assert_allclose(out["Y"], oracle.dense_layer(Q, K, V, X), rtol=1e-13, atol=1e-13)
    for h in range(Hq):
        np.testing.assert_allclose(out["Y"][:, h] - X[:, h],
                                   sdpa_causal(Q[:, h], K[:, h // 2], V[:, h // 2]), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("seed", range(2))
def test_sparse_layer_matches_library_attention_on_the_full_tensors(seed):
    """A layer that really drops tokens, checked without compressing anything: for each query head,
    the library's attention over the full-length tensors under the boolean mask "key kept by this
    head and not after the query", with the library's own grouped-query head mapping (query heads
    share a K/V head in consecutive groups), gives Y - X at the kept tokens; dropped tokens keep X
    exactly.  This pins the gather (rows and K/V head), the compressed attention and the scatter
    together, at per-head selections that differ and leave gaps."""
    L, Hq, Hkv, d, q = 96, 6, 2, 16, 8
    r = np.random.default_rng(40 + seed)
    Q, K, V, X = (r.standard_normal(s) for s in ((L, Hq, d), (L, Hkv, d), (L, Hkv, d), (L, Hq, d)))
    K[r.choice(L, 12, replace=False)] *= 4.0          # uneven scores, so the heads keep different sets
    out = oracle.layer(Q, K, V, X, 0.3, q)
    Lp, idx = out["Lp"], out["idx"]
    assert 0 < Lp < L - 10
    assert len({tuple(idx[h]) for h in range(Hq)}) > 1
    kept = np.zeros((Hq, L), dtype=bool)
    for h in range(Hq):
        kept[h, idx[h]] = True
    mask = kept[:, None, :] & np.tril(np.ones((L, L), dtype=bool))[None]
    mask |= np.eye(L, dtype=bool)[None]                # rows of dropped queries: any finite output
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
    want = torch.nn.functional.scaled_dot_product_attention(
        t(Q), t(K), t(V), attn_mask=torch.from_numpy(mask)[None], enable_gqa=True)[0].numpy()
    for h in range(Hq):
        np.testing.assert_allclose(out["Y"][idx[h], h] - X[idx[h], h], want[h, idx[h]], rtol=1e-11, atol=1e-12)
        drop = ~kept[h]
        assert (out["Y"][drop, h] == X[drop, h]).all()


def test_tau_near_one_drops_everything_but_coverage():
    L, d = 30, 8
    Q, K, V, X = rnd((L, 2, d), 1), rnd((L, 2, d), 2), rnd((L, 2, d), 3), rnd((L, 2, d), 4)
    out = oracle.layer(Q, K, V, X, 1.5, 4)
    assert out["Lp"] == 0 and (out["Y"] == X).all()


# -- storage rounding and load-time layer choice --------------------------------------------------

def test_round_to_storage_matches_library_conversion():
    r = np.random.default_rng(0)
    a = torch.from_numpy(r.standard_normal(20000).astype(np.float32)).to(torch.bfloat16)
    b = torch.from_numpy(r.standard_normal(20000).astype(np.float32) * 1e-3).to(torch.bfloat16)
    exact = a.double().numpy() + b.double().numpy()
    want = (a.float() + b.float()).to(torch.bfloat16).double().numpy()
    assert (oracle.round_to_storage(exact, "bf16") == want).all()
    x = r.standard_normal(1000) * 7
    assert (oracle.round_to_storage(x, "f32") == x.astype(np.float32).astype(np.float64)).all()
    halfway = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8])     # ties go to even
    assert oracle.round_to_storage(halfway, "bf16").tolist() == [1.0, 1.0 + 4 * 2.0 ** -8]


def test_budget_fixed_ratio_hand_cases():
    """Reading R10 on values worked out by hand from the exact float32 ratios."""
    f = oracle.budget_fixed_ratio
    assert f(4096, 0.0) == (0, 4096) and f(4096, 1.0) == (4096, 0)
    assert f(4096, 0.5) == (2048, 2048)
    assert f(5, 0.5) == (3, 2)                        # 2.5 prunes 3: halves round up
    assert f(10, 0.7) == (7, 3)                       # float32(0.7) = 0.69999998..: 6.9999998 -> 7
    assert f(10, 0.3) == (3, 7)                       # float32(0.3) = 0.30000001..
    assert f(4096, 0.3) == (1229, 2867)               # 1228.80005
    assert f(131072, 0.3) == (39322, 91750)           # 39321.60156
    assert f(2 ** 23, 2.0 ** -24) == (1, 2 ** 23 - 1)  # exactly 1/2: rounds up
    assert f(2 ** 23 - 1, 2.0 ** -24) == (0, 2 ** 23 - 1)
    assert f(1000, 1e-30) == (0, 1000)                # a denormal-range ratio prunes nothing


@pytest.mark.parametrize("seed", range(3))
def test_budget_fixed_ratio_is_the_nearest_count(seed):
    """Brute force: k is the count in [0, L] nearest to s*L (larger one on a tie), L' = L - k, and
    k is monotone in s."""
    rng = np.random.default_rng(seed)
    for _ in range(200):
        L = int(rng.integers(1, 3000))
        sp = float(np.float32(rng.random()))
        k, Lp = oracle.budget_fixed_ratio(L, sp)
        x = Fraction(sp) * L
        best = min(range(L + 1), key=lambda j: (abs(j - x), -j))
        assert (k, Lp) == (best, L - best), (L, sp)
    L = 777
    ks = [oracle.budget_fixed_ratio(L, float(np.float32(v)))[0] for v in np.linspace(0, 1, 301)]
    assert all(a <= b for a, b in zip(ks, ks[1:])) and ks[0] == 0 and ks[-1] == L


def test_fixed_ratio_swaps_only_the_budget():
    """The fixed-ratio layer with s = k/L of a coverage-budget layer reproduces that layer."""
    rng = np.random.default_rng(11)
    L, Hq, Hkv, d, q = 40, 4, 2, 16, 4
    Q, K, V, X = (rng.standard_normal(sh) for sh in ((L, Hq, d), (L, Hkv, d), (L, Hkv, d), (L, Hq, d)))
    a = oracle.layer(Q, K, V, X, tau=0.2, q=q)
    assert 0 < a["k"] < L
    b = oracle.layer(Q, K, V, X, tau=0.0, q=q, sparsity=a["k"] / L)
    assert (b["k"], b["Lp"]) == (a["k"], a["Lp"]) and (b["idx"] == a["idx"]).all()
    assert np.array_equal(b["Y"], a["Y"])


def test_varlen_batch_keeps_samples_apart():
    """Samples of a batch never see each other: the first token of every sample attends to itself
    only (its output is its own value row, plus the residual), changing one sample leaves the
    others bit-identical, and identical samples give identical outputs."""
    rng = np.random.default_rng(21)
    lens = [30, 1, 17, 30]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T, Hq, Hkv, d, q = cu[-1], 4, 2, 16, 1
    Q, K, V, X = (rng.standard_normal(sh) for sh in ((T, Hq, d), (T, Hkv, d), (T, Hkv, d), (T, Hq, d)))
    # sample 3 repeats sample 0
    Q[cu[3]:], K[cu[3]:], V[cu[3]:], X[cu[3]:] = Q[:30], K[:30], V[:30], X[:30]
    outs, Y = oracle.layer_varlen(Q, K, V, X, cu, tau=0.0, q=q)
    assert [o["Lp"] for o in outs] == lens                # tau = 0 keeps everything
    for b in range(4):
        assert np.allclose(Y[cu[b]], X[cu[b]] + V[cu[b]][np.arange(Hq) // (Hq // Hkv)], rtol=0, atol=1e-15)
    assert np.array_equal(Y[cu[3]:], Y[:30])
    K2 = K.copy()
    K2[cu[2]:cu[3]] += 1.0
    _, Y2 = oracle.layer_varlen(Q, K2, V, X, cu, tau=0.0, q=q)
    keep = np.r_[0:cu[2], cu[3]:T]
    assert np.array_equal(Y2[keep], Y[keep]) and not np.array_equal(Y2[cu[2]:cu[3]], Y[cu[2]:cu[3]])


# -- block sparsity in the compressed space (reading R11) -------------------------------------------

def _bf16_values(shape, seed):
    return oracle.round_to_storage(np.random.default_rng(seed).standard_normal(shape), "bf16")


def test_block_pool_is_the_block_mean():
    """bf16 values sum exactly in float64, so the pool equals the library's reshaped mean rounded
    to float32; the last, partial block averages only its own rows."""
    X = _bf16_values((300, 16), 3)
    got = oracle.block_pool(X, 256)
    want = X[:256].reshape(2, 128, 16).mean(axis=1).astype(np.float32)
    assert np.array_equal(got, want)
    got = oracle.block_pool(X, 300)
    assert got.shape == (3, 16) and np.array_equal(got[2], X[256:300].mean(axis=0).astype(np.float32))
    assert oracle.block_pool(X, 0).shape == (0, 16)


def test_block_select_hand_case():
    """Weights 0.6 / 0.1 / 0.3 on key blocks 0 / 1 / 2 for query block 2 (kbar chosen so that the
    scaled logits are ln 6, ln 1, ln 3)."""
    d = 4
    kbar = np.zeros((3, d))
    kbar[:, 0] = 2 * np.log([6.0, 1.0, 3.0])          # <qbar, kbar> / sqrt(4) = ln w
    qbar = np.zeros((3, d))
    qbar[:, 0] = 1.0
    keep = oracle.block_select(qbar, kbar, gamma=0.5)
    assert [k.tolist() for k in keep] == [[0], [0, 1], [0, 2]]   # block 2: 0 reaches 0.6, 2 forced
    keep = oracle.block_select(qbar, kbar, gamma=0.65)
    assert keep[2].tolist() == [0, 2]                 # 0.6 + 0.3
    keep = oracle.block_select(qbar, kbar, gamma=0.95)
    assert keep[2].tolist() == [0, 1, 2]
    keep = oracle.block_select(qbar, kbar, gamma=1.0)
    assert keep[2].tolist() == [0, 1, 2]


@pytest.mark.parametrize("seed", range(3))
def test_block_select_is_the_fewest_heaviest_blocks(seed):
    """Brute force over every subset of candidate blocks: the non-forced part of the kept set has the
    minimum size of any subset reaching gamma and the largest weight among subsets of that size."""
    rng = np.random.default_rng(seed)
    nb, d = 9, 8
    qbar, kbar = rng.standard_normal((nb, d)) * 2, rng.standard_normal((nb, d)) * 2
    for gamma in (0.3, 0.7, 0.9):
        keep = oracle.block_select(qbar, kbar, gamma)
        for I in range(nb):
            z = kbar[: I + 1] @ qbar[I] / np.sqrt(d)
            a = np.exp(z - z.max())
            a /= a.sum()
            best_n, best_w = None, None
            for n in range(1, I + 2):
                w = max(sum(a[list(c)]) for c in itertools.combinations(range(I + 1), n))
                if w >= gamma:
                    best_n, best_w = n, w
                    break
            forced = {0, I}
            k = set(keep[I].tolist())
            assert forced <= k
            # the greedy prefix: best_n heaviest blocks (ties impossible with continuous draws)
            top = set(np.argsort(-a, kind="stable")[:best_n].tolist())
            assert k == top | forced, (gamma, I)
            assert abs(sum(a[list(top)]) - best_w) < 1e-12


def test_block_sparse_attention_matches_masked_library_attention():
    """Kept-block attention equals the library's attention under the explicit boolean mask
    (causal and inside a kept block), small blocks for many of them."""
    rng = np.random.default_rng(9)
    n, d, B = 100, 16, 16
    Qh, Kh, Vh = (rng.standard_normal((n, d)) for _ in range(3))
    nb = -(-n // B)
    keep = [np.array(sorted({0, I} | set(rng.choice(I + 1, size=min(I + 1, 2), replace=False).tolist())))
            for I in range(nb)]
    M = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for J in keep[i // B]:
            M[i, J * B: min((J + 1) * B, n)] = True
    M &= np.tril(np.ones((n, n), dtype=bool))
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Qh)[None], torch.from_numpy(Kh)[None], torch.from_numpy(Vh)[None],
        attn_mask=torch.from_numpy(M)[None]).numpy()[0]
    got = oracle.block_sparse_attention_rows(Qh, Kh, Vh, keep, B=B)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12)
    full = [np.arange(I + 1) for I in range(nb)]
    assert np.allclose(oracle.block_sparse_attention_rows(Qh, Kh, Vh, full, B=B),
                       oracle.attention_rows(Qh, Kh, Vh, np.arange(n)), rtol=1e-13, atol=1e-13)


def test_block_sparse_layer_with_full_coverage_is_the_layer():
    rng = np.random.default_rng(12)
    L, Hq, Hkv, d, q = 700, 2, 1, 16, 4
    Q, K, V, X = (rng.standard_normal(sh) for sh in ((L, Hq, d), (L, Hkv, d), (L, Hkv, d), (L, Hq, d)))
    a = oracle.layer(Q, K, V, X, tau=0.1, q=q)
    b = oracle.block_sparse_layer(Q, K, V, X, tau=0.1, q=q, gamma=1.0)
    assert all(len(k) == I + 1 for kh in b["keep"] for I, k in enumerate(kh))
    assert np.allclose(b["Y"], a["Y"], rtol=1e-13, atol=1e-13)
    c = oracle.block_sparse_layer(Q, K, V, X, tau=0.1, q=q, gamma=0.2)
    assert sum(len(k) for kh in c["keep"] for k in kh) < sum(len(k) for kh in b["keep"] for k in kh)


def test_sparse_layers_and_drift():
    R = [0.4, 0.3, 0.5, 0.1, 0.2, 0.05, 0.45, 0.35]
    assert oracle.sparse_layers(R) == [2, 4, 5, 6]
    assert oracle.sparse_layers([0.2] * 4) == [1, 2]                 # ties by layer id
    assert oracle.sparse_layers(sorted(R, reverse=True)) == [5, 6, 7, 8]
    h = rnd((100, 16), 1)
    assert abs(oracle.representation_drift(h, h * 1.25, eps=0.0) - 0.25) < 1e-14
    assert oracle.representation_drift(h, h) == 0.0


# -- planted mistakes must trip a pin ---------------------------------------------------------------

def _mut_no_causal(Q, K, q):
    L, Hq, d = Q.shape
    s = np.zeros((Hq, L))
    for h in range(Hq):
        z = Q[L - q:, h] @ K[:, h * K.shape[1] // Hq].T / np.sqrt(d)
        e = np.exp(z - z.max(1, keepdims=True))
        s[h] = (e / e.sum(1, keepdims=True)).sum(0)
    return s


def _mut_budget_strict(s_l, tau):
    C = np.concatenate([[0.0], np.cumsum(np.sort(s_l))])
    hit = np.nonzero(C > tau)[0]
    k = int(hit[0]) if len(hit) else len(s_l)
    return k, len(s_l) - k


def _mut_select_high_index_ties(s_h, Lp):
    L = s_h.shape[1]
    return np.stack([np.sort(np.lexsort((-np.arange(L), -s_h[h]))[:Lp]) for h in range(s_h.shape[0])])


def _mut_attention_no_scale(Qh, Kh, Vh, pos, rows=None):
    n, d = Qh.shape
    rows = np.arange(n) if rows is None else np.asarray(rows)
    z = Qh[rows] @ Kh.T
    z = np.where(pos[None, :] <= pos[rows][:, None], z, -np.inf)
    e = np.exp(z - z.max(1, keepdims=True))
    return e / e.sum(1, keepdims=True) @ Vh


def _mut_gather_kv_interleaved(Q, K, V, idx):
    Hq, Hkv = Q.shape[1], K.shape[1]
    Qh = np.stack([Q[idx[h], h] for h in range(Hq)])
    Kh = np.stack([K[idx[h], h % Hkv] for h in range(Hq)])
    Vh = np.stack([V[idx[h], h % Hkv] for h in range(Hq)])
    return Qh, Kh, Vh


def _mut_gather_kv_prefix(Q, K, V, idx):
    Hq, Hkv, Lp = Q.shape[1], K.shape[1], idx.shape[1]
    G = Hq // Hkv
    Qh = np.stack([Q[idx[h], h] for h in range(Hq)])
    Kh = np.stack([K[:Lp, h // G] for h in range(Hq)])
    Vh = np.stack([V[idx[h], h // G] for h in range(Hq)])
    return Qh, Kh, Vh


def _mut_decompress_prefix(Oh, idx, L):
    Hq, Lp, d = Oh.shape
    O = np.zeros((L, Hq, d))
    O[:Lp] = Oh.transpose(1, 0, 2)
    return O


def _mut_ratio_floor(L, sparsity):
    k = math.floor(Fraction(float(np.float32(sparsity))) * L)
    return k, L - k


def _mut_block_no_diagonal(qbar, kbar, gamma):
    nb, d = qbar.shape
    keep = []
    for I in range(nb):
        z = (kbar[: I + 1] @ qbar[I]) / np.sqrt(d)
        a = np.exp(z - z.max())
        a = a / a.sum()
        order = np.lexsort((np.arange(I + 1), -a))
        hit = np.nonzero(np.cumsum(a[order]) >= gamma)[0]
        n = int(hit[0]) + 1 if (gamma < 1 and len(hit)) else I + 1
        keep.append(np.array(sorted(set(order[:n].tolist()) | {0}), dtype=np.int64))
    return keep


def _mut_layer_score_unnormalised(s_h):
    return s_h.sum(axis=0)


def _mut_layer_score_max(s_h):
    S = s_h.max(axis=0)
    return S / S.sum()


def _mut_residual_sign(X, O):
    return X - O


def _mut_pool_full_block(Xh, Lp, B=oracle.BLOCK):
    nb = -(-Lp // B)
    out = np.zeros((nb, Xh.shape[1]))
    for b in range(nb):
        out[b] = (Xh[b * B: min(Lp, (b + 1) * B)].sum(axis=0) / B).astype(np.float32)
    return out


def _mut_drift_squared(h_cur, h_next, eps=1e-6):
    num = np.linalg.norm(h_next - h_cur, axis=1) ** 2
    den = np.linalg.norm(h_cur, axis=1) ** 2 + eps
    return float(np.mean(num / den))


def _mut_sparse_most_drifting(R, delta=0.5):
    N = len(R)
    order = sorted(range(N), key=lambda i: (-R[i], i))
    return sorted(i + 1 for i in order[: int(delta * N)])


@pytest.mark.parametrize("name,mutant,pin", [
    ("layer_score", _mut_layer_score_unnormalised, test_layer_score_normalised_and_equal_heads),
    ("layer_score", _mut_layer_score_max, test_layer_score_hand_case),
    ("residual", _mut_residual_sign, lambda: test_tau_zero_layer_is_dense_attention_plus_residual(0)),
    ("block_pool", _mut_pool_full_block, test_block_pool_is_the_block_mean),
    ("representation_drift", _mut_drift_squared, test_sparse_layers_and_drift),
    ("sparse_layers", _mut_sparse_most_drifting, test_sparse_layers_and_drift),
    ("budget_fixed_ratio", _mut_ratio_floor, test_budget_fixed_ratio_hand_cases),
    ("block_select", _mut_block_no_diagonal, test_block_select_hand_case),
    ("head_scores", _mut_no_causal, lambda: test_score_zero_keys_closed_form(64, 16)),
    ("budget", _mut_budget_strict, lambda: test_budget_exhaustive_exact(0)),
    ("select", _mut_select_high_index_ties, test_select_zero_keys_keeps_the_prefix),
    ("attention_rows", _mut_attention_no_scale, lambda: test_dense_attention_matches_library(0)),
    ("gather", _mut_gather_kv_interleaved,
     lambda: test_sparse_layer_matches_library_attention_on_the_full_tensors(0)),
    ("gather", _mut_gather_kv_prefix,
     lambda: test_sparse_layer_matches_library_attention_on_the_full_tensors(0)),
    ("decompress", _mut_decompress_prefix,
     lambda: test_sparse_layer_matches_library_attention_on_the_full_tensors(0)),
])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pin):
    monkeypatch.setattr(oracle, name, mutant)
    monkeypatch.setattr(oracle.tsa_oracle, name, mutant)
    with pytest.raises(AssertionError):
        pin()
