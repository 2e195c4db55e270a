"""Budget and selection on both sides of the one-workgroup limit (rows of at most 32768 scores are
budgeted and selected by a single workgroup per row, longer rows by the multi-block radix select).

Scores are synthetic float32 rows, uploaded as they are, in four shapes: a narrow range (every key
shares its leading bits), exact ties on a coarse grid, a wide range with exact zeros, and one
repeated value.  Checks are exact:
- k equals the smallest count of smallest float32 values whose exact sum reaches tau (integer
  arithmetic on the float32 values), k + L' = L;
- the selection is the oracle's top-L' of the same float32 scores (score descending, index
  ascending), in ascending order; idx past L' is left as it was; inv is its inverse (-1 elsewhere).
"""

import numpy as np
import pytest
import torch

import oracle
from token_sparse_attention_amd import binding

pytestmark = pytest.mark.gpu

LENGTHS = [1, 5, 1023, 1025, 4097, 20001, 32768, 32769, 65537, 100003]


def scores(kind, Hq, L, seed):
    r = np.random.default_rng(seed)
    if kind == "narrow":
        s = 1.0 + r.random((Hq, L)) * 1e-3
    elif kind == "ties":
        s = r.integers(0, 6, size=(Hq, L)) * 0.125
    elif kind == "wide":
        s = np.exp(r.normal(0.0, 8.0, size=(Hq, L)))
        s[r.random((Hq, L)) < 0.05] = 0.0
    else:
        s = np.full((Hq, L), 0.375)
    return s.astype(np.float32)


def exact_budget(vals32, tau32):
    """Every float32 (and tau) times 2^149 is an integer: the budget in exact arithmetic."""
    v = np.sort(vals32.astype(np.float64))
    target = int(np.float64(tau32) * 2.0 ** 149)
    if target <= 0:
        return 0
    acc = 0
    for j, x in enumerate(v):
        acc += int(x * 2.0 ** 149)
        if acc >= target:
            return j + 1
    return len(v)


@pytest.mark.parametrize("L", LENGTHS)
@pytest.mark.parametrize("kind", ["narrow", "ties", "wide", "equal"])
def test_select_exact(gpu, L, kind):
    Hq = 3                                # odd: rows of odd L start off 16-byte boundaries
    s = scores(kind, Hq, L, seed=L % 997)
    s_h = torch.from_numpy(s).to(gpu)
    shape = binding.shape(L, Hq, 1, 128, 1, 0.01, "bf16")
    ws = binding.workspace(binding.stage_workspace_bytes(shape), gpu)
    for Lp in sorted({0, 1, L // 3, L // 2, L - 1, L} - {-1}):
        if Lp < 0 or Lp > L:
            continue
        idx = torch.full((Hq, L), -7, dtype=torch.int32, device=gpu)
        inv = torch.full((Hq, L), -7, dtype=torch.int32, device=gpu)
        binding.select(shape, s_h, torch.tensor([Lp], dtype=torch.int32, device=gpu), idx, inv, ws)
        got, gi = idx.cpu().numpy(), inv.cpu().numpy()
        want = oracle.select(s.astype(np.float64), Lp)
        assert (got[:, :Lp] == want).all(), (kind, L, Lp)
        assert (got[:, Lp:] == -7).all(), (kind, L, Lp)
        for h in range(Hq):
            w = np.full(L, -1)
            w[want[h]] = np.arange(Lp)
            assert (gi[h] == w).all(), (kind, L, Lp, h)


@pytest.mark.parametrize("L", LENGTHS)
@pytest.mark.parametrize("kind", ["narrow", "ties", "wide", "equal"])
def test_budget_exact(gpu, L, kind):
    s = scores(kind, 1, L, seed=L % 991 + 1)[0].astype(np.float64)
    tot = s.sum()
    s_l = (s / tot if tot > 0 else s).astype(np.float32)
    d_sl = torch.from_numpy(s_l).to(gpu)
    for tau in (0.0, 0.005, 0.3, 0.72, 0.9999):
        t32 = float(np.float32(tau))
        shape = binding.shape(L, 1, 1, 128, 1, tau, "bf16")
        ws = binding.workspace(binding.stage_workspace_bytes(shape), gpu)
        kl = torch.full((2,), -5, dtype=torch.int32, device=gpu)
        binding.budget(shape, d_sl, kl[0:1], kl[1:2], ws)
        k, Lp = kl.tolist()
        assert k + Lp == L
        assert k == exact_budget(s_l, t32), (kind, L, tau, k)


def cluster_row(L, n, seed):
    """A row whose middle ranks are a cluster of n keys sharing their leading bits, with exact ties
    (1 + j * 2^-20 for j in 0..7), between n_hi large keys above and small keys below: the
    one-workgroup select ranks the cluster directly once at most 64 keys share the prefix, and runs
    another digit pass first for 65."""
    r = np.random.default_rng(seed)
    s = r.random(L) * 0.25                                   # small keys
    pos = r.permutation(L)
    n_hi = L // 2 - n // 2
    s[pos[:n_hi]] = 2.0 + r.random(n_hi) * 2.0               # large keys
    s[pos[n_hi:n_hi + n]] = 1.0 + r.integers(0, 8, size=n) * 2.0 ** -20
    return s.astype(np.float32), n_hi


@pytest.mark.parametrize("L", [4097, 20001, 32768])
@pytest.mark.parametrize("n", [2, 63, 64, 65, 200])
def test_select_cluster(gpu, L, n):
    s, n_hi = cluster_row(L, n, seed=L + n)
    Hq = 1
    s_h = torch.from_numpy(s[None, :].copy()).to(gpu)
    shape = binding.shape(L, Hq, 1, 128, 1, 0.01, "bf16")
    ws = binding.workspace(binding.stage_workspace_bytes(shape), gpu)
    # L' inside the cluster: its first, middle and last keys, and the ranks just outside it
    for Lp in sorted({n_hi, n_hi + 1, n_hi + n // 2, n_hi + n - 1, n_hi + n, n_hi + n + 1}):
        idx = torch.full((Hq, L), -7, dtype=torch.int32, device=gpu)
        inv = torch.full((Hq, L), -7, dtype=torch.int32, device=gpu)
        binding.select(shape, s_h, torch.tensor([Lp], dtype=torch.int32, device=gpu), idx, inv, ws)
        got, gi = idx.cpu().numpy(), inv.cpu().numpy()
        want = oracle.select(s[None, :].astype(np.float64), Lp)
        assert (got[:, :Lp] == want).all(), (L, n, Lp)
        w = np.full(L, -1)
        w[want[0]] = np.arange(Lp)
        assert (gi[0] == w).all(), (L, n, Lp)


@pytest.mark.parametrize("L", [4097, 20001, 32768])
@pytest.mark.parametrize("n", [2, 63, 64, 65, 200])
def test_budget_cluster(gpu, L, n):
    # ascending mass: the budget's crossing falls among the cluster when tau lies inside its mass
    s, n_hi = cluster_row(L, n, seed=L + 7 * n)
    tot = s.astype(np.float64).sum()
    s_l = (s.astype(np.float64) / tot).astype(np.float32)
    d_sl = torch.from_numpy(s_l).to(gpu)
    v = np.sort(s_l.astype(np.float64))
    below = v[: L - n_hi - n].sum()                          # the small keys
    cl = v[L - n_hi - n: L - n_hi]
    for frac in (0.0, 0.3, 0.5, 0.99):
        tau = below + frac * cl.sum() + (1e-9 if frac == 0.0 else 0.0)
        t32 = float(np.float32(tau))
        shape = binding.shape(L, 1, 1, 128, 1, t32, "bf16")
        ws = binding.workspace(binding.stage_workspace_bytes(shape), gpu)
        kl = torch.full((2,), -5, dtype=torch.int32, device=gpu)
        binding.budget(shape, d_sl, kl[0:1], kl[1:2], ws)
        k, Lp = kl.tolist()
        assert k + Lp == L
        assert k == exact_budget(s_l, t32), (L, n, frac, k)
