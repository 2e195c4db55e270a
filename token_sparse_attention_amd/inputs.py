"""Seeded synthetic inputs for the Token Sparse Attention prefill layer.

This module only draws random tensors; it holds none of the layer's arithmetic.  Both the HIP path
and the CPU oracle are fed from it.

Recipe (all draws from ``numpy.random.Generator(PCG64(seed))``, in this order):

1. Q [L][Hq][d], K [L][Hkv][d], V [L][Hkv][d] and (first layer only) X [L][Hq][d]: iid N(0, 1) fp32.
2. u [Hkv][d]: one N(0, I) direction per KV head, normalised to unit length.
3. Salient positions: n = round(salient_frac * L) per KV head.  A shared part of
   round(shared_frac * n) positions is drawn once, uniformly without replacement from [0, L); each KV
   head then draws its own n - n_shared positions from the complement of the shared part.  In a
   chain, every later layer keeps a random round(layer_overlap * n) of each head's previous set and
   draws the rest from the positions outside that previous set.
4. Keys at a head's salient positions get K[t, g] += 3 u_g; the last q query rows of every query
   head in group g get Q[p, h] += 2 u_g; with ``sink`` > 0 the first ``sink`` keys get K += 2 u_g.
5. Storage rounding: bf16 workloads round every tensor to bfloat16 (round to nearest even, via
   torch); fp32 workloads keep the fp32 draws.
6. Varlen batches: sample b is an independent draw of the same recipe at its own length, seeded by
   the b-th child of SeedSequence(seed + 2000); samples are packed along the token axis.
"""

import numpy as np
import torch

from .configs import Workload, scaled


def _salient_sets(rng, cfg: Workload, prev=None):
    L, n = cfg.L, int(round(cfg.salient_frac * cfg.L))
    everything = np.arange(L)
    sets = []
    if prev is None:
        n_sh = int(round(cfg.shared_frac * n))
        shared = rng.choice(L, n_sh, replace=False)
        rest = np.setdiff1d(everything, shared, assume_unique=True)
        for _ in range(cfg.Hkv):
            own = rng.choice(rest, n - n_sh, replace=False)
            sets.append(np.sort(np.concatenate([shared, own])))
    else:
        n_keep = int(round(cfg.layer_overlap * n))
        for g in range(cfg.Hkv):
            keep = rng.choice(prev[g], n_keep, replace=False)
            outside = np.setdiff1d(everything, prev[g], assume_unique=True)
            new = rng.choice(outside, n - n_keep, replace=False)
            sets.append(np.sort(np.concatenate([keep, new])))
    return sets


def _store(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def make_layer(cfg: Workload, seed=None, with_x=True, prev_sets=None):
    """Draw one layer's inputs.  Returns a dict of CPU tensors in storage dtype plus the salient sets."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    L, Hq, Hkv, d, q = cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.q
    Q = rng.standard_normal((L, Hq, d), dtype=np.float32)
    K = rng.standard_normal((L, Hkv, d), dtype=np.float32)
    V = rng.standard_normal((L, Hkv, d), dtype=np.float32)
    X = rng.standard_normal((L, Hq, d), dtype=np.float32) if with_x else None
    u = rng.standard_normal((Hkv, d))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    u = u.astype(np.float32)
    sets = _salient_sets(rng, cfg, prev_sets)
    G = Hq // Hkv
    for g in range(Hkv):
        K[sets[g], g, :] += 3.0 * u[g]
        if cfg.sink:
            K[: cfg.sink, g, :] += 2.0 * u[g]
        Q[L - q:, g * G:(g + 1) * G, :] += 2.0 * u[g]
    out = dict(Q=_store(Q, cfg.dtype), K=_store(K, cfg.dtype), V=_store(V, cfg.dtype), sets=sets)
    del Q, K, V
    if X is not None:
        out["X"] = _store(X, cfg.dtype)
    return out


def chain_seeds(cfg: Workload):
    """One independent seed per layer of a chain workload."""
    return [int(s.generate_state(1)[0]) for s in np.random.SeedSequence(cfg.seed).spawn(cfg.layers)]


def chain_drift_values(cfg: Workload):
    """Seeded per-layer drift values R_1..R_N for a chain: U(0.05, 0.5) draws sorted descending, so the
    deepest layers are the most stable ones."""
    rng = np.random.Generator(np.random.PCG64(cfg.seed + 1000))
    return np.sort(rng.uniform(0.05, 0.5, cfg.layers))[::-1].copy()


def iter_chain(cfg: Workload):
    """Yield (layer_id, inputs) for every layer of a chain; X is drawn for layer 1 only."""
    prev = None
    for i, s in enumerate(chain_seeds(cfg)):
        lay = make_layer(cfg, seed=s, with_x=(i == 0), prev_sets=prev)
        prev = lay["sets"]
        yield i + 1, lay


def make_batch(cfg: Workload, lengths, seed=None):
    """A varlen batch: one independent draw of `cfg`'s recipe per sample length, packed along the
    token axis.  Returns the packed CPU tensors, cu_seqlens (B+1 offsets) and the per-sample draws."""
    ss = np.random.SeedSequence(cfg.seed + 2000 if seed is None else seed).spawn(len(lengths))
    parts = [make_layer(scaled(cfg, int(L)), seed=int(s.generate_state(1)[0])) for L, s in zip(lengths, ss)]
    cu = np.concatenate([[0], np.cumsum([int(L) for L in lengths])]).astype(np.int64)
    out = {n: torch.cat([p[n] for p in parts], dim=0) for n in ("Q", "K", "V", "X")}
    out["cu_seqlens"] = cu
    out["parts"] = parts
    return out
