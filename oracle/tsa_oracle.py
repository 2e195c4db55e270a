"""CPU oracle for the Token Sparse Attention prefill layer.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import this module.  It shares no code with the HIP library and imports nothing from
it; the product path never calls it.

Plain, slow and obviously correct: numpy float64 on the stored input values (bf16 or fp32 widened
exactly to fp64), natural index order, library primitives (matmul, sort, cumsum, exp) used as single
steps, no blocking or fusion.  Every function cites the passage it follows.  Page names used below:

* "notes"   -- papernotes.org reading notes on the paper (Chinese): sections "Overall framework",
               "Key design 1" (compress-then-decompress), "Key design 2" (Dynamic Token Coverage),
               "Key design 3" (inter-layer representation drift).
* "blog"    -- bxzpzcl.cn article on the method (Chinese): section 1.1 (algorithm details and the
               pseudo-code of the compress / attend / decompress function), 2.1 (importance scoring
               and budget), 2.2 (drift-based layer choice).
* "summary" -- gist.science structured summary (English): "2. Methodology", parts "Core
               Architecture", "Dynamic Token Coverage", "Sparse Layer Selection".

Readings taken where the pages are silent or disagree (each is also listed in the design notes):

R1  Scoring softmax uses the attention scale 1/sqrt(d) and is causal: recent query at position p
    sees keys t <= p.  The "pool" the notes mention after the column sum is the identity (the blog's
    formula s_h = sum(A, dim=0) has none).
R2  "normalize" in s_l = normalize(sum_h s_h) is division by the total, so s_l sums to 1.
R3  Budget: k = the smallest j in [0, L] whose j smallest s_l values sum to >= tau (the notes'
    inequality); k = L when no j qualifies.  L' = L - k.
R4  Per-head top-L': order by (s_h descending, index ascending), keep L', emit ascending.
R5  GQA: query head h reads KV head floor(h / (Hq / Hkv)); head h is ranked by its own s_h.
R6  Compressed attention is causal by ORIGINAL positions (S_h[j] <= S_h[i]) with scale 1/sqrt(d).
R7  Decompress writes +0.0 into unselected rows; the residual is Y = X + Decompress(O_hat) per head,
    with no output projection.
R11 Block sparsity inside the compressed space (the pages stack a block-sparse kernel after the
    token filter but describe no block rule of their own): blocks of 128 compressed rows; each
    block's Q_hat and K_hat rows are mean-pooled (sum in float64, divide, round once to float32);
    query block I weighs its causal key blocks J <= I by softmax_J(<qbar_I, kbar_J> / sqrt(d)) and
    keeps the fewest heaviest blocks (ties: lower J) whose weight reaches gamma (all when gamma >= 1
    or when no prefix reaches it), plus block 0 and the diagonal block I; attention then sees only
    the kept blocks, causally inside the diagonal block.
R10 Fixed-ratio budget (the ablation baseline): the pruned count k is s*L rounded to the nearest
    integer, halves rounded up, on the exact value of the stored float32 ratio s; L' = L - k.
"""

from fractions import Fraction
import math

import numpy as np


def gqa_group(h, Hq, Hkv):
    """KV head read by query head h (reading R5)."""
    return h // (Hq // Hkv)


# -- Stage 1: Dynamic Token Coverage scoring ----------------------------------------------------

def head_scores(Q, K, q):
    """s_h[h, t] = sum over the last q queries of their causal softmax weight on key t.

    notes, Key design 2: recent queries attend to all keys in a lightweight attention A_hat; the
    column sums give the head-level token score.  blog 2.1: A_hat in R^{q x L} from the last q
    queries, s_h = sum(A_hat, dim=0).  summary, Dynamic Token Coverage: weights summed vertically.
    Readings R1 and R5.

    Q: [L][Hq][d], K: [L][Hkv][d] float64.  Returns s_h: [Hq][L] float64.
    """
    return head_scores_recent(Q[Q.shape[0] - q:], K)


def head_scores_recent(Q_recent, K):
    """head_scores given only the recent query rows Q_recent = Q[L-q:] ([q][Hq][d])."""
    q, Hq, d = Q_recent.shape
    L, Hkv = K.shape[0], K.shape[1]
    s_h = np.zeros((Hq, L))
    pos = np.arange(L)
    recent = np.arange(L - q, L)                      # query positions p = L-q .. L-1
    for h in range(Hq):
        g = gqa_group(h, Hq, Hkv)
        z = (Q_recent[:, h, :] @ K[:, g, :].T) / np.sqrt(d)      # [q][L] logits
        visible = pos[None, :] <= recent[:, None]                # causal
        z = np.where(visible, z, -np.inf)
        m = z.max(axis=1, keepdims=True)
        e = np.where(visible, np.exp(z - m), 0.0)
        a = e / e.sum(axis=1, keepdims=True)                     # row softmax
        s_h[h] = a.sum(axis=0)                                   # column sum
    return s_h


def layer_score(s_h):
    """s_l = normalize(sum_h s_h), normalised to unit total (notes, Key design 2; blog 2.1; R2)."""
    S = s_h.sum(axis=0)
    return S / S.sum()


# -- Stage 2: coverage budget ---------------------------------------------------------------------

def budget(s_l, tau):
    """Smallest k whose k smallest layer scores cover at least tau; returns (k, L' = L - k).

    notes, Key design 2: sort s_l ascending and find the smallest k_sparse with
    sum_{j<=k_sparse} s_l[I[j]] >= tau; keep k_keep = L - k_sparse.  blog 2.1 states the same.
    Reading R3 (k = L when even the full sum stays below tau).
    """
    L = len(s_l)
    v = np.sort(s_l)                                   # ascending
    C = np.concatenate([[0.0], np.cumsum(v)])          # C[j] = sum of the j smallest
    hit = np.nonzero(C >= tau)[0]
    k = int(hit[0]) if len(hit) else L
    return k, L - k


def budget_fixed_ratio(L, sparsity):
    """The ablation's fixed budget: prune the share s of the L tokens, keep L' = (1 - s) L.

    notes, Ablations (dynamic tau = 0.005 against a fixed s = 0.3, tau = 0.010 against s = 0.5) and
    Key design 2 (a fixed keep ratio cut the same way at every length, the thing the coverage budget
    replaces).  Reading R10: k = round(s * L), halves up, in exact rational arithmetic on the stored
    float32 value of s.  Returns (k, L').
    """
    s = Fraction(float(np.float32(sparsity)))
    k = math.floor(s * L + Fraction(1, 2))
    return k, L - k


# -- Stage 3: per-head selection ------------------------------------------------------------------

def select(s_h, Lp):
    """S_h = the L' tokens with the largest s_h of each head, ascending (reading R4).

    notes, Key design 2: each head then takes its own top-k_keep subset S_h.  summary, Dynamic Token
    Coverage, head-wise selection: after the global budget every head selects independently.
    Returns idx [Hq][L'] int64.
    """
    Hq, L = s_h.shape
    t = np.arange(L)
    idx = np.empty((Hq, Lp), dtype=np.int64)
    for h in range(Hq):
        order = np.lexsort((t, -s_h[h]))               # score descending, then index ascending
        idx[h] = np.sort(order[:Lp])
    return idx


# -- Stage 4: compress and attend -----------------------------------------------------------------

def gather(Q, K, V, idx):
    """Q_hat, K_hat, V_hat: rows S_h of each head's Q, K, V; [Hq][L'][d] each.

    notes, Overall framework and Key design 1: gather Q, K, V by S_h into dense L' x d tensors.
    blog 1.1 (pseudo-code): gather of Q, K, V by the token indices.  Reading R5 for K and V.
    """
    L, Hq, d = Q.shape
    Hkv = K.shape[1]
    Qh = np.stack([Q[idx[h], h, :] for h in range(Hq)])
    Kh = np.stack([K[idx[h], gqa_group(h, Hq, Hkv), :] for h in range(Hq)])
    Vh = np.stack([V[idx[h], gqa_group(h, Hq, Hkv), :] for h in range(Hq)])
    return Qh, Kh, Vh


def attention_rows(Qh, Kh, Vh, pos, rows=None):
    """Causal softmax attention of one head in the compressed space, for the given output rows.

    blog 1.1: O_hat = softmax(Q_hat K_hat^T / sqrt(d)) V_hat.  The mask is written by original
    positions (reading R6): key j is visible to query i when pos[j] <= pos[i].
    Qh, Kh, Vh: [n][d]; pos: [n] original positions.  Returns [len(rows)][d].
    """
    n, d = Qh.shape
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    if len(rows) == 0:                      # L' = 0: nothing is attended
        return np.zeros((0, d))
    z = (Qh[rows] @ Kh.T) / np.sqrt(d)
    visible = pos[None, :] <= pos[rows][:, None]
    z = np.where(visible, z, -np.inf)
    m = z.max(axis=1, keepdims=True)
    e = np.where(visible, np.exp(z - m), 0.0)
    return (e / e.sum(axis=1, keepdims=True)) @ Vh


def compressed_attention(Qh, Kh, Vh, idx, rows=None):
    """O_hat for every head: [Hq][L' or len(rows)][d] (notes, Key design 1)."""
    return np.stack([attention_rows(Qh[h], Kh[h], Vh[h], idx[h], rows) for h in range(Qh.shape[0])])


# -- Stage 5: decompress and residual -------------------------------------------------------------

def decompress(Oh, idx, L):
    """Scatter O_hat back into a zero [L][Hq][d] tensor; unselected rows stay +0.0.

    notes, Key design 1: scatter O_hat to the matching rows of a zero-initialised L x d tensor;
    unselected rows keep 0 (a hard mask).  blog 1.1: zeros_like then scatter_.  Reading R7.
    """
    Hq, _, d = Oh.shape
    O = np.zeros((L, Hq, d))
    for h in range(Hq):
        O[idx[h], h, :] = Oh[h]
    return O


def residual(X, O):
    """X_{l+1} = X_l + Decompress(O_hat) (notes, Key design 1; summary, Core Architecture)."""
    return X + O


# -- Block sparsity stacked on the token selection --------------------------------------------------

BLOCK = 128


def block_pool(Xh, Lp, B=BLOCK):
    """Mean of every block of B consecutive compressed rows of one head (the last block over its
    valid rows), summed row by row in float64 and rounded once to float32 (reading R11).

    notes, Key findings and blog 3.2: token selection first, then block-level sparse attention on the
    compressed, contiguous Q_hat K_hat V_hat.  Xh: [>= L'][d].  Returns [ceil(L'/B)][d] float64
    holding float32 values."""
    nb = -(-Lp // B)
    out = np.zeros((nb, Xh.shape[1]))
    for b in range(nb):
        acc = np.zeros(Xh.shape[1])
        rows = range(b * B, min(Lp, (b + 1) * B))
        for r in rows:
            acc = acc + Xh[r]
        out[b] = (acc / len(rows)).astype(np.float32)
    return out


def block_select(qbar, kbar, gamma):
    """Kept key blocks of every query block (reading R11), each ascending.

    For query block I: weights a_J = softmax over J <= I of <qbar_I, kbar_J> / sqrt(d); order J by
    (a_J descending, J ascending) and take the shortest prefix whose cumulative weight reaches gamma
    (every J when gamma >= 1 or no prefix does); add J = 0 and J = I."""
    nb, d = qbar.shape
    keep = []
    for I in range(nb):
        z = (kbar[: I + 1] @ qbar[I]) / np.sqrt(d)
        a = np.exp(z - z.max())
        a = a / a.sum()
        order = np.lexsort((np.arange(I + 1), -a))
        cum = np.cumsum(a[order])
        hit = np.nonzero(cum >= gamma)[0]
        n = int(hit[0]) + 1 if (gamma < 1 and len(hit)) else I + 1
        keep.append(np.array(sorted(set(order[:n].tolist()) | {0, I}), dtype=np.int64))
    return keep


def block_sparse_attention_rows(Qh, Kh, Vh, keep, rows=None, B=BLOCK):
    """Causal attention of one head in the compressed space where row i (query block i // B) sees
    only keys j <= i inside its kept key blocks (reading R11)."""
    n, d = Qh.shape
    rows = np.arange(n) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), Vh.shape[1]))
    for o, i in enumerate(rows):
        blocks = keep[i // B]
        j = np.concatenate([np.arange(J * B, min((J + 1) * B, n)) for J in blocks])
        j = j[j <= i]
        z = Kh[j] @ Qh[i] / np.sqrt(d)
        e = np.exp(z - z.max())
        out[o] = (e / e.sum()) @ Vh[j]
    return out


def block_sparse_layer(Q, K, V, X, tau, q, gamma):
    """The token-sparse layer with block sparsity inside the compressed attention."""
    L = Q.shape[0]
    s_h = head_scores(Q, K, q)
    s_l = layer_score(s_h)
    k, Lp = budget(s_l, tau)
    idx = select(s_h, Lp)
    Qh, Kh, Vh = gather(Q, K, V, idx)
    keep = [block_select(block_pool(Qh[h], Lp), block_pool(Kh[h], Lp), gamma) for h in range(Qh.shape[0])]
    Oh = np.stack([block_sparse_attention_rows(Qh[h], Kh[h], Vh[h], keep[h]) for h in range(Qh.shape[0])])
    O = decompress(Oh, idx, L)
    Y = residual(X, O) if X is not None else O
    return dict(s_h=s_h, s_l=s_l, k=k, Lp=Lp, idx=idx, keep=keep, Oh=Oh, Y=Y)


# -- The whole layer and its dense counterpart ----------------------------------------------------

def layer(Q, K, V, X, tau, q, sparsity=None):
    """One Token Sparse Attention prefill layer, stage by stage.  Returns a dict of every stage.

    With sparsity given, the fixed-ratio budget replaces the coverage budget (tau is then unused)."""
    L = Q.shape[0]
    s_h = head_scores(Q, K, q)
    s_l = layer_score(s_h)
    k, Lp = budget(s_l, tau) if sparsity is None else budget_fixed_ratio(L, sparsity)
    idx = select(s_h, Lp)
    Qh, Kh, Vh = gather(Q, K, V, idx)
    Oh = compressed_attention(Qh, Kh, Vh, idx)
    O = decompress(Oh, idx, L)
    Y = residual(X, O) if X is not None else O
    return dict(s_h=s_h, s_l=s_l, k=k, Lp=Lp, idx=idx, Qh=Qh, Kh=Kh, Vh=Vh, Oh=Oh, O=O, Y=Y)


def layer_varlen(Q, K, V, X, cu_seqlens, tau, q):
    """A batch of independent sequences packed along the token axis (sample b owns tokens
    cu_seqlens[b] .. cu_seqlens[b+1]-1): each sample is one layer on its own, with its own scores,
    budget and keep count, so the keep counts differ across the batch (notes, Limitations: the
    ragged L' of batched inference).  Returns the per-sample stage dicts and the packed Y."""
    outs, Ys = [], []
    for b in range(len(cu_seqlens) - 1):
        t = slice(cu_seqlens[b], cu_seqlens[b + 1])
        r = layer(Q[t], K[t], V[t], None if X is None else X[t], tau, q)
        outs.append(r)
        Ys.append(r["Y"])
    return outs, np.concatenate(Ys, axis=0)


def dense_attention_rows(Q, K, V, h, rows=None):
    """Full-length causal attention of query head h with its GQA KV head (the dense baseline that
    the sparse layers replace; notes, Overall framework: non-sparse layers keep dense attention)."""
    L, Hq, _ = Q.shape
    g = gqa_group(h, Hq, K.shape[1])
    return attention_rows(Q[:, h, :], K[:, g, :], V[:, g, :], np.arange(L), rows)


def dense_layer(Q, K, V, X):
    """Y = X + causal attention on the full length, every head ([L][Hq][d])."""
    L, Hq, d = Q.shape
    O = np.stack([dense_attention_rows(Q, K, V, h) for h in range(Hq)], axis=1)
    return X + O if X is not None else O


# -- Load-time layer choice (not on the per-layer path) -------------------------------------------

def representation_drift(h_cur, h_next, eps=1e-6):
    """R_l = mean_t ||h_{l+1,t} - h_{l,t}||_2 / (||h_{l,t}||_2 + eps) (notes, Key design 3;
    blog 2.2).  h_cur, h_next: [T][D]."""
    num = np.linalg.norm(h_next - h_cur, axis=1)
    den = np.linalg.norm(h_cur, axis=1) + eps
    return float(np.mean(num / den))


def sparse_layers(R, delta=0.5):
    """L_sparse = { l : rank(R_l) / N <= delta }, rank 1 = the smallest drift, ties by layer id
    (notes, Key design 3: the least-drifting half of the layers by default).  1-based ids."""
    N = len(R)
    order = sorted(range(N), key=lambda i: (R[i], i))
    rank = {i: r + 1 for r, i in enumerate(order)}
    return sorted(i + 1 for i in range(N) if rank[i] / N <= delta)


# -- Storage rounding used by exact comparisons ---------------------------------------------------

def round_to_storage(x, dtype):
    """Round fp64 values to the storage type, to nearest even.

    fp32: one rounding.  bf16: fp64 -> fp32 -> bf16; the two-step path is exact for the sums of two
    stored values that the residual produces (a 24-bit intermediate is at least 2*8+2 bits, so the
    double rounding equals a single rounding of the exact sum).  Returns fp64 holding the rounded
    values.
    """
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f.astype(np.float64)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)
