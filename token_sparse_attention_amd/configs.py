"""The five synthetic workloads of the Token Sparse Attention prefill layer.

Shapes follow the attention shapes the pages evaluate on (LLaMA-3.1-8B-Instruct: 32 query heads,
8 KV heads, head dim 128; contexts 4K / 32K / 128K, with q = 16 recent queries and tau = 0.005 as the
LLaMA default -- papernotes.org reading notes, "Key design 2" and "Loss function / training strategy";
bxzpzcl.cn article, section 4.1 for q = 64 beyond 256K).  The salient-token planting is a synthetic
stand-in for the pages' RULER workloads (no dataset or weights are used).

Each entry is plain data; the generator in ``inputs.py`` turns it into tensors.
"""

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    L: int                 # tokens
    Hq: int                # query heads
    Hkv: int               # key/value heads (GQA when Hkv < Hq)
    d: int                 # head dim
    q: int                 # recent queries used for scoring
    tau: float             # coverage threshold
    dtype: str             # "f32" or "bf16" storage / compute type of Q, K, V, X
    salient_frac: float    # planted salient positions per KV head, as a fraction of L
    shared_frac: float     # part of each head's salient set that all heads share
    sink: int = 0          # leading positions whose keys get an extra 2*u push
    seed: int = 0
    layers: int = 1        # >1: attention-only chain with the residual carried
    layer_overlap: float = 0.0   # fraction of a head's salient set kept from the previous layer
    sparse_layers: tuple = field(default_factory=tuple)  # 1-based ids of sparse layers (chain only)


WORKLOADS = {
    1: Workload("tiny_fp32_L1024_H4_d64", L=1024, Hq=4, Hkv=4, d=64, q=16, tau=0.005, dtype="f32",
                salient_frac=0.03, shared_frac=1.0, seed=1),
    2: Workload("bf16_L4096_H32_d128", L=4096, Hq=32, Hkv=32, d=128, q=16, tau=0.005, dtype="bf16",
                salient_frac=0.02, shared_frac=0.5, seed=2),
    3: Workload("bf16_L32768_H32_KV8_d128_sink", L=32768, Hq=32, Hkv=8, d=128, q=16, tau=0.01,
                dtype="bf16", salient_frac=0.01, shared_frac=1.0, sink=64, seed=3),
    4: Workload("bf16_L131072_H32_KV8_d128", L=131072, Hq=32, Hkv=8, d=128, q=16, tau=0.005,
                dtype="bf16", salient_frac=0.005, shared_frac=0.3, seed=4),
    5: Workload("bf16_chain8_L262144_H32_KV8_d128_q64", L=262144, Hq=32, Hkv=8, d=128, q=64,
                tau=0.002, dtype="bf16", salient_frac=0.005, shared_frac=0.3, seed=5, layers=8,
                layer_overlap=0.4, sparse_layers=(5, 6, 7, 8)),
}


def scaled(cfg: Workload, L: int, **over) -> Workload:
    """The same workload recipe at another length (for small parity cases)."""
    kw = dict(cfg.__dict__)
    kw.update(L=L, **over)
    kw["name"] = f"{cfg.name}@L{L}"
    return Workload(**kw)
