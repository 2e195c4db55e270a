"""Thin helpers over the binding: a layer object that owns its workspace, and the load-time choice
of sparse layers.  Argument marshalling and bookkeeping only; all arithmetic of the layer runs in
libtsa.so."""

import torch

from . import binding


class SparseLayer:
    """One Token Sparse Attention prefill layer of a fixed shape on one device.

    Owns the layer workspace and a device int32[2] that receives {k, L'} on every call, so the keep
    count never forces a host synchronisation.
    """

    def __init__(self, L, Hq, Hkv, d, q, tau, dtype="bf16", device="cuda"):
        self.shape = binding.shape(L, Hq, Hkv, d, q, tau, dtype)
        st = binding.check_args(self.shape)
        if st != 0:
            raise binding.TsaError("tsa_check_args", st)
        self.device = torch.device(device)
        self.ws = binding.workspace(binding.layer_workspace_bytes(self.shape), self.device)
        self.kLp = torch.zeros(2, dtype=torch.int32, device=self.device)

    @classmethod
    def for_workload(cls, cfg, device="cuda"):
        return cls(cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.q, cfg.tau, cfg.dtype, device)

    def __call__(self, Q, K, V, X, Y=None, stream=None):
        """Y = X + Decompress(attention on each head's kept tokens).  Y defaults to a new tensor;
        pass Y=X to update the residual stream in place."""
        if Y is None:
            Y = torch.empty_like(Q if X is None else X)
        binding.layer(self.shape, Q, K, V, X, Y, self.kLp, self.ws, stream)
        return Y

    def keep_count(self):
        """(k, L') of the last call (synchronises with the device)."""
        k, Lp = self.kLp.tolist()
        return k, Lp


class DenseLayer:
    """Dense causal attention over the full length plus the residual (the layers TSA leaves dense)."""

    def __init__(self, L, Hq, Hkv, d, q=1, tau=0.0, dtype="bf16", device="cuda"):
        self.shape = binding.shape(L, Hq, Hkv, d, q, tau, dtype)
        self.device = torch.device(device)
        self.ws = binding.workspace(binding.dense_workspace_bytes(self.shape), self.device)

    @classmethod
    def for_workload(cls, cfg, device="cuda"):
        return cls(cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.q, cfg.tau, cfg.dtype, device)

    def __call__(self, Q, K, V, X, Y=None, stream=None):
        if Y is None:
            Y = torch.empty_like(Q if X is None else X)
        binding.dense_attn_causal(self.shape, Q, K, V, X, Y, self.ws, stream)
        return Y


def select_sparse_layers(drift, delta=0.5):
    """Layers that run Token Sparse Attention, chosen once at load time from the inter-layer
    representation drift R_l (papernotes.org reading notes, "Key design 3"; bxzpzcl.cn article,
    section 2.2): rank the layers by drift (rank 1 = the most stable, ties by layer id) and keep
    those with rank / N <= delta, by default the least-drifting half.  Returns 1-based layer ids."""
    n = len(drift)
    order = sorted(range(n), key=lambda i: (float(drift[i]), i))
    return sorted(i + 1 for r, i in enumerate(order) if (r + 1) / n <= delta)
