"""Host-side rules of bench.py that need no GPU: the counter-derived traffic figure is reported only
for the shape and kernel source it was measured on, a multi-GPU request is refused, and the parity
verdict attached to the CPU baseline accepts the oracle's own layer and rejects planted mistakes."""

import os
import subprocess
import sys

import numpy as np
import torch

import bench
import oracle
from token_sparse_attention_amd.configs import WORKLOADS
from token_sparse_attention_amd.inputs import make_layer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_only_for_the_profiled_shape():
    kv = dict(ln.split(":", 1) for ln in open(bench.TRAFFIC_FILE) if ":" in ln and not ln.startswith("#"))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    prof = WORKLOADS[4]
    assert (kv["workload_L"], kv["workload_Hq"], kv["workload_d"]) == (str(prof.L), str(prof.Hq), str(prof.d))
    t = bench.measured_traffic(prof)
    if kv["attention_source_sha256_16"] == bench.source_hash(bench.ATTN_SOURCE):
        assert t == int(kv["hbm_bytes_per_launch"])
    else:
        assert t is None
    # the 256K chain has another shape: its launch was never counted
    assert bench.measured_traffic(WORKLOADS[5]) is None
    assert bench.measured_traffic(WORKLOADS[2]) is None


def test_traffic_null_when_source_changed(monkeypatch):
    monkeypatch.setattr(bench, "source_hash", lambda path: "0000000000000000")
    assert bench.measured_traffic(WORKLOADS[4]) is None


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _oracle_run(cfg):
    """The oracle's own layer on a small workload, shaped like a device run (Y as stored, idx padded
    to [Hq][L]), and the oracle's sampled attention rows as the CPU baseline keeps them."""
    inp = make_layer(cfg)
    f64 = lambda t: t.double().numpy()
    Q, K, V, X = (f64(inp[n]) for n in ("Q", "K", "V", "X"))
    r = oracle.layer(Q, K, V, X, float(np.float32(cfg.tau)), cfg.q)
    Lp = r["Lp"]
    Y = torch.from_numpy(r["Y"]).to(torch.float32)
    idx = torch.full((cfg.Hq, cfg.L), -1, dtype=torch.int32)
    idx[:, :Lp] = torch.from_numpy(np.asarray(r["idx"], dtype=np.int32))
    rng = np.random.default_rng(1)
    kept = {}
    for h in (0, cfg.Hq - 1):
        rows = np.sort(rng.choice(Lp, 16, replace=False))
        kept[h] = [(rows, r["Oh"][h][rows])]
    return inp, r, Y, idx, kept


def test_parity_verdict_accepts_the_oracle_and_rejects_planted_errors():
    cfg = WORKLOADS[1]
    inp, r, Y, idx, kept = _oracle_run(cfg)
    k, Lp = r["k"], r["Lp"]
    args = (cfg, inp["X"], r["s_h"], r["s_l"], k, Lp, r["idx"], kept)
    ok = bench.parity_verdict(*args, k, Lp, Y, idx)
    assert ok["pass"] and ok["heads_selection_equal"] == cfg.Hq and ok["output_rows_checked"] == 32
    assert ok["unselected_rows_equal_X"] and ok["output_outside_tolerance"] == 0
    # a wrong value at one sampled output row
    rows, _ = kept[0][0]
    Yb = Y.clone()
    Yb[int(r["idx"][0][rows[3]]), 0, 5] += 0.01
    bad = bench.parity_verdict(*args, k, Lp, Yb, idx)
    assert not bad["pass"] and bad["output_outside_tolerance"] == 1
    # a token a head did not keep must stay X
    dropped = int(np.setdiff1d(np.arange(cfg.L), r["idx"][0])[0])
    Yb = Y.clone()
    Yb[dropped, 0, 0] += 1.0
    assert not bench.parity_verdict(*args, k, Lp, Yb, idx)["unselected_rows_equal_X"]
    # a selection that swaps a clearly kept token for a clearly dropped one
    ib = idx.clone()
    top = int(np.argmax(r["s_h"][1]))
    low = int(np.argmin(r["s_h"][1]))
    sel = set(r["idx"][1].tolist())
    assert top in sel and low not in sel
    sel = sorted((sel - {top}) | {low})
    ib[1, :Lp] = torch.tensor(sel, dtype=torch.int32)
    v = bench.parity_verdict(*args, k, Lp, Y, ib)
    assert not v["pass"] and v["heads_selection_equal"] == cfg.Hq - 1 and v["heads_within_tie_band"] == 0
    # a budget off by one is outside the coverage band
    assert not bench.parity_verdict(*args, k + 1, Lp, Y, idx)["budget_ok"]


def test_stage_traffic_only_for_unchanged_sources(monkeypatch):
    prof = WORKLOADS[4]
    got = bench.measured_stage_traffic(prof)
    kv = dict(ln.split(":", 1) for ln in open(bench.STAGE_TRAFFIC_FILE) if ":" in ln and not ln.startswith("#"))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    for st, srcs in bench.STAGE_SOURCES.items():
        now = [bench.source_hash(os.path.join(ROOT, "token_sparse_attention_amd", "csrc", src)) for src in srcs]
        if all(kv[f"source_sha256_16 {src}"] == h for src, h in zip(srcs, now)):
            assert got[st] == int(kv[f"{st}_hbm_bytes"])
        else:
            assert st not in got
    assert bench.measured_stage_traffic(WORKLOADS[5]) == {}
    monkeypatch.setattr(bench, "source_hash", lambda path: "0000000000000000")
    assert bench.measured_stage_traffic(prof) == {}


def test_attention_counters_only_on_the_counted_shape_and_source(monkeypatch):
    got = bench.measured_counters(WORKLOADS[4])
    kv = dict(ln.split(":", 1) for ln in open(bench.COUNTERS_FILE) if ":" in ln and not ln.startswith("#"))
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv["attention_source_sha256_16"] == bench.source_hash(bench.ATTN_SOURCE):
        assert got["mfma_busy_fraction"] == float(kv["mfma_busy_fraction"])
        assert 0.0 < got["mfma_busy_fraction"] < 1.0 and got["lds_bank_conflicts"] >= 0
    else:
        assert got is None
    assert bench.measured_counters(WORKLOADS[5]) is None
    monkeypatch.setattr(bench, "source_hash", lambda path: "0000000000000000")
    assert bench.measured_counters(WORKLOADS[4]) is None


def _sweep_evidence_from_oracle(cfg, kind, **param):
    """Evidence shaped like bench.sweep_evidence's, built from the oracle's own layer (the stored
    output rounded to the storage type as the device writes it)."""
    inp = make_layer(cfg)
    f64 = lambda t: t.double().numpy()
    Q, K, V, X = (f64(inp[n]) for n in ("Q", "K", "V", "X"))
    tau = float(np.float32(param.get("tau", cfg.tau)))
    if kind == "block":
        r = oracle.block_sparse_layer(Q, K, V, X, tau, cfg.q, param["gamma"])
    else:
        r = oracle.layer(Q, K, V, X, tau, cfg.q, sparsity=param.get("sparsity"))
    Lp = r["Lp"]
    Y = oracle.round_to_storage(r["Y"], cfg.dtype)
    rng = np.random.default_rng(3)
    rows = {h: np.sort(rng.choice(Lp, 6, replace=False)) for h in range(cfg.Hq)}
    ev = {"kind": kind, **param, "k_gpu": r["k"], "Lp_gpu": Lp, "sel": np.asarray(r["idx"]),
          "rows": {h: (rw, Y[r["idx"][h][rw], h]) for h, rw in rows.items()},
          "unselected_rows_equal_X": True, "all_rows_written": True}
    if kind == "block":
        ev["block_lists"] = {h: r["keep"][h] for h in range(cfg.Hq)}
    return (Q, K, V, X), r, ev


def test_sweep_verdict_accepts_the_oracle_and_rejects_planted_errors():
    cfg = WORKLOADS[1]
    for kind, param in (("tau", {"tau": 0.5}), ("ratio", {"sparsity": 0.3}), ("block", {"tau": 0.3, "gamma": 0.5})):
        (Q, K, V, X), r, ev = _sweep_evidence_from_oracle(cfg, kind, **param)
        v = bench.sweep_verdict(cfg, Q, K, V, X, r["s_h"], r["s_l"], ev)
        assert v["pass"], (kind, v)
        assert v["heads_selection_equal"] == cfg.Hq and v["output_rows_checked"] == 6 * cfg.Hq
        # one sampled output element off by more than the tolerance
        bad = dict(ev, rows=dict(ev["rows"]))
        rw, y = bad["rows"][1]
        y = y.copy()
        y[2, 7] += 0.05
        bad["rows"][1] = (rw, y)
        assert not bench.sweep_verdict(cfg, Q, K, V, X, r["s_h"], r["s_l"], bad)["pass"], kind
        # a row the layer never wrote, or a dropped token that lost its X
        for flag in ("all_rows_written", "unselected_rows_equal_X"):
            assert not bench.sweep_verdict(cfg, Q, K, V, X, r["s_h"], r["s_l"], dict(ev, **{flag: False}))["pass"]
        # a keep count one off
        assert not bench.sweep_verdict(cfg, Q, K, V, X, r["s_h"], r["s_l"], dict(ev, k_gpu=ev["k_gpu"] + 1))["pass"]
        # a head keeping a clearly dropped token instead of its best one
        sel = ev["sel"].copy()
        top, low = int(np.argmax(r["s_h"][0])), int(np.argmin(r["s_h"][0]))
        assert top in set(sel[0].tolist()) and low not in set(sel[0].tolist())
        sel[0] = np.sort(np.array(sorted((set(sel[0].tolist()) - {top}) | {low})))
        v = bench.sweep_verdict(cfg, Q, K, V, X, r["s_h"], r["s_l"], dict(ev, sel=sel))
        assert not v["pass"] and v["heads_selection_equal"] == cfg.Hq - 1
        if kind == "block":
            # a kept-block list that drops a block the oracle keeps
            lists = dict(ev["block_lists"])
            h = 2
            I = max(range(len(lists[h])), key=lambda i: len(lists[h][i]))
            assert len(lists[h][I]) > 2
            lists[h] = list(lists[h])
            lists[h][I] = lists[h][I][[0, -1]]
            v = bench.sweep_verdict(cfg, Q, K, V, X, r["s_h"], r["s_l"], dict(ev, block_lists=lists))
            assert not v["pass"] and v["heads_block_lists_equal"] == cfg.Hq - 1
