"""Benchmark of the Token Sparse Attention prefill layer on one MI355X.

One step = one full layer (score -> budget -> select -> gather -> compressed causal attention ->
scatter + residual) through the C ABI on the L = 131072, 32/8-head, d = 128, bf16 workload with
inputs resident in HBM.  Prints one JSON line: the layer latency, the speedup over this library's
own dense causal attention on the full length, per-stage times with their roofline fractions, the
roofline of the dominant kernel (the compressed attention, bf16 matrix cores) and the CPU oracle
timed on a bounded sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from token_sparse_attention_amd import binding  # noqa: E402
from token_sparse_attention_amd.configs import WORKLOADS  # noqa: E402
from token_sparse_attention_amd.inputs import chain_drift_values, iter_chain, make_batch, make_layer  # noqa: E402
from token_sparse_attention_amd.runtime import select_sparse_layers  # noqa: E402

METRIC = "TSA layer ms & speedup vs own dense attn at L=128K; MFMA util, HBM GB/s"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
FP32_PEAK_TFLOPS = 157.3       # MI355X fp32 vector peak


T_START = time.perf_counter()


def progress(msg):
    """One line on stderr per finished phase (stdout carries only the JSON record)."""
    print(f"[bench {time.perf_counter() - T_START:7.1f} s] {msg}", file=sys.stderr, flush=True)


def timed(fn, steps, warmup, stream):
    """Mean ms per call of fn() over `steps` calls, HIP events on the launch stream."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(steps):
        fn()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def gpu_clocks():
    """Shader clock, memory clock and power lines as rocm-smi prints them, or None when the tool is
    unavailable."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower"], capture_output=True, text=True, timeout=20)
    except (OSError, subprocess.SubprocessError):
        return None
    keep = [" ".join(ln.split()) for ln in r.stdout.splitlines()
            if any(k in ln for k in ("sclk", "mclk", "Power (W)", "Power:")) and ln.strip()]
    return keep or None


class ClockSampler:
    """Reads gpu_clocks() once, `delay` seconds after start(), from a background thread (the
    sample then falls inside a timed region that lasts longer than the delay)."""

    def __init__(self, delay):
        import threading
        self.delay, self.value = delay, None
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        time.sleep(self.delay)
        self.value = gpu_clocks()

    def start(self):
        self.thread.start()
        return self

    def result(self):
        self.thread.join(timeout=30)
        return self.value


def timed_pair(fa, fb, steps, warmup, stream):
    """Per-call ms of fa() and of fb() over `steps` calls of each, alternating a, b, a, b, ... so that
    clock drift over the run affects both alike; every call is bracketed by synchronizations and HIP
    events on the launch stream."""
    for _ in range(warmup):
        fa()
        fb()
    ta, tb = [], []
    for _ in range(steps):
        for fn, acc in ((fa, ta), (fb, tb)):
            torch.cuda.synchronize()
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            fn()
            t1.record(stream)
            torch.cuda.synchronize()
            acc.append(t0.elapsed_time(t1))
    return ta, tb


def make_flush(dev):
    """A 512 MiB float32 buffer whose read evicts every input from the 256 MB last-level cache."""
    return torch.zeros(128 << 20, dtype=torch.float32, device=dev)


def evict(flush):
    """Reads the flush buffer (one reduction).  A read leaves the caches clean: writing the buffer
    instead would leave 256 MB of dirty lines whose write-back then lands inside the next timed call
    (on this part that halves the rate of a following 268 MB read, 5.2 -> 2.7 TB/s)."""
    return flush.amax()


def timed_cold(fn, steps, warmup, stream, flush):
    """Per-call ms of fn() over `steps` calls, each after reading a 512 MiB scratch buffer so the
    256 MB last-level cache holds none of fn's inputs; HIP events around each call."""
    for _ in range(warmup):
        fn()
    times = []
    for _ in range(steps):
        evict(flush)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        fn()
        t1.record(stream)
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1))
    return times


def pct(times):
    """p10 / p50 / p90 of per-call ms."""
    p10, p50, p90 = np.percentile(np.asarray(times, dtype=np.float64), [10, 50, 90])
    return {"p10": round(float(p10), 4), "p50": round(float(p50), 4), "p90": round(float(p90), 4)}


def hbm_practical(dev, steps=10):
    """What plain torch device operations reach on this GPU, as context for the stage fractions
    (all against the 8 TB/s published peak): a write-only fill, a copy and a read-only reduction of a
    2 GiB buffer, median of `steps` calls each."""
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    b.fill_(2)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    fill_ms = float(np.median(timed_calls(lambda: a.fill_(3), steps, 1, stream)))
    copy_ms = float(np.median(timed_calls(lambda: b.copy_(a), steps, 1, stream)))
    af = a.view(torch.float32)
    read_ms = float(np.median(timed_calls(lambda: af.amax(), steps, 1, stream)))
    del a, b, af
    torch.cuda.empty_cache()
    fill, copy, read = n / (fill_ms * 1e-3) / 1e9, 2 * n / (copy_ms * 1e-3) / 1e9, n / (read_ms * 1e-3) / 1e9
    return {"write_only_fill_GB_s": round(fill, 1), "fill_frac": round(fill / HBM_PEAK_GBS, 4),
            "copy_GB_s": round(copy, 1), "copy_frac": round(copy / HBM_PEAK_GBS, 4),
            "read_only_GB_s": round(read, 1), "read_frac": round(read / HBM_PEAK_GBS, 4),
            "how": "torch fill_, copy_ and amax on 2 GiB device buffers, median of per-call HIP events"}


def timed_calls(fn, steps, warmup, stream):
    """Per-call ms of fn() in steady state (no cache flush), every call bracketed by HIP events."""
    for _ in range(warmup):
        fn()
    times = []
    for _ in range(steps):
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        fn()
        t1.record(stream)
        torch.cuda.synchronize()
        times.append(t0.elapsed_time(t1))
    return times


def algorithmic(cfg, Lp, union_rows):
    """Bytes (or flops) each stage must move (or compute) by definition, independent of how."""
    e = 2 if cfg.dtype == "bf16" else 4
    L, Hq, Hkv, d, q = cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.q
    return {
        "score": L * Hkv * d * e + q * Hq * d * e + 4 * Hq * L + 4 * L,
        "budget": 4 * L + 8,
        "select": 4 * Hq * L + 4 * Hq * Lp + 4 * Hq * L,
        "gather": Hq * Lp * d * e + 2 * union_rows * d * e + 4 * Hq * Lp + 3 * Hq * Lp * d * e,
        "scatter": 2 * L * Hq * d * e + Hq * Lp * d * e + 4 * Hq * L,
        "attn_flops": 4 * d * Hq * Lp * (Lp + 1) // 2,
        "dense_flops": 4 * d * Hq * L * (L + 1) // 2,
    }


PARITY_TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}   # |gpu - ref| <= atol + rtol |ref|


def host_info():
    """The host the CPU baseline ran on: CPU model, logical CPUs and memory, from /proc."""
    info = {"logical_cpus": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            info["cpu_model"] = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), None)
        with open("/proc/meminfo") as f:
            kib = next((int(ln.split()[1]) for ln in f if ln.startswith("MemTotal:")), None)
        info["ram_gib"] = round(kib / 2 ** 20, 1) if kib else None
    except OSError:
        pass
    return info


def cpu_baseline(cfg, inp, k_gpu, Lp_gpu, Y_gpu, idx_gpu, pending=(), budget_s=12.0):
    """The CPU oracle (float64, as it stands) on a bounded sample of the same workload, on ONE thread
    (its BLAS limited to one), scaled to one full layer: scoring, budget and selection run in full
    and are measured; gather + attention run on a sample of output rows of a few heads and are
    extrapolated by the exact causal pair count; decompress + residual runs on a sample of rows and
    is extrapolated by the row count.  Returns that timing, the parity verdict of the GPU run being
    reported (from the same oracle results), and a verdict for every supplementary line in
    `pending` (evidence from sweep_evidence)."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    f64 = lambda t: t.double().numpy()
    Q, K, V, X = (f64(inp[n]) for n in ("Q", "K", "V", "X"))
    stages = {}
    with threadpool_limits(limits=1):
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        t0 = time.perf_counter()
        s_h = oracle.head_scores(Q, K, cfg.q)
        stages["score"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        s_l = oracle.layer_score(s_h)
        k, Lp = oracle.budget(s_l, float(np.float32(cfg.tau)))
        stages["layer_score_and_budget"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        idx = oracle.select(s_h, Lp)
        stages["select"] = time.perf_counter() - t0
        # attention on sampled rows of sampled heads, batches of rows until about budget_s of work;
        # the pair count of compressed row i is i + 1
        rng = np.random.default_rng(0)
        heads = [0, cfg.Hq // 2 + 1]
        t0 = time.perf_counter()
        sampled_pairs, n_rows = 0.0, 0
        per_head, kept = {}, {h: [] for h in heads}
        while time.perf_counter() - t0 < budget_s:
            for h in heads:
                if h not in per_head:
                    g = oracle.gqa_group(h, cfg.Hq, cfg.Hkv)
                    per_head[h] = (Q[idx[h], h, :], K[idx[h], g, :], V[idx[h], g, :])
                rows = np.sort(rng.choice(Lp, 16, replace=False))
                qh, kh, vh = per_head[h]
                o = oracle.attention_rows(qh, kh, vh, idx[h], rows)
                if len(kept[h]) < 8:
                    kept[h].append((rows, o))
                sampled_pairs += float(np.sum(rows + 1))
                n_rows += len(rows)
        t_att = time.perf_counter() - t0
        total_pairs = cfg.Hq * Lp * (Lp + 1) / 2.0
        stages["gather_and_attention"] = t_att * total_pairs / sampled_pairs
        # decompress + residual on a sample of rows (cost linear in rows)
        n_dec = 4096
        t0 = time.perf_counter()
        Oh = np.zeros((cfg.Hq, n_dec, cfg.d))
        oracle.residual(X[:n_dec], oracle.decompress(Oh, np.tile(np.arange(n_dec), (cfg.Hq, 1)), n_dec))
        stages["decompress_and_residual"] = (time.perf_counter() - t0) * cfg.L / n_dec
    measured = ("score", "layer_score_and_budget", "select")
    total_ms = 1e3 * sum(stages.values())
    base = {"value": round(total_ms, 1), "unit": "ms", "cores": int(cores), "kind": "oracle",
            "extrapolated": True,
            "stages_ms": {k2: {"ms": round(1e3 * v, 1), "how": "measured" if k2 in measured else "extrapolated"}
                          for k2, v in stages.items()},
            "sample": (f"numpy float64 oracle on one thread (BLAS limited to 1) on this workload: scoring, "
                       f"budget and selection measured in full ({sum(stages[m] for m in measured):.1f} s); "
                       f"gather+attention on {n_rows} random rows of {len(heads)} heads ({t_att:.1f} s), "
                       f"extrapolated by the causal pair count to {cfg.Hq} heads x L'={Lp}; decompress+residual "
                       f"on {n_dec} rows, extrapolated to L={cfg.L}"),
            "oracle_k": int(k), "oracle_Lp": int(Lp), "gpu_Lp": int(Lp_gpu), "host": host_info()}
    par = parity_verdict(cfg, inp["X"], s_h, s_l, k, Lp, idx, kept, k_gpu, Lp_gpu, Y_gpu, idx_gpu)
    sweeps = [sweep_verdict(cfg, Q, K, V, X, s_h, s_l, ev) for ev in pending]
    return base, par, sweeps


class _QRows:
    """Head h's compressed query rows Q[pos[i], h] read only where the oracle asks for them (its
    attention takes the sampled rows of Q_hat); shape as the full [len(pos)][d] array."""

    def __init__(self, Q, pos, h, d):
        self.Q, self.pos, self.h, self.shape = Q, pos, h, (len(pos), d)

    def __getitem__(self, rows):
        return np.asarray(self.Q[self.pos[rows], self.h, :], dtype=np.float64)


class _F64Rows:
    """Indexing into a stored (bf16) host tensor that returns float64 numpy rows, so the verdict can
    read a 256K layer's rows without widening the whole tensor."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, key):
        return self.t[key].double().numpy()


def chain_verdicts(cfg, pending):
    """The oracle leg for the 256K chain's lines (its tau sweep and its sparse layers): the oracle's
    scores of each line's own layer inputs, then sweep_verdict on that line.  Part of the CPU-baseline
    (oracle) leg: skipped with --no-cpu-baseline."""
    import oracle
    out, cache = [], {}
    for _, ev in pending:
        inp = ev["inputs"]
        key = id(inp["K"])
        if key not in cache:
            cache.clear()
            s_h = oracle.head_scores_recent(inp["Q"][cfg.L - cfg.q:].double().numpy(), inp["K"].double().numpy())
            cache[key] = (s_h, oracle.layer_score(s_h))
        s_h, s_l = cache[key]
        out.append(sweep_verdict(cfg, _F64Rows(inp["Q"]), _F64Rows(inp["K"]), _F64Rows(inp["V"]), _F64Rows(ev["X_in"]),
                                 s_h, s_l, ev))
    return out


def sweep_verdict(cfg, Q, K, V, X, s_h, s_l, ev):
    """One supplementary line against the oracle (float64 inputs Q, K, V, X and the oracle's s_h,
    s_l of the same workload), with the parity tests' rules: the keep count (the fixed-ratio count
    exactly; a coverage budget equal to the oracle's or on both sides of the threshold within 1e-5),
    each head's selection equal to the oracle's top-L' or differing only on scores within 1e-6 of the
    boundary, Y at the sampled rows within the floating-point tolerance against the oracle's
    attention on that selection (block-sparse lines: on the kept-block lists, which must equal the
    oracle's), dropped tokens equal to X bitwise, and every element of Y written."""
    import oracle
    k_gpu, Lp = ev["k_gpu"], ev["Lp_gpu"]
    if ev["kind"] == "ratio":
        k, Lp_or = oracle.budget_fixed_ratio(cfg.L, ev["sparsity"])
        budget_ok = k == k_gpu
    else:
        tau = float(np.float32(ev["tau"]))
        k, Lp_or = oracle.budget(s_l, tau)
        Cs = np.concatenate([[0.0], np.cumsum(np.sort(s_l))])
        budget_ok = k == k_gpu or (Cs[k_gpu] >= tau * (1 - 1e-5) and (k_gpu == 0 or Cs[k_gpu - 1] < tau * (1 + 1e-5)))
    out = {"k_oracle": int(k), "k_gpu": int(k_gpu), "budget_ok": bool(budget_ok)}
    want = oracle.select(s_h, Lp)          # the oracle's top-L' at the GPU's keep count
    sel = ev["sel"]
    equal, in_band, ok_heads = 0, 0, []
    for h in range(cfg.Hq):
        if np.array_equal(sel[h], want[h]):
            equal += 1
            ok_heads.append(h)
            continue
        diff = np.setxor1d(sel[h], want[h])
        b = np.sort(s_h[h])[::-1][Lp - 1]
        if (np.abs(s_h[h][diff] - b) <= 1e-6 * b).all():
            in_band += 1
            ok_heads.append(h)
    atol, rtol = PARITY_TOL[cfg.dtype]
    G = cfg.Hq // cfg.Hkv
    n_rows, worst, bad, lists_equal = 0, 0.0, 0, None
    if ev["kind"] == "block":
        lists_equal = 0
    for h, (rows, got) in ev["rows"].items():
        if h not in ok_heads:
            continue
        pos = sel[h]
        Qh, Kh, Vh = _QRows(Q, pos, h, cfg.d), K[pos, h // G, :], V[pos, h // G, :]
        if ev["kind"] == "block":
            keep = oracle.block_select(oracle.block_pool(Qh, Lp), oracle.block_pool(Kh, Lp), ev["gamma"])
            gl = ev["block_lists"][h]
            same = len(gl) == len(keep) and all(np.array_equal(a, b) for a, b in zip(gl, keep))
            lists_equal += int(same)
            if not same:
                continue
            o = oracle.block_sparse_attention_rows(Qh, Kh, Vh, keep, rows)
        else:
            o = oracle.attention_rows(Qh, Kh, Vh, pos, rows)
        ref = X[pos[rows], h, :] + o
        err = np.abs(got - ref)
        worst = max(worst, float(err.max()))
        bad += int((err > atol + rtol * np.abs(ref)).sum())
        n_rows += len(rows)
    out.update({"heads_selection_equal": equal, "heads_within_tie_band": in_band, "output_rows_checked": n_rows,
                "output_max_abs_err": round(worst, 6), "output_tolerance": f"{atol:g} + {rtol:g} |ref|",
                "output_outside_tolerance": bad, "unselected_rows_equal_X": ev["unselected_rows_equal_X"],
                "all_rows_written": ev["all_rows_written"]})
    if lists_equal is not None:
        out["heads_block_lists_equal"] = lists_equal
    out["pass"] = bool(budget_ok and equal + in_band == cfg.Hq and bad == 0 and (n_rows > 0 or Lp == 0)
                       and ev["unselected_rows_equal_X"] and ev["all_rows_written"]
                       and (lists_equal is None or lists_equal == len(ev["rows"])))
    return out


def parity_verdict(cfg, X_stored, s_h, s_l, k, Lp, idx, kept, k_gpu, Lp_gpu, Y_gpu, idx_gpu):
    """The reported GPU run against the oracle, with the acceptance rules of the parity tests:
    k equal, or both sides of the coverage threshold within 1e-5 relative; per-head selections equal,
    or differing only on scores within 1e-6 of the boundary; the layer output at the oracle's sampled
    attention rows within the floating-point tolerance; tokens a head did not keep equal to X
    bitwise."""
    tau = float(np.float32(cfg.tau))
    Cs = np.concatenate([[0.0], np.cumsum(np.sort(s_l))])
    budget_ok = k == k_gpu or (Cs[k_gpu] >= tau * (1 - 1e-5) and (k_gpu == 0 or Cs[k_gpu - 1] < tau * (1 + 1e-5)))
    out = {"k_oracle": int(k), "k_gpu": int(k_gpu), "budget_ok": bool(budget_ok)}
    if Lp != Lp_gpu:
        out.update({"selection_compared": False, "pass": bool(budget_ok)})
        return out
    gsel = idx_gpu[:, :Lp].cpu().numpy().astype(np.int64)
    equal, in_band = 0, 0
    for h in range(cfg.Hq):
        if np.array_equal(gsel[h], idx[h]):
            equal += 1
            continue
        diff = np.setxor1d(gsel[h], idx[h])
        bnd = np.sort(s_h[h])[::-1][Lp - 1]
        in_band += int((np.abs(s_h[h][diff] - bnd) <= 1e-6 * bnd).all())
    atol, rtol = PARITY_TOL[cfg.dtype]
    X64 = X_stored.double()
    n_rows, worst, bad, unsel_ok = 0, 0.0, 0, True
    for h, samples in kept.items():
        if not np.array_equal(gsel[h], idx[h]):
            continue
        for rows, o in samples:
            tok = idx[h][rows]
            got = Y_gpu[torch.as_tensor(tok, device=Y_gpu.device), h].double().cpu().numpy()
            ref = X64[torch.as_tensor(tok), h].numpy() + o
            err = np.abs(got - ref)
            worst = max(worst, float(err.max()))
            bad += int((err > atol + rtol * np.abs(ref)).sum())
            n_rows += len(rows)
        dropped = np.setdiff1d(np.arange(cfg.L), idx[h])[:64]
        if len(dropped):
            t = torch.as_tensor(dropped)
            unsel_ok &= bool(torch.equal(Y_gpu[t.to(Y_gpu.device), h].cpu(), X_stored[t, h]))
    out.update({"selection_compared": True, "heads_selection_equal": equal, "heads_within_tie_band": in_band,
                "output_rows_checked": n_rows, "output_max_abs_err": round(worst, 6),
                "output_tolerance": f"{atol:g} + {rtol:g} |ref|", "output_outside_tolerance": bad,
                "unselected_rows_equal_X": unsel_ok})
    out["pass"] = bool(budget_ok and equal + in_band == cfg.Hq and bad == 0 and n_rows > 0 and unsel_ok)
    return out


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attention_L131072_bf16.txt")
ATTN_SOURCE = os.path.join(ROOT, "token_sparse_attention_amd", "csrc", "attention.hip")


def source_hash(path):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(cfg):
    """HBM bytes per launch of the compressed attention from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE, each divided by the factor the same counter reads for a plain copy
    of known size), or None when that summary is missing, was taken on another shape than `cfg`'s,
    or the kernel source has changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("attention_source_sha256_16") != source_hash(ATTN_SOURCE):
        return None
    if (kv.get("workload_L"), kv.get("workload_Hq"), kv.get("workload_d")) != (str(cfg.L), str(cfg.Hq), str(cfg.d)):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


# the sources of each stage's kernels (the score stage includes the layer score's kernels)
STAGE_SOURCES = {"score": ("score.hip", "select.hip"), "budget": ("select.hip",), "select": ("select.hip",),
                 "gather": ("move.hip",), "scatter": ("move.hip",)}
STAGE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_stages_L131072_bf16.txt")


COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_attention_L131072_bf16.txt")


def measured_counters(cfg):
    """The attention kernel's counted matrix-core busy fraction and instruction mix from the
    committed counter summary, or None off the counted shape or once the kernel source changed."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    for line in open(COUNTERS_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("attention_source_sha256_16") != source_hash(ATTN_SOURCE):
        return None
    if (kv.get("workload_L"), kv.get("workload_Hq"), kv.get("workload_d")) != (str(cfg.L), str(cfg.Hq), str(cfg.d)):
        return None
    try:
        return {"mfma_busy_fraction": float(kv["mfma_busy_fraction"]), "valu_per_mfma": float(kv["valu_per_mfma"]),
                "lds_per_mfma": float(kv["lds_per_mfma"]), "lds_bank_conflicts": int(kv["lds_bank_conflicts"]),
                "source": os.path.relpath(COUNTERS_FILE, ROOT)}
    except (KeyError, ValueError):
        return None


def traffic_probe(cfg, dev):
    """A short run for the counter passes: three compressed-attention launches on this workload's
    shape (L' = L, random bf16) and three copies of a 1 GiB buffer (the calibration of known size),
    then each memory-bound stage once through its own ABI call on this workload's inputs, after a
    512 MiB read that evicts its inputs from the caches."""
    s = binding.shape_of(cfg)
    C = binding.capacity(cfg.L)
    g = torch.Generator(device=dev).manual_seed(0)
    Qh = torch.randn(cfg.Hq, C, cfg.d, device=dev, generator=g).to(torch.bfloat16)
    Kh = torch.randn(cfg.Hq, C, cfg.d, device=dev, generator=g).to(torch.bfloat16)
    Vht = torch.randn(cfg.Hq, cfg.d, C, device=dev, generator=g).to(torch.bfloat16)
    Oh = torch.empty_like(Qh)
    lp = torch.tensor([cfg.L], dtype=torch.int32, device=dev)
    for _ in range(3):
        binding.attn_causal(s, Qh, Kh, Vht, lp, Oh)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst, Vht
    inp = make_layer(cfg)
    Q, K, V, X = (inp[n].to(dev) for n in ("Q", "K", "V", "X"))
    del inp
    sws = binding.workspace(binding.stage_workspace_bytes(s), dev)
    s_h = torch.empty(cfg.Hq, cfg.L, dtype=torch.float32, device=dev)
    s_l = torch.empty(cfg.L, dtype=torch.float32, device=dev)
    kl = torch.zeros(2, dtype=torch.int32, device=dev)
    idx = torch.empty(cfg.Hq, cfg.L, dtype=torch.int32, device=dev)
    inv = torch.empty_like(idx)
    Vht = torch.empty(cfg.Hq, cfg.d, C, dtype=Q.dtype, device=dev)
    Y = torch.empty_like(X)
    flush = make_flush(dev)
    stages = [("score", lambda: binding.score(s, Q, K, s_h, s_l, sws)),
              ("budget", lambda: binding.budget(s, s_l, kl[0:1], kl[1:2], sws)),
              ("select", lambda: binding.select(s, s_h, kl[1:2], idx, inv, sws)),
              ("gather", lambda: binding.gather(s, Q, K, V, idx, kl[1:2], Qh, Kh, Vht)),
              ("scatter", lambda: binding.scatter_residual(s, Oh, idx, inv, kl[1:2], X, Y))]
    for _, fn in stages:
        evict(flush)
        fn()
        torch.cuda.synchronize()
    print(json.dumps({"traffic_probe": cfg.name, "copy_bytes": 1 << 30, "attention_launches": 3,
                      "stages": [n for n, _ in stages], "k": int(kl[0]), "L_keep": int(kl[1])}), flush=True)


def measured_stage_traffic(cfg):
    """Counted HBM bytes per call of each memory-bound stage from the committed counter summary, for
    the stages whose kernel source still hashes as it did when counted, on the counted shape only."""
    if not os.path.exists(STAGE_TRAFFIC_FILE):
        return {}
    kv = {}
    for line in open(STAGE_TRAFFIC_FILE):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if (kv.get("workload_L"), kv.get("workload_Hq"), kv.get("workload_d")) != (str(cfg.L), str(cfg.Hq), str(cfg.d)):
        return {}
    out = {}
    for st, srcs in STAGE_SOURCES.items():
        same = all(kv.get(f"source_sha256_16 {src}") == source_hash(os.path.join(ROOT, "token_sparse_attention_amd",
                                                                                "csrc", src)) for src in srcs)
        if same and f"{st}_hbm_bytes" in kv:
            out[st] = int(float(kv[f"{st}_hbm_bytes"]))
    return out


def sweep_evidence(cfg, s, Q, K, V, X, run_layer, stages, heads=None, rows_per_head=6, seed=0):
    """What the oracle leg needs to judge one supplementary line, from one untimed call of the same
    layer on a NaN-filled output: the keep count the layer reported, the selection the stage entry
    points make at the same setting (the layer is bitwise equal to its stages), Y at a few sampled
    compressed rows of every head, whether the tokens a head dropped kept X bit for bit, and whether
    every element of Y was written (no NaN left)."""
    dev = Q.device
    Y = torch.full_like(X, float("nan"))
    kLp = torch.zeros(2, dtype=torch.int32, device=dev)
    run_layer(Y, kLp)
    k, Lp = kLp.tolist()
    idx = stages()
    all_finite = bool(torch.isfinite(Y).all())
    sel = idx[:, :Lp].cpu().numpy().astype(np.int64)
    rng = np.random.default_rng(seed)
    heads = range(cfg.Hq) if heads is None else heads
    rows, unsel_ok = {}, True
    for h in heads:
        if Lp == 0:
            break
        r = {0, Lp - 1, min(1, Lp - 1)} | set(rng.integers(0, Lp, size=rows_per_head - 3).tolist())
        r = np.array(sorted(r), dtype=np.int64)
        tok = torch.as_tensor(sel[h][r], device=dev)
        rows[h] = (r, Y[tok, h].double().cpu().numpy())
        dropped = np.setdiff1d(np.arange(cfg.L), sel[h])
        if len(dropped):
            t = torch.as_tensor(rng.choice(dropped, min(32, len(dropped)), replace=False), device=dev)
            unsel_ok &= bool(torch.equal(Y[t, h], X[t, h]))
    return {"k_gpu": int(k), "Lp_gpu": int(Lp), "sel": sel, "rows": rows, "unselected_rows_equal_X": unsel_ok,
            "all_rows_written": all_finite}


def _stage_selection(cfg, s, Q, K, budget_fn):
    """The stage entry points' selection at shape s: score, then budget_fn(s_l, kl), then select."""
    dev = Q.device
    sws = binding.workspace(binding.stage_workspace_bytes(s), dev)
    s_h = torch.empty(cfg.Hq, cfg.L, dtype=torch.float32, device=dev)
    s_l = torch.empty(cfg.L, dtype=torch.float32, device=dev)
    kl = torch.zeros(2, dtype=torch.int32, device=dev)
    idx = torch.empty(cfg.Hq, cfg.L, dtype=torch.int32, device=dev)
    binding.score(s, Q, K, s_h, s_l, sws)
    budget_fn(s_l, kl, sws)
    binding.select(s, s_h, kl[1:2], idx, None, sws)
    return idx


def tau_sweep(cfg, Q, K, V, X, dense_ms, steps, warmup, stream):
    """The pages' sparsity regime at this workload's shapes: coverage thresholds that prune roughly
    17% / 54% / 75% of the (nearly uniform) layer score, layer time and speedup over dense, plus the
    evidence the oracle leg judges each line by."""
    out, pend = [], []
    for tau in (0.15, 0.50, 0.72):
        s = binding.shape(cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.q, tau, cfg.dtype)
        ws = binding.workspace(binding.layer_workspace_bytes(s), Q.device)
        kLp = torch.zeros(2, dtype=torch.int32, device=Q.device)
        Y = torch.empty_like(X)
        ms = timed(lambda: binding.layer(s, Q, K, V, X, Y, kLp, ws), steps, warmup, stream)
        k, Lp = kLp.tolist()
        del Y
        ev = sweep_evidence(cfg, s, Q, K, V, X, lambda Yn, kl: binding.layer(s, Q, K, V, X, Yn, kl, ws),
                            lambda: _stage_selection(cfg, s, Q, K, lambda sl, kl, w: binding.budget(
                                s, sl, kl[0:1], kl[1:2], w)), seed=int(tau * 100))
        out.append({"supplementary": True, "tau": tau, "k": k, "L_keep": Lp, "pruned_frac": round(k / cfg.L, 4),
                    "layer_ms": round(ms, 3),
                    "speedup_vs_dense": round(dense_ms / ms, 3)})
        pend.append((out[-1], dict(ev, kind="tau", tau=tau)))
        del ws
    return out, pend


def ratio_sweep(cfg, Q, K, V, X, dense_ms, steps, warmup, stream):
    """The ablation's fixed-ratio budget (s = 0.3 and 0.5 of the tokens pruned regardless of the
    scores) at this workload's shapes: layer time and speedup over dense, plus parity evidence."""
    s = binding.shape_of(cfg)
    ws = binding.workspace(binding.layer_workspace_bytes(s), Q.device)
    kLp = torch.zeros(2, dtype=torch.int32, device=Q.device)
    Y = torch.empty_like(X)
    out, pend = [], []
    for sp in (0.3, 0.5):
        ms = timed(lambda: binding.layer_ratio(s, sp, Q, K, V, X, Y, kLp, ws), steps, warmup, stream)
        k, Lp = kLp.tolist()
        ev = sweep_evidence(cfg, s, Q, K, V, X, lambda Yn, kl: binding.layer_ratio(s, sp, Q, K, V, X, Yn, kl, ws),
                            lambda: _stage_selection(cfg, s, Q, K, lambda sl, kl, w: binding.budget_ratio(
                                s, sp, kl[0:1], kl[1:2])), seed=int(sp * 100))
        out.append({"supplementary": True, "sparsity": sp, "k": k, "L_keep": Lp, "layer_ms": round(ms, 3),
                    "speedup_vs_dense": round(dense_ms / ms, 3)})
        pend.append((out[-1], dict(ev, kind="ratio", sparsity=sp)))
    del ws, Y
    return out, pend


BLOCK_PARITY_HEADS = (0, 21)


def block_sparse_sweep(cfg, Q, K, V, X, dense_ms, steps, warmup, stream):
    """Block sparsity stacked on the token selection at this workload's shapes: for a coverage
    threshold tau (token budget) and a block coverage gamma, the share of causal key blocks kept,
    the layer time and the speedup over dense, plus parity evidence (the kept-block lists of two
    heads and sampled output rows of those heads)."""
    dev = Q.device
    out, pend = [], []
    for tau in (cfg.tau, 0.5):
        s = binding.shape(cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.q, tau, cfg.dtype)
        C, NB = binding.capacity(cfg.L), binding.block_count(cfg.L)
        sws = binding.workspace(binding.stage_workspace_bytes(s), dev)
        s_h = torch.empty(cfg.Hq, cfg.L, dtype=torch.float32, device=dev)
        s_l = torch.empty(cfg.L, dtype=torch.float32, device=dev)
        kl = torch.zeros(2, dtype=torch.int32, device=dev)
        idx = torch.empty(cfg.Hq, cfg.L, dtype=torch.int32, device=dev)
        binding.score(s, Q, K, s_h, s_l, sws)
        binding.budget(s, s_l, kl[0:1], kl[1:2], sws)
        binding.select(s, s_h, kl[1:2], idx, None, sws)
        Qh = torch.empty(cfg.Hq, C, cfg.d, dtype=Q.dtype, device=dev)
        Kh, Vht = torch.empty_like(Qh), torch.empty(cfg.Hq, cfg.d, C, dtype=Q.dtype, device=dev)
        binding.gather(s, Q, K, V, idx, kl[1:2], Qh, Kh, Vht)
        del sws, s_h, s_l, Vht
        Lp = int(kl[1])
        nb = -(-Lp // 128)
        blist = torch.empty(cfg.Hq, NB, NB, dtype=torch.int16, device=dev)
        bcnt = torch.empty(cfg.Hq, NB, dtype=torch.int32, device=dev)
        bws = binding.workspace(binding.block_select_workspace_bytes(s), dev)
        lws = binding.workspace(binding.layer_block_sparse_workspace_bytes(s), dev)
        Y = torch.empty_like(X)
        for gamma in (0.9, 0.5):
            binding.block_select(s, gamma, Qh, Kh, kl[1:2], blist, bcnt, bws)
            kept = int(bcnt[:, :nb].sum()) / (cfg.Hq * nb * (nb + 1) / 2)
            ms = timed(lambda: binding.layer_block_sparse(s, gamma, Q, K, V, X, Y, None, lws), steps, warmup, stream)
            ev = sweep_evidence(cfg, s, Q, K, V, X,
                                lambda Yn, k2: binding.layer_block_sparse(s, gamma, Q, K, V, X, Yn, k2, lws),
                                lambda: idx, heads=BLOCK_PARITY_HEADS, rows_per_head=16, seed=int(gamma * 10))
            lists = {h: [blist[h, I, :int(bcnt[h, I])].cpu().numpy().astype(np.int64) for I in range(nb)]
                     for h in BLOCK_PARITY_HEADS}
            out.append({"supplementary": True, "tau": tau, "gamma": gamma, "L_keep": Lp,
                        "kept_block_frac": round(kept, 4),
                        "layer_ms": round(ms, 3), "speedup_vs_dense": round(dense_ms / ms, 3)})
            pend.append((out[-1], dict(ev, kind="block", tau=tau, gamma=gamma, block_lists=lists)))
        del Qh, Kh, blist, bcnt, bws, lws, Y, idx
    return out, pend


VARLEN_LENGTHS = [32768, 24576, 16384, 16384, 8192, 8192, 4096, 4096]


def varlen_batch(steps, warmup, stream, dev):
    """A ragged batch (8 samples of 4K-32K tokens, the 32K workload's recipe, one independent draw
    per sample): the batched layer with one attention launch over every sample's keep count, the
    same samples one tsa_layer call after another, and the batched dense baseline."""
    cfg = WORKLOADS[3]
    b = make_batch(cfg, VARLEN_LENGTHS)
    cu = [int(v) for v in b["cu_seqlens"]]
    Q, K, V, X = (b[n].to(dev) for n in ("Q", "K", "V", "X"))
    out = {"supplementary": True, "workload": f"varlen batch of {len(cu) - 1} ({cfg.name} recipe)",
           "lengths": VARLEN_LENGTHS,
           "tokens": cu[-1]}
    for tau in (cfg.tau, 0.5):
        s = binding.shape(cu[-1], cfg.Hq, cfg.Hkv, cfg.d, cfg.q, tau, cfg.dtype)
        ws = binding.workspace(binding.layer_varlen_workspace_bytes(s, cu), dev)
        kLp = torch.zeros(len(cu) - 1, 2, dtype=torch.int32, device=dev)
        Y = torch.empty_like(X)
        ms = timed(lambda: binding.layer_varlen(s, cu, Q, K, V, X, Y, kLp, ws), steps, warmup, stream)
        del ws
        per = []
        for i in range(len(cu) - 1):
            sb = binding.shape(cu[i + 1] - cu[i], cfg.Hq, cfg.Hkv, cfg.d, cfg.q, tau, cfg.dtype)
            r = slice(cu[i], cu[i + 1])
            per.append((sb, Q[r], K[r], V[r], X[r], Y[r], binding.workspace(binding.layer_workspace_bytes(sb), dev)))

        def one_by_one():
            for sb, q_, k_, v_, x_, y_, w_ in per:
                binding.layer(sb, q_, k_, v_, x_, y_, None, w_)
        ms_seq = timed(one_by_one, steps, warmup, stream)
        del per
        out[f"tau_{tau}"] = {"keep_counts": [int(v) for v in kLp[:, 1].tolist()], "layer_varlen_ms": round(ms, 3),
                             "per_sample_layers_ms": round(ms_seq, 3),
                             "tokens_per_s": round(cu[-1] / (ms * 1e-3), 1)}
    s = binding.shape(cu[-1], cfg.Hq, cfg.Hkv, cfg.d, cfg.q, cfg.tau, cfg.dtype)
    dws = binding.workspace(binding.dense_varlen_workspace_bytes(s, cu), dev)
    Yd = torch.empty_like(X)
    dms = timed(lambda: binding.dense_attn_causal_varlen(s, cu, Q, K, V, X, Yd, dws), steps, warmup, stream)
    out["dense_varlen_ms"] = round(dms, 3)
    for tau in (cfg.tau, 0.5):
        out[f"tau_{tau}"]["speedup_vs_dense"] = round(dms / out[f"tau_{tau}"]["layer_varlen_ms"], 3)
    return out


def varlen_trace(dev, calls=5):
    """A short run for a kernel trace of the batched layer: the varlen batch above at the 32K
    workload's tau, one warm-up call, then `calls` calls of tsa_layer_varlen."""
    cfg = WORKLOADS[3]
    b = make_batch(cfg, VARLEN_LENGTHS)
    cu = [int(v) for v in b["cu_seqlens"]]
    Q, K, V, X = (b[n].to(dev) for n in ("Q", "K", "V", "X"))
    del b
    s = binding.shape(cu[-1], cfg.Hq, cfg.Hkv, cfg.d, cfg.q, cfg.tau, cfg.dtype)
    ws = binding.workspace(binding.layer_varlen_workspace_bytes(s, cu), dev)
    kLp = torch.zeros(len(cu) - 1, 2, dtype=torch.int32, device=dev)
    Y = torch.empty_like(X)
    for _ in range(calls + 1):
        binding.layer_varlen(s, cu, Q, K, V, X, Y, kLp, ws)
    torch.cuda.synchronize()
    progress(f"varlen trace: {calls + 1} calls of tsa_layer_varlen, keep counts {kLp[:, 1].tolist()}")


def measure_workload(cfg, Q, K, V, X, steps, warmup, stream, sample_clocks=False):
    """Everything timed on one workload with inputs resident in HBM: the whole layer and the dense
    baseline alternately step by step, then every stage through its own ABI call (memory-bound
    stages with a cold last-level cache, the attention in steady state).  Returns the record and
    the tensors a later parity check needs (Y of the layer, the stage call's selection)."""
    dev = Q.device
    s = binding.shape_of(cfg)
    C = binding.capacity(cfg.L)
    ws = binding.workspace(binding.layer_workspace_bytes(s), dev)
    kLp = torch.zeros(2, dtype=torch.int32, device=dev)
    Y = torch.empty_like(X)
    dws = binding.workspace(binding.dense_workspace_bytes(s), dev)
    Yd = torch.empty_like(X)
    sampler = ClockSampler(delay=1.0).start() if sample_clocks else None   # the loop runs for seconds
    tl, td = timed_pair(lambda: binding.layer(s, Q, K, V, X, Y, kLp, ws),
                        lambda: binding.dense_attn_causal(s, Q, K, V, X, Yd, dws), steps, warmup, stream)
    clocks = sampler.result() if sampler else None
    layer_ms, dense_ms = float(np.mean(tl)), float(np.mean(td))
    k, Lp = kLp.tolist()
    del dws, Yd, ws

    sws = binding.workspace(binding.stage_workspace_bytes(s), dev)
    s_h = torch.empty(cfg.Hq, cfg.L, dtype=torch.float32, device=dev)
    s_l = torch.empty(cfg.L, dtype=torch.float32, device=dev)
    kl = torch.zeros(2, dtype=torch.int32, device=dev)
    idx = torch.empty(cfg.Hq, cfg.L, dtype=torch.int32, device=dev)
    inv = torch.empty(cfg.Hq, cfg.L, dtype=torch.int32, device=dev)
    Qh = torch.empty(cfg.Hq, C, cfg.d, dtype=Q.dtype, device=dev)
    Kh = torch.empty_like(Qh)
    Vht = torch.empty(cfg.Hq, cfg.d, C, dtype=Q.dtype, device=dev)
    Oh = torch.empty_like(Qh)
    Ys = torch.empty_like(X)
    flush = make_flush(dev)
    calls = {}
    calls["score"] = timed_cold(lambda: binding.score(s, Q, K, s_h, s_l, sws), steps, 1, stream, flush)
    calls["budget"] = timed_cold(lambda: binding.budget(s, s_l, kl[0:1], kl[1:2], sws), steps, 1, stream, flush)
    calls["select"] = timed_cold(lambda: binding.select(s, s_h, kl[1:2], idx, inv, sws), steps, 1, stream, flush)
    calls["gather"] = timed_cold(lambda: binding.gather(s, Q, K, V, idx, kl[1:2], Qh, Kh, Vht), steps, 1, stream,
                                 flush)
    att_ms = timed(lambda: binding.attn_causal(s, Qh, Kh, Vht, kl[1:2], Oh), steps, 1, stream)
    calls["scatter"] = timed_cold(lambda: binding.scatter_residual(s, Oh, idx, inv, kl[1:2], X, Ys), steps, 1,
                                  stream, flush)
    del flush, Qh, Kh, Vht, Oh, Ys, sws, inv
    assert kl.tolist() == [k, Lp]
    sl = s_l.double().cpu().numpy()
    # rows of K/V actually read by the gather: the union of the selections of each KV group
    G = cfg.Hq // cfg.Hkv
    sel = idx[:, :Lp].cpu().numpy()
    union_rows = sum(len(np.unique(sel[g * G:(g + 1) * G])) for g in range(cfg.Hkv))
    alg = algorithmic(cfg, Lp, union_rows)

    stages = {}
    for name in ("score", "budget", "select", "gather", "scatter"):
        ms = float(np.median(calls[name]))
        rate = alg[name] / (ms * 1e-3) / 1e9
        stages[name] = {"ms": round(ms, 4), "ms_percentiles": pct(calls[name]), "algorithmic_bytes": int(alg[name]),
                        "GB_s": round(rate, 1), "hbm_frac": round(rate / HBM_PEAK_GBS, 4)}
    peak = BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else FP32_PEAK_TFLOPS
    frac_key = "mfma_frac" if cfg.dtype == "bf16" else "fp32_vector_frac"
    att_tf = alg["attn_flops"] / (att_ms * 1e-3) / 1e12
    stages["attention"] = {"ms": round(att_ms, 4), "algorithmic_flops": int(alg["attn_flops"]),
                           "TFLOP_s": round(att_tf, 1), frac_key: round(att_tf / peak, 4)}
    dense_tf = alg["dense_flops"] / (dense_ms * 1e-3) / 1e12
    rec = {
        "workload": cfg.name, "L": cfg.L, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d, "q": cfg.q, "tau": cfg.tau,
        "dtype": cfg.dtype, "seed": cfg.seed, "k": k, "L_keep": Lp,
        "s_l_min_times_L": round(float(sl.min()) * cfg.L, 4), "s_l_max_times_L": round(float(sl.max()) * cfg.L, 4),
        "layer_ms": round(layer_ms, 4), "layer_ms_percentiles": pct(tl),
        "dense_ms": round(dense_ms, 4), "dense_ms_percentiles": pct(td),
        "speedup_vs_dense": round(dense_ms / layer_ms, 4),
        "attention_only_speedup": round(dense_ms / att_ms, 4),
        "dense_TFLOP_s": round(dense_tf, 1), "dense_" + frac_key: round(dense_tf / peak, 4),
        "overhead_frac_of_attention": round((layer_ms - att_ms) / att_ms, 4),
        "stages": stages,
    }
    return rec, {"Y": Y, "idx": idx, "k": k, "Lp": Lp, "clocks": clocks, "att_tf": att_tf, "peak": peak}


CHAIN_PARITY_HEADS = (0, 13, 18, 31)


def chain_c5(steps, warmup, stream, dev, with_evidence=True):
    """The 8-layer attention-only chain at L = 256K (32/8 heads, d = 128, q = 64, tau = 0.002): the
    least-drifting half (layers 5-8, from the seeded drift values) run Token Sparse Attention, the
    others dense causal attention, and the residual X is carried from each layer to the next.  Each
    layer's inputs are drawn from the chain recipe just before it runs and are resident in HBM when
    it is timed.  For the speedup over an all-dense chain the dense attention is also timed on the
    sparse layers' inputs.  Before the chain runs, the coverage thresholds of the pages' sparsity
    regime are swept on layer 1's inputs at this shape.  Returns the chain record, the sweep lines
    and, for the oracle leg, the evidence of every sparse line."""
    cfg = WORKLOADS[5]
    sparse = select_sparse_layers(chain_drift_values(cfg))
    s = binding.shape_of(cfg)
    ws = binding.workspace(binding.layer_workspace_bytes(s), dev)
    dws = binding.workspace(binding.dense_workspace_bytes(s), dev)
    kLp = torch.zeros(2, dtype=torch.int32, device=dev)
    X = Y = Yd = None
    layers, sweep, pend = [], [], []
    t_start = time.perf_counter()
    for layer_id, inp in iter_chain(cfg):
        Q, K, V = (inp[n].to(dev) for n in ("Q", "K", "V"))
        if X is None:
            X = inp["X"].to(dev)
            Y, Yd = torch.empty_like(X), torch.empty_like(X)
        keep = {n: inp[n] for n in ("Q", "K", "V")} if with_evidence else None
        del inp
        if layer_id == 1:
            X_in1 = X.cpu() if with_evidence else None
            for tau in (0.15, 0.50, 0.72):
                st = binding.shape(cfg.L, cfg.Hq, cfg.Hkv, cfg.d, cfg.q, tau, cfg.dtype)
                tl, td = timed_pair(lambda: binding.layer(st, Q, K, V, X, Y, kLp, ws),
                                    lambda: binding.dense_attn_causal(st, Q, K, V, X, Yd, dws), max(2, steps // 2), 1,
                                    stream)
                k, Lp = kLp.tolist()
                line = {"supplementary": True, "tau": tau, "k": k, "L_keep": Lp, "pruned_frac": round(k / cfg.L, 4),
                        "layer_ms": round(float(np.median(tl)), 3), "dense_ms": round(float(np.median(td)), 3),
                        "speedup_vs_dense": round(float(np.median(td)) / float(np.median(tl)), 3)}
                sweep.append(line)
                if with_evidence:
                    ev = sweep_evidence(cfg, st, Q, K, V, X, lambda Yn, kl: binding.layer(st, Q, K, V, X, Yn, kl, ws),
                                        lambda: _stage_selection(cfg, st, Q, K, lambda sl, kl, w: binding.budget(
                                            st, sl, kl[0:1], kl[1:2], w)), heads=CHAIN_PARITY_HEADS,
                                        rows_per_head=6, seed=int(tau * 100))
                    pend.append((line, dict(ev, kind="tau", tau=tau, inputs=keep, X_in=X_in1)))
            progress("c5 tau sweep done")
        rec = {"layer": layer_id, "kind": "sparse" if layer_id in sparse else "dense"}
        if layer_id in sparse:
            tl, td = timed_pair(lambda: binding.layer(s, Q, K, V, X, Y, kLp, ws),
                                lambda: binding.dense_attn_causal(s, Q, K, V, X, Yd, dws), steps, warmup, stream)
            k, Lp = kLp.tolist()
            rec.update({"ms": round(float(np.median(tl)), 3), "ms_percentiles": pct(tl), "k": k, "L_keep": Lp,
                        "dense_ms_same_inputs": round(float(np.median(td)), 3)})
            if with_evidence:
                X_in = X.cpu()
                ev = sweep_evidence(cfg, s, Q, K, V, X, lambda Yn, kl: binding.layer(s, Q, K, V, X, Yn, kl, ws),
                                    lambda: _stage_selection(cfg, s, Q, K, lambda sl, kl, w: binding.budget(
                                        s, sl, kl[0:1], kl[1:2], w)), heads=CHAIN_PARITY_HEADS, rows_per_head=6,
                                    seed=layer_id)
                pend.append((rec, dict(ev, kind="tau", tau=cfg.tau, inputs=keep, X_in=X_in)))
            binding.layer(s, Q, K, V, X, Y, kLp, ws)          # the chain's own pass: Y = this layer's output
        else:
            td = timed_calls(lambda: binding.dense_attn_causal(s, Q, K, V, X, Y, dws), steps, warmup, stream)
            rec.update({"ms": round(float(np.median(td)), 3), "ms_percentiles": pct(td),
                        "dense_ms_same_inputs": round(float(np.median(td)), 3)})
        X, Y = Y, X                                            # the residual stream carried to the next layer
        layers.append(rec)
        progress(f"c5 chain layer {layer_id} ({rec['kind']}): {rec['ms']:.1f} ms")
        del Q, K, V, keep
    total = sum(r["ms"] for r in layers)
    dense_total = sum(r["dense_ms_same_inputs"] for r in layers)
    out = {"workload": cfg.name, "sparse_layers": sparse, "layers": layers, "total_ms": round(total, 3),
           "all_dense_total_ms": round(dense_total, 3), "speedup_vs_all_dense": round(dense_total / total, 4),
           "wall_s": round(time.perf_counter() - t_start, 1)}
    return out, sweep, pend


def graph_replay(steps, warmup, stream, dev):
    """The fused layer captured once in a HIP graph and replayed, against the same call made
    eagerly, on the shorter workloads (where ~21 small launches weigh most) and on the varlen batch.
    The library allocates nothing and never syncs, so one capture serves every replay; the replayed
    output is checked bitwise against the eager one."""

    def cap(fn):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        torch.cuda.synchronize()
        return g

    out = []
    for n in (2, 3):
        cfg = WORKLOADS[n]
        inp = make_layer(cfg)
        Q, K, V, X = (inp[m].to(dev) for m in ("Q", "K", "V", "X"))
        s = binding.shape_of(cfg)
        ws = binding.workspace(binding.layer_workspace_bytes(s), dev)
        Ye, Yg = torch.empty_like(X), torch.empty_like(X)
        eager = timed(lambda: binding.layer(s, Q, K, V, X, Ye, None, ws), steps, warmup, stream)
        g = cap(lambda: binding.layer(s, Q, K, V, X, Yg, None, ws))
        replay = timed(g.replay, steps, warmup, stream)
        out.append({"supplementary": True, "workload": cfg.name, "eager_ms": round(eager, 4),
                    "graph_replay_ms": round(replay, 4),
                    "bitwise_equal": bool(torch.equal(Ye, Yg))})
        del g, Q, K, V, X, ws, Ye, Yg
    cfg = WORKLOADS[3]
    b = make_batch(cfg, VARLEN_LENGTHS)
    cu = [int(v) for v in b["cu_seqlens"]]
    Q, K, V, X = (b[m].to(dev) for m in ("Q", "K", "V", "X"))
    s = binding.shape(cu[-1], cfg.Hq, cfg.Hkv, cfg.d, cfg.q, cfg.tau, cfg.dtype)
    ws = binding.workspace(binding.layer_varlen_workspace_bytes(s, cu), dev)
    Ye, Yg = torch.empty_like(X), torch.empty_like(X)
    eager = timed(lambda: binding.layer_varlen(s, cu, Q, K, V, X, Ye, None, ws), steps, warmup, stream)
    g = cap(lambda: binding.layer_varlen(s, cu, Q, K, V, X, Yg, None, ws))
    replay = timed(g.replay, steps, warmup, stream)
    out.append({"supplementary": True, "workload": f"varlen batch of {len(cu) - 1} ({cfg.name} recipe)",
                "eager_ms": round(eager, 4),
                "graph_replay_ms": round(replay, 4), "bitwise_equal": bool(torch.equal(Ye, Yg))})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", type=int, default=4, help="workload number (4 = L=128K headline)")
    ap.add_argument("--no-tau-sweep", action="store_true")
    ap.add_argument("--no-varlen", action="store_true")
    ap.add_argument("--no-block-sparse", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay line")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload records of the other workloads")
    ap.add_argument("--no-chain", action="store_true", help="skip the 8-layer 256K chain (and its tau sweep)")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="only run the short kernel sequence used for the rocprofv3 counter passes")
    ap.add_argument("--varlen-trace", action="store_true",
                    help="only run the varlen batch's layer a few times, for a rocprofv3 kernel trace")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the layer runs on one MI355X (no multi-GPU path is built); "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X", file=sys.stderr)
        sys.exit(2)

    cfg = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    binding.lib()
    if args.traffic_probe:
        traffic_probe(cfg, dev)
        return
    if args.varlen_trace:
        varlen_trace(dev)
        return
    t_gen = time.perf_counter()
    inp = make_layer(cfg)
    t_gen = time.perf_counter() - t_gen
    Q, K, V, X = (inp[n].to(dev) for n in ("Q", "K", "V", "X"))
    stream = torch.cuda.current_stream()

    progress(f"inputs of {cfg.name} drawn in {t_gen:.1f} s")
    rec, keep = measure_workload(cfg, Q, K, V, X, args.steps, args.warmup, stream, sample_clocks=True)
    progress(f"layer {rec['layer_ms']:.3f} ms, dense {rec['dense_ms']:.3f} ms, stages timed")
    layer_ms, dense_ms = rec["layer_ms"], rec["dense_ms"]
    frac_key = "mfma_frac" if cfg.dtype == "bf16" else "fp32_vector_frac"
    out = {
        "metric": METRIC,
        "value": round(layer_ms, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(layer_ms, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "L": cfg.L, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d, "q": cfg.q,
                   "tau": cfg.tau, "seed": cfg.seed, "k": keep["k"], "L_keep": keep["Lp"],
                   "parallelism": "single GPU"},
    }
    for key in ("layer_ms_percentiles", "dense_ms", "dense_ms_percentiles", "speedup_vs_dense",
                "attention_only_speedup", "dense_TFLOP_s", "dense_" + frac_key, "overhead_frac_of_attention",
                "s_l_min_times_L", "s_l_max_times_L", "stages"):
        out[key] = rec[key]
    for st, nbytes in measured_stage_traffic(cfg).items():
        out["stages"][st]["counted_hbm_bytes"] = nbytes
        out["stages"][st]["counted_over_algorithmic"] = round(nbytes / out["stages"][st]["algorithmic_bytes"], 3)
    out["roofline"] = {"bound": "mfma" if cfg.dtype == "bf16" else "alu",
                       "kernel": f"compressed causal attention ({cfg.dtype})",
                       "achieved": round(keep["att_tf"], 1), "peak": keep["peak"], "unit": "TFLOP/s",
                       "frac": round(keep["att_tf"] / keep["peak"], 4), "traffic": measured_traffic(cfg),
                       "counters": measured_counters(cfg)}
    out["input_gen_s"] = round(t_gen, 1)
    sub = max(2, args.steps // 2)
    pending = []
    if not args.no_tau_sweep:
        out["supplementary_tau_sweep"], p1 = tau_sweep(cfg, Q, K, V, X, dense_ms, sub, 1, stream)
        out["supplementary_fixed_ratio"], p2 = ratio_sweep(cfg, Q, K, V, X, dense_ms, sub, 1, stream)
        pending += p1 + p2
        progress("tau sweep and fixed ratio done")
    if not args.no_block_sparse:
        out["supplementary_block_sparse"], p3 = block_sparse_sweep(cfg, Q, K, V, X, dense_ms, sub, 1, stream)
        pending += p3
        progress("block sparsity done")
    out["gpu_clocks_during_layer_and_dense"] = keep["clocks"]
    out["hbm_practical"] = hbm_practical(dev)
    if not args.no_cpu_baseline:
        Yc, idxc = keep["Y"], keep["idx"]
        out["cpu_baseline"], out["parity_vs_oracle"], verdicts = cpu_baseline(
            cfg, inp, keep["k"], keep["Lp"], Yc, idxc, pending=[ev for _, ev in pending])
        for (line, _), v in zip(pending, verdicts):
            line["parity_vs_oracle"] = v
        progress(f"oracle timed; parity pass = {out['parity_vs_oracle']['pass']}; supplementary lines passing: "
                 f"{sum(v['pass'] for v in verdicts)} of {len(verdicts)}")
    # a supplementary speedup is reported only for a line whose output passed the oracle check
    for line, _ in pending:
        if not line.get("parity_vs_oracle", {}).get("pass", False):
            line["speedup_vs_dense_withheld"] = line.pop("speedup_vs_dense")
    del Q, K, V, X, inp, keep
    torch.cuda.empty_cache()
    if not args.no_varlen:
        out["supplementary_varlen"] = varlen_batch(sub, 1, stream, dev)
        progress("varlen batch done")
    if not args.no_graph:
        out["supplementary_graph"] = graph_replay(sub, 1, stream, dev)
        progress("graph replay done")
    if not args.no_configs:
        recs = []
        for n in sorted(WORKLOADS):
            if n == args.workload or WORKLOADS[n].layers > 1:      # the chain has a record of its own
                continue
            c = WORKLOADS[n]
            t0 = time.perf_counter()
            part = make_layer(c)
            Qc, Kc, Vc, Xc = (part[m].to(dev) for m in ("Q", "K", "V", "X"))
            del part
            r, _ = measure_workload(c, Qc, Kc, Vc, Xc, 3 if c.L > 131072 else sub, 1, stream)
            r["wall_s"] = round(time.perf_counter() - t0, 1)
            recs.append(r)
            progress(f"{c.name}: layer {r['layer_ms']:.3f} ms, dense {r['dense_ms']:.3f} ms")
            del Qc, Kc, Vc, Xc, _
            torch.cuda.empty_cache()
        out["supplementary_configs"] = recs
    if not args.no_chain and args.workload != 5:
        evidence = not args.no_cpu_baseline
        out["supplementary_chain_c5"], sweep5, pend5 = chain_c5(3, 1, stream, dev, with_evidence=evidence)
        out["supplementary_tau_sweep_c5"] = sweep5
        if evidence:
            for (line, _), v in zip(pend5, chain_verdicts(WORKLOADS[5], pend5)):
                line["parity_vs_oracle"] = v
            progress(f"c5 chain and sweep judged: {sum(v['parity_vs_oracle']['pass'] for v, _ in pend5)} of "
                     f"{len(pend5)} lines pass")
        for line, _ in pend5:
            if not line.get("parity_vs_oracle", {}).get("pass", False):
                key = "speedup_vs_dense" if "speedup_vs_dense" in line else None
                if key:
                    line["speedup_vs_dense_withheld"] = line.pop(key)
        del pend5
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
