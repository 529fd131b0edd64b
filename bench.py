"""Benchmark of the hybrid-mask attention hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input resident in HBM:
  ha_classify_tiles  (segment table -> row limits + tile ranges)
  ha_qk_prologue     (q/k RMSNorm + 3-axis interleaved mRoPE)
  ha_attn_fwd_planned (hybrid-mask GQA flash attention)
on the HiDream-O1-style 2048^2 text-to-image workload: batch 2 (CFG cond/uncond), 258
causal tokens (256 text + 2 markers) then 4096 generation patches (64x64 grid) with full
attention; GQA 32/8, head dim 128, bf16.

Metric: useful (mask-aware) attention TFLOP/s, 4 * d * Hq * (allowed query-key pairs) per
pass, over the whole step. In the K timed steps, HIP events on the launch stream bracket
only the attention launch, which gives that kernel's own duration for the MFMA roofline. A
second pass of K steps, untimed as a whole, brackets each kernel and gives the classifier's
and the prologue's (each record leaves a few microseconds between two launches, so the
timed steps carry only the two the roofline needs). Three copies of the inputs are cycled so the 256 MB
Infinity Cache cannot serve a step from the previous one.

"qkv_projection" times the step before the path, the layer's QKV projection with the
prologue in its epilogue (ha_qkv_prologue), against three hipBLASLt projections plus
ha_qk_prologue.

"training_layouts" times ha_attn_fwd_lse and ha_attn_bwd whole on the multi-image
training sequence (Gen Images hidden from the tokens after them) and on the same shape with
plain image segments.

"prefix_step" times a denoising step that reuses the causal text prefix (its rotated q, k
and output rows) from an earlier step: the prologue and attention rows from the text end.

The training backward (ha_attn_bwd after ha_attn_fwd_lse) is timed on its own afterwards
and reported under "backward" (8 d FLOP per allowed pair and query head); it is not part
of the step.

"configs" times every other workload shape: the whole ha_attn_fwd call (classifier, split
plan, prologue, attention, merge) and, where the planned path takes the layout, the
attention kernel alone (ha_attn_fwd_planned), each call between HIP events.

"clocks" samples the GPU's core (sclk) and memory (mclk) clocks through amdsmi from a
thread while the step runs back to back for about a second ("clock_window"), and reports
the attention kernel's fraction of the bf16 peak at the measured core clock beside the
fraction of the published peak (which assumes 2.4 GHz).

"careful_pass" times the attention at the HunyuanImage layout when one KV group's scores
are shifted by about +86 log2 units (which sends its work items through the careful
re-referencing pass) against the same inputs unshifted.

    python bench.py [--steps K] [--warmup W] [--workload hd2048] [--no-cpu-baseline] [--no-backward]
                    [--no-prefix] [--no-training-layouts] [--no-qkv] [--no-configs] [--no-clocks]
                    [--no-careful]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

BF16_PEAK_TFLOPS = 256 * 4096 * 2.4e9 / 1e12   # 256 CU x 4096 bf16 FLOP/clk/CU x 2.4 GHz
HBM_PEAK_GBPS = 8000.0
METRIC = "hybrid-mask attention TFLOP/s (useful) and % bf16 MFMA peak, 1 MI355X"
ATTN_SRC = os.path.join(ROOT, "unified_text_pixel_amd", "csrc", "ha_attn_fwd.hip")
COUNTERS = os.path.join(ROOT, "profiles", "attn_hd2048_counters.json")


def kernel_sha() -> str:
    return hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()[:16]


def attn_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter runs, or None
    when the kernel source has changed since they were taken."""
    try:
        rec = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def allowed_pairs(segments: np.ndarray, S: int) -> int:
    """Allowed query-key pairs of one batch item, summed per segment in closed form:
    causal [a, a+L) -> sum (i+1); full -> L*S; image (generalized causal or Gen Image) ->
    L*(a+L); then each Gen Image's L keys are removed from the S - (a+L) rows after it."""
    n = 0
    for a, L, kind in segments:
        a, L = int(a), int(L)
        n += L * a + L * (L + 1) // 2 if kind == 0 else (L * S if kind == 1 else L * (a + L))
    for a, L, kind in segments:
        if kind == 3:
            n -= int(L) * (S - int(a) - int(L))
    return n


def cpu_baseline(w, x, target_s=12.0):
    """Time the oracle, as it is, on a bounded sample of the same workload: whole KV groups
    (their query heads) of batch item 0, then item 1, ..., until about target_s seconds are
    spent or the whole workload is done."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    import workloads as W

    n_threads = os.cpu_count() or 1
    limiter = threadpool_limits(limits=n_threads, user_api="blas")  # every host core, stated
    group = w.n_q_heads // w.n_kv_heads
    flops, elapsed, done = 0.0, 0.0, []
    for b in range(w.batch):
        sub = W.Inputs(workload=w.replace(batch=1), q=x.q[b:b + 1], k=x.k[b:b + 1],
                       v=x.v[b:b + 1], q_bits=None, k_bits=None, v_bits=None, w_q=x.w_q,
                       w_k=x.w_k, positions=x.positions[b:b + 1],
                       segments=x.segments[b:b + 1])
        pairs = allowed_pairs(x.segments[b], w.seq_len)
        heads = 0
        while heads < w.n_q_heads:
            if done and elapsed + elapsed / len(done) > target_s:
                break
            t0 = time.perf_counter()
            oracle.hot_path(sub, heads=range(heads, heads + group))
            elapsed += time.perf_counter() - t0
            flops += 4.0 * w.head_dim * group * pairs
            done.append((b, heads))
            heads += group
        if heads < w.n_q_heads:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] + [1])
    limiter.restore_original_limits()
    per_item = {}
    for b, h in done:
        per_item[b] = per_item.get(b, 0) + group
    what = ", ".join(f"item {b}: {n} of {w.n_q_heads} query heads" for b, n in per_item.items())
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "blas_threads_set": n_threads,
            "sample": f"{what}; whole path per head group (norm, mRoPE, explicit mask, fp64 "
                      f"attention), {elapsed:.1f} s; BLAS threads set to os.cpu_count()={n_threads}"}


def prefix_leg(w, x, sets, desc, pro, stream, step, warmup, steps):
    """A denoising step that reuses the causal text prefix: the prologue from the text end
    (ha_qk_prologue_from) and the attention rows from the text end (ha_attn_fwd_planned_from)
    over buffers a whole step filled; the tile plan is the same every step. Timed like the
    whole step: the steps back to back between two events, then again with events around
    each call for the breakdown."""
    import torch
    from unified_text_pixel_amd import binding as B
    seg = x.segments[0]
    p = int(seg[0][1]) if int(seg[0][2]) == 0 and int(seg[0][0]) == 0 else 0
    for s in sets:
        step(s)

    def run(s, ev=None):
        if ev:
            ev[0].record(stream)
        B.ha_qk_prologue_from(desc, pro, s["q"], s["k"], s["qr"], s["kr"], p, stream)
        if ev:
            ev[1].record(stream)
        B.ha_attn_fwd_planned_from(desc, s["qr"], s["kr"], s["v"], s["lim"], s["ranges"], s["out"], p,
                                   stream)
        if ev:
            ev[2].record(stream)

    for i in range(warmup):
        run(sets[i % len(sets)])
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        run(sets[i % len(sets)])
    t1.record(stream)
    torch.cuda.synchronize()
    for i in range(steps):
        run(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    return {"begin": p, "ms_per_step": t0.elapsed_time(t1) / steps,
            "prologue_ms": float(np.mean([e[0].elapsed_time(e[1]) for e in evs])),
            "attn_ms": float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))}


def qkv_leg(w, x, dev, stream, warmup, steps, hidden=4096):
    """The step before the path: the layer's QKV projection (hidden 4096 -> (Hq + 2 Hkv) d)
    with the prologue in its epilogue (ha_qkv_prologue), against the unfused route: three
    torch linear calls (hipBLASLt) into contiguous q, k, v, then ha_qk_prologue. Each call
    timed alone with HIP events on the launch stream, median of max(5, K/4) calls."""
    import torch
    import torch.nn.functional as Fn
    import workloads as W
    from unified_text_pixel_amd import api, binding as B
    from workloads.device import projection_to_device
    proj = W.generate_projection(w, hidden)
    xd, wd = projection_to_device(proj)
    desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, x.segments)
    cs = api.rope_table(w.rope_theta, w.head_dim, w.seq_len) if w.rope != "none" else None
    pro = B.PrologueDesc(w.rope, dev["positions"], cs, 0 if cs is None else cs.shape[0], dev["w_q"], dev["w_k"],
                         w.norm_eps, w.mrope_sections, q_out_scale=B.ha_q_prescale(desc))
    T, nq, nkv = w.batch * w.seq_len, w.n_q_heads * w.head_dim, w.n_kv_heads * w.head_dim
    q = torch.empty((w.batch, w.seq_len, w.n_q_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    k = torch.empty((w.batch, w.seq_len, w.n_kv_heads, w.head_dim), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    x2 = xd.view(T, hidden)
    wq, wk, wv = wd[:nq], wd[nq:nq + nkv], wd[nq + nkv:]

    def fused():
        B.ha_qkv_prologue(desc, pro, xd, hidden, wd, q, k, v, stream=stream)

    def gemms():
        torch.matmul(x2, wq.t(), out=q.view(T, nq))
        torch.matmul(x2, wk.t(), out=k.view(T, nkv))
        torch.matmul(x2, wv.t(), out=v.view(T, nkv))

    def prologue():
        B.ha_qk_prologue(desc, pro, q, k, qr, kr, stream=stream)

    # references: one hipBLASLt GEMM against the concatenated weight (all outputs at once),
    # and a plain device copy of as many bytes as the prologue reads (q and k) and writes,
    # three buffer pairs cycled as the step cycles its inputs (534 MB: past the 256 MB
    # Infinity Cache, so the copy runs from and to HBM like the prologue in the step)
    qkv = torch.empty((T, nq + 2 * nkv), dtype=torch.bfloat16, device="cuda")
    csrc = [torch.empty(q.numel() + k.numel(), dtype=torch.bfloat16, device="cuda") for _ in range(3)]
    cdst = [torch.empty_like(c) for c in csrc]
    ncopy = [0]

    def concat():
        torch.matmul(x2, wd.t(), out=qkv)

    def copy():
        i = ncopy[0] % 3
        ncopy[0] += 1
        cdst[i].copy_(csrc[i])

    def timed(fn):
        for _ in range(max(1, warmup // 2)):
            fn()
        n = max(5, steps // 4)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
        torch.cuda.synchronize()
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in ev])), n

    fms, n = timed(fused)
    gms, _ = timed(gemms)
    pms, _ = timed(prologue)
    cms, _ = timed(concat)
    yms, _ = timed(copy)
    flop = 2.0 * T * hidden * (nq + 2 * nkv)
    tf = flop / (fms / 1e3) / 1e12
    cbytes = 2 * csrc[0].numel() * csrc[0].element_size()
    return {"tokens": T, "hidden": hidden, "outputs": nq + 2 * nkv, "gflop": flop / 1e9,
            "fused_ms": fms, "fused_tflops": tf, "fused_frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
            "unfused_gemm_ms": gms, "unfused_gemm_tflops": flop / (gms / 1e3) / 1e12,
            "unfused_prologue_ms": pms, "unfused_total_ms": gms + pms,
            "concat_gemm_ms": cms, "concat_gemm_tflops": flop / (cms / 1e3) / 1e12,
            "copy_ref": {"bytes": cbytes, "ms": yms, "gbps": cbytes / (yms / 1e3) / 1e9,
                         "what": "torch copy_ of a bf16 tensor the size of q and k together (read + write), 3 buffer pairs cycled"},
            "calls": n}


def training_layout_leg(names, warmup, steps):
    """Training forward (ha_attn_fwd_lse) and backward (ha_attn_bwd) of whole layouts,
    each call timed alone with HIP events on the launch stream: the multi-image training
    sequence (Gen Images hidden from later tokens) beside the same shape with plain image
    segments. Useful FLOPs: 4 d per allowed pair and query head forward, 8 d backward."""
    import torch
    import workloads as W
    from unified_text_pixel_amd import api, binding as B
    from workloads.device import to_device
    stream = torch.cuda.current_stream()
    res = {}
    for name in names:
        w = W.get_config(name)
        x = W.generate(w)
        dev = to_device(x)
        desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, x.segments)
        cs = api.rope_table(w.rope_theta, w.head_dim, w.seq_len) if w.rope != "none" else None
        pro = B.PrologueDesc(w.rope, dev["positions"], cs, 0 if cs is None else cs.shape[0],
                             dev["w_q"], dev["w_k"], w.norm_eps, w.mrope_sections)
        ws = torch.empty(max(B.ha_attn_workspace_bytes(desc, pro), B.ha_attn_bwd_workspace_bytes(desc, pro)),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty_like(dev["q"])
        lse = torch.empty((w.batch, w.n_q_heads, w.seq_len), dtype=torch.float32, device="cuda")
        dout = torch.randn(dev["q"].shape, generator=torch.Generator(device="cuda").manual_seed(7),
                           device="cuda").to(torch.bfloat16)
        dq, dk, dv = torch.empty_like(dev["q"]), torch.empty_like(dev["k"]), torch.empty_like(dev["v"])
        dw = [torch.empty(w.head_dim, device="cuda") if w.qk_norm else None for _ in range(2)]

        def fwd():
            B.ha_attn_fwd_lse(desc, pro, dev["q"], dev["k"], dev["v"], out, lse, ws, stream=stream)

        def bwd():
            B.ha_attn_bwd(desc, pro, dev["q"], dev["k"], dev["v"], out, lse, dout, dq, dk, dv, dw[0], dw[1], ws,
                          stream=stream)

        def timed(fn, n):
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
            torch.cuda.synchronize()
            for e in ev:
                e[0].record(stream)
                fn()
                e[1].record(stream)
            torch.cuda.synchronize()
            return float(np.median([e[0].elapsed_time(e[1]) for e in ev]))

        for _ in range(max(1, warmup // 2)):
            fwd()
            bwd()
        n = max(5, steps // 4)
        fms, bms = timed(fwd, n), timed(bwd, n)
        pairs = sum(allowed_pairs(x.segments[b], w.seq_len) for b in range(w.batch))
        flop = 4.0 * w.head_dim * w.n_q_heads * pairs
        res[name] = {"segments": x.segments[0].tolist(), "allowed_pairs": pairs,
                     "fwd_lse_ms": fms, "fwd_tflops": flop / (fms / 1e3) / 1e12,
                     "bwd_ms": bms, "bwd_tflops": 2 * flop / (bms / 1e3) / 1e12, "calls": n}
    return res


def backward_leg(w, x, dev, useful_fwd, stream, warmup, steps, nsets):
    """Training backward (ha_attn_bwd: rebuilt prologue, dK/dV, dQ, rotary and RMSNorm
    backward) after a forward with lse, timed alone with HIP events on the launch stream.
    Algorithmic work: 8 d FLOP per allowed (query, key) pair and query head (dV, dP, dQ and
    dK products; the recomputed scores are not counted), twice the forward's."""
    import torch
    from unified_text_pixel_amd import api, binding as B
    desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, x.segments)
    cs = api.rope_table(w.rope_theta, w.head_dim, w.seq_len) if w.rope != "none" else None
    pro = B.PrologueDesc(w.rope, dev["positions"], cs, 0 if cs is None else cs.shape[0],
                         dev["w_q"], dev["w_k"], w.norm_eps, w.mrope_sections)
    ws = torch.empty(max(B.ha_attn_workspace_bytes(desc, pro), B.ha_attn_bwd_workspace_bytes(desc, pro)),
                     dtype=torch.uint8, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(5)
    sets = []
    for _ in range(nsets):
        o = {"q": dev["q"].clone(), "k": dev["k"].clone(), "v": dev["v"].clone(),
             "out": torch.empty_like(dev["q"]),
             "lse": torch.empty((w.batch, w.n_q_heads, w.seq_len), dtype=torch.float32, device="cuda"),
             "dout": torch.randn(dev["q"].shape, generator=gen, device="cuda").to(torch.bfloat16),
             "dq": torch.empty_like(dev["q"]), "dk": torch.empty_like(dev["k"]), "dv": torch.empty_like(dev["v"])}
        norm = w.qk_norm
        o["dwq"] = torch.empty(w.head_dim, device="cuda") if norm else None
        o["dwk"] = torch.empty(w.head_dim, device="cuda") if norm else None
        B.ha_attn_fwd_lse(desc, pro, o["q"], o["k"], o["v"], o["out"], o["lse"], ws, stream=stream)
        sets.append(o)

    def bwd(o):
        B.ha_attn_bwd(desc, pro, o["q"], o["k"], o["v"], o["out"], o["lse"], o["dout"], o["dq"], o["dk"],
                      o["dv"], o["dwq"], o["dwk"], ws, stream=stream)

    for i in range(max(1, warmup // 2)):
        bwd(sets[i % nsets])
    n = max(5, steps // 4)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[i][0].record(stream)
        bwd(sets[i % nsets])
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([e[0].elapsed_time(e[1]) for e in ev])
    flop = 2.0 * useful_fwd
    tf = flop / (float(np.median(ms)) / 1e3) / 1e12
    return {"ms": {"median": float(np.median(ms)), "p10": float(np.percentile(ms, 10)),
                   "p90": float(np.percentile(ms, 90))},
            "gflop": flop / 1e9, "flop_per_pair_head": 8 * w.head_dim,
            "tflops": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS, "calls": n}


class ClockSampler:
    """Polls the GPU's current core and memory clocks (MHz) through amdsmi from a thread, about
    every millisecond, between start() and stop(): the clock-info query and, every tenth poll,
    the metrics table's per-XCD current gfx clocks (mean over the XCDs). Records why when
    amdsmi is unavailable."""

    def __init__(self, interval_s=0.001):
        import threading
        self.interval = interval_s
        self.sclk, self.mclk, self.xcd_sclk, self.error = [], [], [], None
        self.metrics_error = None
        self._stop = threading.Event()
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self._smi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
            self._read()
        except Exception as e:  # noqa: BLE001  (no SMI access: the record says so)
            self.error = f"{type(e).__name__}: {e}"

    def _read(self):
        smi = self._smi
        g = smi.amdsmi_get_clock_info(self._h, smi.AmdSmiClkType.GFX)
        m = smi.amdsmi_get_clock_info(self._h, smi.AmdSmiClkType.MEM)
        return float(g["clk"]), float(m["clk"])

    def _read_xcds(self):
        """Mean of the metrics table's per-XCD current gfx clocks (entries amdsmi marks N/A or
        zero are left out); None when the table has none."""
        mt = self._smi.amdsmi_get_gpu_metrics_info(self._h)
        v = mt.get("current_gfxclks")
        vals = [float(x) for x in (v if isinstance(v, (list, tuple)) else [v]) if isinstance(x, (int, float)) and x > 0]
        return float(np.mean(vals)) if vals else None

    def _run(self):
        k = 0
        while not self._stop.is_set():
            try:
                g, m = self._read()
                self.sclk.append(g)
                self.mclk.append(m)
            except Exception as e:  # noqa: BLE001
                self.error = f"{type(e).__name__}: {e}"
                return
            if k % 10 == 0 and self.metrics_error is None:
                try:
                    x = self._read_xcds()
                    if x is not None:
                        self.xcd_sclk.append(x)
                except Exception as e:  # noqa: BLE001
                    self.metrics_error = f"{type(e).__name__}: {e}"
            k += 1
            time.sleep(self.interval)

    def start(self):
        import threading
        if self.error is None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()

    def stop(self):
        self._stop.set()
        if self._thread is not None:
            self._thread.join()

    def summary(self):
        def st(v):
            # "median" is taken over the active samples (at least half the highest reading):
            # some boards report an idle level for most polls while the kernels run
            if not v:
                return None
            a = np.array(v)
            act = a[a >= 0.5 * a.max()]
            return {"median": float(np.median(act)), "median_all": float(np.median(a)), "min": float(a.min()),
                    "max": float(a.max()), "samples": len(v), "active_samples": int(act.size)}
        return {"source": "amdsmi_get_clock_info (current clock, MHz)", "sclk_mhz": st(self.sclk),
                "mclk_mhz": st(self.mclk), "error": self.error,
                "xcd_sclk_mhz": st(self.xcd_sclk), "xcd_source": "amdsmi_get_gpu_metrics_info current_gfxclks (mean over XCDs)",
                "metrics_error": self.metrics_error}


def clock_window(step, sets, stream, useful, seconds=1.0):
    """The step back to back for about `seconds` with the clock sampler running; HIP events
    around every attention launch. Returns the clocks and the attention throughput of that
    window, with its fraction of the bf16 peak at the measured core clock."""
    import torch
    sampler = ClockSampler()
    probe = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step(sets[0], probe)
    torch.cuda.synchronize()
    per = max(time.perf_counter() - t0, 1e-4)
    n = int(min(5000, max(50, seconds / per)))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
    sampler.start()
    for i in range(n):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    sampler.stop()
    att = np.array([e[2].elapsed_time(e[3]) for e in evs])
    tf = useful / (float(att.mean()) / 1e3) / 1e12
    out = sampler.summary()
    out.update({"steps": n, "attn_kernel_ms": {"mean": float(att.mean()), "median": float(np.median(att))},
                "attn_tflops": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS})
    # the fraction at the measured clock, from the first reading that is plausible: a clock
    # under which the measured throughput would exceed the dense peak is not the clock the
    # kernel ran at, and neither is one that reads the same in every sample of a window of
    # back-to-back launches, during which the firmware moves the core clock with power and
    # temperature (some boards report a fixed level through these queries)
    for key in ("sclk_mhz", "xcd_sclk_mhz"):
        if out.get(key):
            peak = 256 * 4096 * out[key]["median"] * 1e6 / 1e12
            constant = out[key]["samples"] > 10 and out[key]["min"] == out[key]["max"]
            if tf <= peak and not constant:
                out["clock_used"] = key
                out["bf16_peak_at_measured_sclk_tflops"] = peak
                out["frac_at_measured_sclk"] = tf / peak
                break
            out.setdefault("implausible", []).append(key + (" (constant over the window)" if constant else " (above the dense peak)"))
    return out


def _timed_calls(fn, stream, n):
    import torch
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
    torch.cuda.synchronize()
    for i, e in enumerate(ev):
        e[0].record(stream)
        fn(i)
        e[1].record(stream)
    torch.cuda.synchronize()
    return np.array([e[0].elapsed_time(e[1]) for e in ev])


def configs_leg(names, warmup, steps):
    """Every workload shape besides the headline: the whole ha_attn_fwd call (classifier,
    split plan where the planner takes one, prologue, attention, merge), eager and replayed
    from a HIP graph, and, for layouts the
    planned path takes (no Gen Images), the attention kernel alone (ha_attn_fwd_planned after
    one classifier and prologue call). HIP events around each call on the launch stream;
    input sets cycled so that together they exceed the 256 MB Infinity Cache."""
    import torch
    import workloads as W
    from unified_text_pixel_amd import api, binding as B
    from workloads.device import to_device
    stream = torch.cuda.current_stream()
    all_cfg = dict(W.CONFIGS)
    all_cfg.update(W.page_shape_configs())
    res = {}
    for name in names:
        w = all_cfg[name]
        x = W.generate(w)
        dev = to_device(x)
        desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, x.segments)
        pdesc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, x.segments,
                           q_prescaled=1)
        cs = api.rope_table(w.rope_theta, w.head_dim, w.seq_len) if w.rope != "none" else None
        pro = B.PrologueDesc(w.rope, dev["positions"], cs, 0 if cs is None else cs.shape[0],
                             dev["w_q"], dev["w_k"], w.norm_eps, w.mrope_sections)
        ppro = B.PrologueDesc(w.rope, dev["positions"], cs, 0 if cs is None else cs.shape[0],
                              dev["w_q"], dev["w_k"], w.norm_eps, w.mrope_sections,
                              q_out_scale=B.ha_q_prescale(pdesc))
        nbytes = B.ha_attn_workspace_bytes(desc, pro)
        set_bytes = 3 * dev["q"].numel() * dev["q"].element_size() + 3 * dev["k"].numel() * dev["k"].element_size()
        nsets = int(min(6, max(1, -(-300e6 // set_bytes))))
        _, _, nq, _ = B.ha_tile_shape(desc)
        sets = []
        for _ in range(nsets):
            sets.append({"q": dev["q"].clone(), "k": dev["k"].clone(), "v": dev["v"].clone(),
                         "out": torch.empty_like(dev["q"]), "qr": torch.empty_like(dev["q"]),
                         "kr": torch.empty_like(dev["k"]),
                         "ws": torch.empty(max(256, nbytes), dtype=torch.uint8, device="cuda"),
                         "ranges": torch.empty((w.batch, nq, 2), dtype=torch.int32, device="cuda"),
                         "lim": torch.empty((w.batch, w.seq_len), dtype=torch.int32, device="cuda")})
        pairs = sum(allowed_pairs(x.segments[b], w.seq_len) for b in range(w.batch))
        useful = 4.0 * w.head_dim * w.n_q_heads * pairs

        def whole(i):
            s = sets[i % nsets]
            B.ha_attn_fwd(desc, pro, s["q"], s["k"], s["v"], s["out"], s["ws"], stream=stream)

        for i in range(max(2, warmup)):
            whole(i)
        n = max(10, steps // 2)
        ms = _timed_calls(whole, stream, n)
        r = {"description": w.description, "batch": w.batch, "seq_len": w.seq_len,
             "allowed_pairs": pairs, "useful_gflop": useful / 1e9, "sets": nsets,
             "fwd_ms": {"mean": float(ms.mean()), "median": float(np.median(ms))},
             "fwd_tflops": useful / (float(np.median(ms)) / 1e3) / 1e12,
             "split_plan": nbytes > B.ha_attn_workspace_bytes(
                 B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, x.segments,
                            split_parts=1), pro)}
        # the same call captured in a HIP graph per input set, replayed: the launch gaps go
        graphs = []
        for s in sets:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                B.ha_attn_fwd(desc, pro, s["q"], s["k"], s["v"], s["out"], s["ws"])
            graphs.append(g)

        def replay(i):
            graphs[i % nsets].replay()

        for i in range(max(2, warmup)):
            replay(i)
        gm = _timed_calls(replay, stream, n)
        r.update({"fwd_graph_ms": {"mean": float(gm.mean()), "median": float(np.median(gm))},
                  "fwd_graph_tflops": useful / (float(np.median(gm)) / 1e3) / 1e12})
        del graphs
        if not any(int(k) == 3 for k in x.segments[..., 2].ravel()):
            for s in sets:
                B.ha_classify_tiles(pdesc, None, s["ranges"], s["lim"], stream)
                B.ha_qk_prologue(pdesc, ppro, s["q"], s["k"], s["qr"], s["kr"], stream)

            def planned(i):
                s = sets[i % nsets]
                B.ha_attn_fwd_planned(pdesc, s["qr"], s["kr"], s["v"], s["lim"], s["ranges"], s["out"], stream)

            for i in range(max(2, warmup)):
                planned(i)
            am = _timed_calls(planned, stream, n)
            tf = useful / (float(am.mean()) / 1e3) / 1e12
            r.update({"attn_kernel_ms": {"mean": float(am.mean()), "median": float(np.median(am)),
                                         "p10": float(np.percentile(am, 10)), "p90": float(np.percentile(am, 90))},
                      "attn_tflops": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS})
        res[name] = r
        del sets
        torch.cuda.empty_cache()
    return res


def careful_leg(warmup, steps, shift=26.0, group=3):
    """The HunyuanImage layout with no rotation (so a shift is the same for every key of a
    row) and q/k unnormalised, as it is: clean inputs against inputs where query component 0
    of KV group `group`'s query heads and key component 0 of that group from key 300 on are
    raised by `shift`, which moves those rows' scores by about shift^2 * scale * log2(e) =
    +86 log2 units and sends the group's work items through the careful re-referencing pass.
    With the XCD-aware order that group's items all run on one XCD, so the kernel time is
    that XCD's time: the ratio of the two kernel times is about the careful pass's cost per
    affected work item."""
    import torch
    import workloads as W
    from unified_text_pixel_amd import binding as B
    from workloads.device import to_device
    stream = torch.cuda.current_stream()
    w = W.get_config("hunyuan").replace(rope="none")
    res = {"layout": "hunyuan segments, no rotation", "shift_log2": shift * shift / np.sqrt(w.head_dim) * np.log2(np.e),
           "kv_group": group}
    G = w.n_q_heads // w.n_kv_heads
    for label in ("clean", "shifted"):
        x = W.generate(w)
        if label == "shifted":
            x.q[:, :, group * G:(group + 1) * G, 0] += shift
            x.k[:, 300:, group, 0] += shift
            bits = W.f32_to_bf16_bits(x.q)
            x.q, x.q_bits = W.bf16_bits_to_f32(bits).reshape(x.q.shape), bits.reshape(x.q.shape)
            bits = W.f32_to_bf16_bits(x.k)
            x.k, x.k_bits = W.bf16_bits_to_f32(bits).reshape(x.k.shape), bits.reshape(x.k.shape)
        dev = to_device(x)
        desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, x.segments)
        _, _, nq, _ = B.ha_tile_shape(desc)
        ranges = torch.empty((w.batch, nq, 2), dtype=torch.int32, device="cuda")
        lim = torch.empty((w.batch, w.seq_len), dtype=torch.int32, device="cuda")
        B.ha_classify_tiles(desc, None, ranges, lim, stream)
        out = torch.empty_like(dev["q"])
        ws = torch.empty(max(256, B.ha_attn_workspace_bytes(desc, None)), dtype=torch.uint8, device="cuda")

        def planned(i):
            B.ha_attn_fwd_planned(desc, dev["q"], dev["k"], dev["v"], lim, ranges, out, stream)

        def whole(i):
            B.ha_attn_fwd(desc, None, dev["q"], dev["k"], dev["v"], out, ws, stream=stream)

        for i in range(max(2, warmup)):
            planned(i)
            whole(i)
        n = max(10, steps // 2)
        am, wm = _timed_calls(planned, stream, n), _timed_calls(whole, stream, n)
        res[label] = {"attn_kernel_ms": float(np.median(am)), "fwd_ms": float(np.median(wm))}
    res["kernel_ratio"] = res["shifted"]["attn_kernel_ms"] / res["clean"]["attn_kernel_ms"]
    res["fwd_ratio"] = res["shifted"]["fwd_ms"] / res["clean"]["fwd_ms"]
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="hd2048")
    ap.add_argument("--sets", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-prefix", action="store_true")
    ap.add_argument("--no-training-layouts", action="store_true")
    ap.add_argument("--no-qkv", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--no-clocks", action="store_true")
    ap.add_argument("--no-careful", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    from unified_text_pixel_amd import api, binding as B
    from workloads.device import to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    B.load_library()
    w = W.get_config(args.workload)
    print(f"bench: generating {w.name} inputs", file=sys.stderr, flush=True)
    x = W.generate(w)
    dev = to_device(x)
    # the prologue writes q prescaled by softmax scale * log2(e), which the attention
    # kernel then takes as is (q_prescaled = 1): the same path ha_attn_fwd runs
    desc = B.AttnDesc(w.batch, w.seq_len, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype,
                      x.segments, q_prescaled=1)
    cs = api.rope_table(w.rope_theta, w.head_dim, w.seq_len) if w.rope != "none" else None
    pro = B.PrologueDesc(w.rope, dev["positions"], cs, 0 if cs is None else cs.shape[0],
                         dev["w_q"], dev["w_k"], w.norm_eps, w.mrope_sections,
                         q_out_scale=B.ha_q_prescale(desc))
    bq, bk, nq, nk = B.ha_tile_shape(desc)
    sets = []
    for _ in range(args.sets):
        sets.append({
            "q": dev["q"].clone(), "k": dev["k"].clone(), "v": dev["v"].clone(),
            "qr": torch.empty_like(dev["q"]), "kr": torch.empty_like(dev["k"]),
            "out": torch.empty_like(dev["q"]),
            "ranges": torch.empty((w.batch, nq, 2), dtype=torch.int32, device="cuda"),
            "lim": torch.empty((w.batch, w.seq_len), dtype=torch.int32, device="cuda"),
        })
    stream = torch.cuda.current_stream()

    def step(s, ev=None, attn_only=False):
        if ev and not attn_only:
            ev[0].record(stream)
        B.ha_classify_tiles(desc, None, s["ranges"], s["lim"], stream)
        if ev and not attn_only:
            ev[1].record(stream)
        B.ha_qk_prologue(desc, pro, s["q"], s["k"], s["qr"], s["kr"], stream)
        if ev:
            ev[2].record(stream)
        B.ha_attn_fwd_planned(desc, s["qr"], s["kr"], s["v"], s["lim"], s["ranges"], s["out"],
                              stream)
        if ev:
            ev[3].record(stream)

    if args.copy_mib:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i], attn_only=True)
    t_end.record(stream)
    torch.cuda.synchronize()
    step_ms = t_start.elapsed_time(t_end) / args.steps
    att_ms = np.array([e[2].elapsed_time(e[3]) for e in evs])
    # the classifier's and the prologue's times: the same steps again, every kernel bracketed
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(sets[i % len(sets)], evs[i])
    torch.cuda.synchronize()
    cls_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    pro_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])

    pairs = sum(allowed_pairs(x.segments[b], w.seq_len) for b in range(w.batch))
    useful = 4.0 * w.head_dim * w.n_q_heads * pairs
    att_s = float(att_ms.mean()) / 1e3
    att_tflops = useful / att_s / 1e12
    elem = 2 if w.dtype == "bf16" else 4
    pro_bytes = 2.0 * elem * w.batch * w.seq_len * (w.n_q_heads + w.n_kv_heads) * w.head_dim
    pro_gbps = pro_bytes / (float(pro_ms.mean()) / 1e3) / 1e9
    traffic = attn_traffic()

    rec = {
        "metric": METRIC,
        "value": useful / (step_ms / 1e3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": step_ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.description}", "batch": w.batch,
                   "seq_len": w.seq_len, "segments": x.segments[0].tolist(),
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "rope": w.rope, "qk_norm": w.qk_norm, "allowed_pairs": pairs,
                   "useful_gflop_per_step": useful / 1e9, "tile": [bq, bk]},
        "attn_kernel_ms": {"mean": float(att_ms.mean()), "median": float(np.median(att_ms)),
                           "p10": float(np.percentile(att_ms, 10)),
                           "p90": float(np.percentile(att_ms, 90))},
        "attn_tflops": att_tflops,
        "pct_bf16_peak": 100.0 * att_tflops / BF16_PEAK_TFLOPS,
        "prologue_ms": float(pro_ms.mean()), "prologue_gbps": pro_gbps,
        "classify_ms": float(cls_ms.mean()),
        "roofline": {"bound": "mfma", "achieved": att_tflops, "peak": BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": att_tflops / BF16_PEAK_TFLOPS,
                     "traffic": traffic},
        "prologue_roofline": {"bound": "hbm", "achieved": pro_gbps, "peak": HBM_PEAK_GBPS,
                              "unit": "GB/s", "frac": pro_gbps / HBM_PEAK_GBPS},
        "attn_kernel_sha": kernel_sha(),
    }
    if not args.no_clocks:
        rec["clocks"] = clock_window(step, sets, stream, useful)
    if not args.no_prefix:
        rec["prefix_step"] = prefix_leg(w, x, sets, desc, pro, stream, step, args.warmup, args.steps)
    if not args.no_backward and w.dtype == "bf16":
        rec["backward"] = backward_leg(w, x, dev, useful, stream, args.warmup, args.steps, args.sets)
    if not args.no_qkv and w.head_dim == 128 and w.dtype == "bf16":
        rec["qkv_projection"] = qkv_leg(w, x, dev, stream, args.warmup, args.steps)
    if not args.no_training_layouts:
        rec["training_layouts"] = training_layout_leg(["hunyuan_multigen", "hunyuan"], args.warmup, args.steps)
    if not args.no_configs:
        names = [n for n in ("hd1024", "edit", "hunyuan", "hunyuan_multigen", "page1024", "page2048")
                 if n != w.name]
        print("bench: timing the other workload shapes", file=sys.stderr, flush=True)
        rec["configs"] = configs_leg(names, args.warmup, args.steps)
    if not args.no_careful:
        rec["careful_pass"] = careful_leg(args.warmup, args.steps)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(w, x)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
