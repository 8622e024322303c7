"""Benchmark of the fused attention forward on one MI355X.

python bench.py [--steps K] [--warmup W] [--config NAME] [--seq S] [--no-cpu]

One step is one pass of the hot path over resident synthetic inputs:
  * dense configs: one attn_fwd call (all heads, all q-blocks);
  * block-sparse: build the kept list, then attn_fwd_blocksparse;
  * quantised: quantise Q, K (INT8 per block) and V (FP8 per channel), build
    the kept list, then attn_fwd_qbsa.
Untimed steps first (a settling phase of --settle-s seconds, then the W
warm-up steps), then exactly K timed steps between two device
synchronisations; HIP events on the launch stream give the per-step times.
Prints one JSON line. The default workload is the dense B=1 N=40 S=8192 D=128
operator shape, on which the headline metric is quoted.

--copy-calibration BYTES runs a plain device copy of BYTES bytes (used to scale
the FETCH_SIZE / WRITE_SIZE counters of a counter run to bytes).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS (executed + dense-equiv), % MFMA peak, S=8K–64K"
PEAK_BF16 = 2500.0   # TFLOP/s, MI355X published dense bf16 and fp16 MFMA
PEAK_FP8 = 5000.0    # TFLOP/s (fp8) / TOP/s (int8), published dense
HBM_PEAK = 8000.0    # GB/s
KERNEL_SOURCES = {
    "dense": ["attn_fwd_kernel.h", "attn_fwd_bf16.hip", "qattn_internal.h"],
    "blocksparse": ["attn_fwd_kernel.h", "attn_fwd_bf16.hip", "quant.hip", "qattn_internal.h"],
    "qbsa": ["attn_qbsa.hip", "quant.hip", "qattn_internal.h"],
    "backward": ["attn_bwd.hip", "qattn_internal.h"],
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "quantized_attention_tiled_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def flop_counts(w):
    """(executed, useful, dense_equivalent) flop counts: 2 D flops per (q, k)
    pair for Q.K^T and again for P.V. Executed counts the (row, key) pairs of
    the tiles the kernel processes: whole kept 128-key blocks for block-sparse;
    for causal masks, the rows of each 128-row q-block (one workgroup) run over
    the keys up to the end of the 64-key tile that holds the diagonal of the
    q-block's last row."""
    D = w.D
    fpp = 2 * (D + w.v.shape[-1])  # flops per (q, k) pair: Q.K^T over D and P.V over Dv
    if w.layout == "TND":
        lens = np.diff(w.cu_seqlens_q)
        dense = useful = executed = 0
        for L in lens:
            L = int(L)
            dense += L * L
            if w.sparse_mode in (2, 3):          # Lq == Lkv here, so both causal modes coincide
                useful += L * (L + 1) // 2
                for r0 in range(0, L, 128):
                    r1 = min(L, r0 + 128)
                    executed += (r1 - r0) * min(L, ((r1 + 63) // 64) * 64)
            else:
                useful += L * L
                executed += L * L
        f = fpp * w.Nq
        return f * executed, f * useful, f * dense
    dense = w.B * w.Nq * w.Sq * w.Skv
    if w.keep is not None:
        blk = np.minimum(128, w.Skv - np.arange(w.keep.shape[3]) * 128)
        rows = np.minimum(128, w.Sq - np.arange(w.keep.shape[2]) * 128)
        per_row = (w.keep.astype(np.int64) * blk[None, None, None, :]).sum(axis=3)
        pairs = int((per_row * rows[None, None, :]).sum())
        return fpp * pairs, fpp * pairs, fpp * dense
    return fpp * dense, fpp * dense, fpp * dense


def algorithmic_bytes(w, kind):
    """Minimum HBM bytes of one step: read every input once, write every output once."""
    el = lambda a: int(np.prod(a.shape))  # noqa: E731
    ml = 2 * 4 * w.Nq * w.Sq * (w.B if w.layout == "BNSD" else 1)
    eo = el(w.q) // w.D * w.v.shape[-1]  # output elements (head dimension Dv)
    if kind == "dense":
        return 2 * (el(w.q) + el(w.k) + el(w.v)) + 2 * eo + ml
    if kind == "blocksparse":
        return 2 * (el(w.q) + el(w.k) + el(w.v)) + 2 * eo + ml + el(w.keep) + 4 * el(w.keep)
    # quantised: bf16 in, int8/fp8 codes out and read back, bf16 O
    return (2 * (el(w.q) + el(w.k) + el(w.v)) + (el(w.q) + el(w.k) + el(w.v)) * 2 + 2 * el(w.q) + ml
            + 5 * el(w.keep))


def run_cpu_baseline(w, kind, budget_s: float):
    """Time the oracle, as it stands, on a bounded sample of the same workload."""
    import oracle
    from workloads import bf16_bits_to_f32

    try:
        from threadpoolctl import threadpool_info
        cores = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = 1
    f64 = lambda x: bf16_bits_to_f32(x).astype(np.float64)  # noqa: E731
    D = w.D
    t0 = time.perf_counter()
    flops = 0
    done = 0
    # (head, q-block) pairs in head-major order, until the time budget is spent
    if kind == "dense" and w.layout == "BNSD":
        nqb = (w.Sq + 127) // 128
        h = -1
        while time.perf_counter() - t0 < budget_s and done < w.Nq * nqb:
            if done % nqb == 0:
                h += 1
                q0, k0, v0 = f64(w.q[0, h]), f64(w.k[0, h // (w.Nq // w.Nkv)]), f64(w.v[0, h // (w.Nq // w.Nkv)])
            qb = done % nqb
            rows = np.arange(qb * 128, min(w.Sq, qb * 128 + 128))
            oracle.attention_rows(q0, k0, v0, w.scale, rows)
            flops += 4 * D * len(rows) * w.Skv
            done += 1
        sample = (f"{done} (head, 128-row q-block) pairs, heads 0..{h}, each against all {w.Skv} keys: "
                  f"explicit float64 score rows, softmax and P.V")
    elif kind == "dense":
        cu = w.cu_seqlens_q
        g = w.Nq // w.Nkv
        pairs = [(b, h) for h in range(w.Nq) for b in range(w.B)]
        for b, h in pairs:
            if time.perf_counter() - t0 >= budget_s:
                break
            s0, s1 = int(cu[b]), int(cu[b + 1])
            L = s1 - s0
            qh, kh, vh = f64(w.q[s0:s1, h]), f64(w.k[s0:s1, h // g]), f64(w.v[s0:s1, h // g])
            for qb in range((L + 127) // 128):
                rows = np.arange(qb * 128, min(L, qb * 128 + 128))
                oracle.attention_rows(qh, kh, vh, w.scale, rows, sparse_mode=w.sparse_mode)
                flops += 4 * D * len(rows) * min(L, int(rows[-1]) + 1)
            done += 1
        sample = f"{done} (sequence, head) pairs, whole sequences, causal rows (useful flops)"
    elif kind == "blocksparse":
        nqb = w.keep.shape[2]
        h = -1
        while time.perf_counter() - t0 < budget_s and done < w.Nq * nqb:
            if done % nqb == 0:
                h += 1
                q0, k0, v0 = f64(w.q[0, h]), f64(w.k[0, h]), f64(w.v[0, h])
            qb = done % nqb
            oracle.attention_block_sparse(q0, k0, v0, w.scale, w.keep[0, h], qblocks=[qb])
            flops += 4 * D * 128 * 128 * int(w.keep[0, h, qb].sum())
            done += 1
        sample = f"{done} (head, q-block) pairs, heads 0..{h}, kept 128-key blocks gathered (executed flops)"
    else:
        nqb = w.keep.shape[2]
        h = -1
        while time.perf_counter() - t0 < budget_s and done < w.Nq * nqb:
            if done % nqb == 0:
                h += 1
                qc, qs = oracle.quantize_qk_perblock_int8(f64(w.q[:, h:h + 1]))
                kc, ks = oracle.quantize_qk_perblock_int8(f64(w.k[:, h:h + 1]))
                vc, vs = oracle.quantize_v_perchannel_fp8(f64(w.v[:, h:h + 1]))
            qb = done % nqb
            kept = np.nonzero(w.keep[0, h, qb])[0]
            oracle.qbsa_qblock(qc[0, 0], kc[0, 0], vc[0, 0], qs[0, 0, qb], ks[0, 0], vs[0, 0], w.scale, kept, qb)
            flops += 4 * D * 128 * 128 * len(kept)
            done += 1
        sample = (f"{done} (head, q-block) pairs, heads 0..{h}: quantise the head's Q/K/V, then the tiled "
                  f"FP8 schedule of each q-block (executed ops)")
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": sample + f"; {flops / 1e9:.2f} GFLOP in {dt:.1f} s", "seconds": round(dt, 2)}


def load_traffic(config_name: str, kind: str):
    path = os.path.join(ROOT, "profiles", f"traffic_{config_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_source_sha") != source_hash(kind):
        return None          # kernel changed since the counters were taken
    return t.get("traffic_bytes_per_launch")


def copy_calibration(nbytes: int):
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "launches": 3}), flush=True)


def _smi_clock_power(smi):
    """One `amd-smi metric -c -p` reading: (gfx clock averaged over the XCDs in MHz, socket power in
    W), or None when the tool is missing or prints something else."""
    import subprocess
    try:
        r = subprocess.run([smi, "metric", "-c", "-p", "--json"], capture_output=True, text=True, timeout=15)
        d = json.loads(r.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clks = [c["clk"]["value"] for key, c in g["clock"].items()
                if key.startswith("gfx_") and isinstance(c, dict) and isinstance(c.get("clk"), dict)
                and isinstance(c["clk"].get("value"), (int, float))]
        pw = g["power"]["socket_power"]["value"]
    except Exception:  # noqa: BLE001 - a missing or changed tool only ends the sampling
        return None
    if not clks or not isinstance(pw, (int, float)):
        return None
    return float(np.mean(clks)), float(pw)


class ClockSampler:
    """The GPU clock and socket power while the timed steps run: a host thread reads `amd-smi metric
    -c -p` back to back between start() and stop(). The tool's readings lag the load by up to about
    a second, so readings taken in the first `settle` seconds are dropped; the timed region must
    last a few seconds for several readings to remain."""

    def __init__(self, settle: float = 0.8):
        import shutil
        self.smi = shutil.which("amd-smi")
        self.settle = settle
        self.samples = []
        self._stop = None
        self._thread = None

    def start(self):
        import threading
        if self.smi is None:
            return self
        self._stop = threading.Event()
        t0 = time.perf_counter()

        def loop():
            while not self._stop.is_set():
                r = _smi_clock_power(self.smi)
                if r is None:
                    break
                if not self._stop.is_set():
                    self.samples.append((round(time.perf_counter() - t0, 2), round(r[0]), r[1]))

        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join(timeout=30)
        kept = [x for x in self.samples if x[0] >= self.settle]
        if not kept:
            return None
        return {"median_mhz": int(np.median([c for _, c, _ in kept])),
                "socket_power_w": round(float(np.median([w for _, _, w in kept]))),
                "samples_t_s_mhz_w": kept, "source": "amd-smi metric -c -p, read while the timed steps ran"}


def sustained_clock_power(step, step_ms, seconds=3.0, settle=1.0):
    """GPU clock and socket power while the step runs back to back for about `seconds` (the power
    study's schedules): one thread keeps launching steps while this one reads amd-smi. Readings
    before `settle` seconds are dropped (the tool lags the load). Returns the kept samples (time,
    gfx clock averaged over the XCDs, socket power) and their medians, or None without amd-smi."""
    import shutil
    import threading
    import torch
    smi = shutil.which("amd-smi")
    if smi is None:
        return None
    n = max(1, int(seconds * 1e3 / max(step_ms, 1e-3)))
    busy = threading.Event()
    busy.set()

    def launcher():
        for _ in range(n):
            step()
        torch.cuda.synchronize()
        busy.clear()

    t = threading.Thread(target=launcher, daemon=True)
    t0 = time.perf_counter()
    t.start()
    time.sleep(settle)
    samples = []
    while busy.is_set() and len(samples) < 12 and time.perf_counter() - t0 < 4 * seconds:
        r = _smi_clock_power(smi)
        if r is None:
            break
        if busy.is_set():
            samples.append((round(time.perf_counter() - t0, 2), round(r[0]), r[1]))
    t.join(timeout=60)
    if not samples:
        return None
    return {"sclk_mhz": round(float(np.median([c for _, c, _ in samples]))),
            "socket_power_w": round(float(np.median([w for _, _, w in samples]))),
            "samples_t_s_mhz_w": samples}


def operator_sweep(seqs, sparsities=(0.0, 0.5, 0.9), reps=5, qblock_order=True):
    """The single-operator sweep of the EagleQBSA article (section 4, Fig. 4.1) on this GPU: B=1,
    N=40, D=128, for each S and block sparsity: bf16 dense attention, bf16 block-sparse attention
    (BSA) and the quantised block-sparse kernel (QBSA; Q, K, V quantised beforehand, untimed).
    QBSA with every block kept is the quantised dense case. Inputs are N(0,1) bf16 drawn on the GPU
    from a fixed seed; a mask keeps the diagonal plus i.i.d. blocks with probability 1 - sparsity.
    Prints one JSON line per case (median of `reps` launches), then the speed ratios."""
    import torch
    import quantized_attention_tiled_amd as qa
    qa.load()
    dev = torch.device("cuda:0")
    B, N, D = 1, 40, 128
    scale = 1.0 / float(np.sqrt(D))

    def timed(fn):
        t0 = time.perf_counter()  # warm up for at least half a second (clocks ramp under load)
        while True:
            fn()
            torch.cuda.synchronize()
            if time.perf_counter() - t0 > 0.5:
                break
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        return float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))

    ratios = []
    for S in seqs:
        gen = torch.Generator(device=dev).manual_seed(7000 + S)
        q, k, v = (torch.randn(B, N, S, D, generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
        qq, qs = qa.quantize_qk_perblock_int8(q)
        kq, ks = qa.quantize_qk_perblock_int8(k)
        vq, vs = qa.quantize_v_perchannel_fp8(v)
        o = torch.empty_like(q)
        m = torch.empty((B, N, S), dtype=torch.float32, device=dev)
        l = torch.empty_like(m)
        QB = (S + 127) // 128
        dense_flop = 4 * D * N * S * S
        t_dense = timed(lambda: qa.attn_fwd(q, k, v, scale=scale, out=o, softmax_max=m, softmax_sum=l))
        print(json.dumps({"sweep": "operator", "S": S, "sparsity": 0.0, "kernel": "bf16_dense", "ms": round(t_dense, 4),
                          "executed_tflops": round(dense_flop / t_dense / 1e9, 1),
                          "pct_peak": round(100 * dense_flop / t_dense / 1e9 / PEAK_BF16, 1)}), flush=True)
        for sp in sparsities:
            keep = (torch.rand(B, N, QB, QB, generator=gen, device=dev) >= sp).to(torch.uint8)
            keep[:, :, torch.arange(QB), torch.arange(QB)] = 1
            counts, idx = qa.build_kv_block_list(keep)
            order = qa.build_qblock_order(counts) if qblock_order else None
            kept = float(keep.float().mean())
            ex = 4 * D * 128 * 128 * int(keep.sum())
            t_bsa = timed(lambda: qa.attn_fwd_blocksparse(q, k, v, counts, idx, scale=scale, out=o, softmax_max=m,
                                                          softmax_sum=l, qblock_order=order))
            t_q = timed(lambda: qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=scale, out=o, softmax_max=m,
                                                 softmax_sum=l, qblock_order=order))
            for kern, t, peak in (("bf16_bsa", t_bsa, PEAK_BF16), ("qbsa", t_q, PEAK_FP8)):
                print(json.dumps({"sweep": "operator", "S": S, "sparsity": sp, "kept_fraction": round(kept, 4),
                                  "kernel": kern, "ms": round(t, 4), "executed_tflops": round(ex / t / 1e9, 1),
                                  "dense_equiv_tflops": round(dense_flop / t / 1e9, 1),
                                  "pct_peak": round(100 * ex / t / 1e9 / peak, 1)}), flush=True)
            ratios.append({"S": S, "sparsity": sp, "dense_over_bsa": round(t_dense / t_bsa, 2),
                           "dense_over_qbsa": round(t_dense / t_q, 2), "bsa_over_qbsa": round(t_bsa / t_q, 2)})
        del q, k, v, qq, kq, vq, o
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": "ratios", "rows": ratios}), flush=True)
    return 0


def power_study(S, gaps_ms, chunk_counts=(10,), seconds=3.0):
    """The single-GPU part of the power-cap page's schedules (FA_Power_Cap: InsertComm splits the
    attention by head chunks with each chunk's all-to-all in front of it; BlockAttn also splits the
    local queries into 2 blocks), compared with one call (Baseline: all communication, then one
    attention). The shape is one GPU's share of the page's Wan2.2 attention at Ulysses degree 4:
    B=1, N=10 of 40 heads, D=128, S tokens; 10 chunks of one head (loop_time 10), or fewer, larger
    chunks (`chunk_counts`, each dividing N). The communication
    is stood in for by idle gaps (one spinning thread): `gap` ms per layer, split evenly over the
    chunks (Baseline: one gap before its one call), so every schedule idles for the same time. For each schedule and gap, prints one JSON line: time per layer, the
    attention and gap parts of it (HIP events around every launch and gap), and the gfx clock and
    socket power while the schedule runs back to back."""
    import torch
    import quantized_attention_tiled_amd as qa
    qa.load()
    dev = torch.device("cuda:0")
    B, N, D = 1, 10, 128
    gen = torch.Generator(device=dev).manual_seed(2024)
    q, k, v = (torch.randn((B, N, S, D), generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    m = torch.empty((B, N, S), dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    nqb = (S + 127) // 128
    scale = D ** -0.5
    stream = torch.cuda.current_stream(dev)

    def fa(hr=None, br=None):
        qa.attn_fwd(q, k, v, scale=scale, head_range=hr, qblock_range=br, out=o, softmax_max=m, softmax_sum=l)

    # spin-kernel cycles per ms, from a timed calibration (its counter need not run at a fixed rate)
    def cycles_for(ms_target):
        if ms_target <= 0:
            return 0
        c = 1_000_000
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            torch.cuda._sleep(c)
            e1.record(stream)
            torch.cuda.synchronize()
            c = max(1000, int(c * ms_target / max(e0.elapsed_time(e1), 1e-3)))
        return c

    def schedule(kind, gap_cycles, chunks, events=None):
        parts = []  # ("gap" | "fa", start event, end event)

        def seg(tag, fn):
            if events is None:
                fn()
                return
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            parts.append((tag, e0, e1))

        if kind == "baseline":
            if gap_cycles:
                seg("gap", lambda: torch.cuda._sleep(gap_cycles))
            seg("fa", fa)
        else:
            per = N // chunks
            for c in range(chunks):
                if gap_cycles:
                    seg("gap", lambda: torch.cuda._sleep(gap_cycles))
                hr = (c * per, (c + 1) * per)
                if kind == "insertcomm":
                    seg("fa", lambda: fa(hr))
                else:
                    seg("fa", lambda: fa(hr, (0, nqb // 2)))
                    seg("fa", lambda: fa(hr, (nqb // 2, nqb)))
        if events is not None:
            events.extend(parts)

    cases = [(gap, "baseline", 1) for gap in gaps_ms] + \
        [(gap, kind, c) for c in chunk_counts for gap in gaps_ms for kind in ("insertcomm", "blockattn")]
    for gap, kind, chunks in cases:
        if N % chunks:
            raise ValueError(f"{chunks} chunks do not divide {N} heads")
        cyc = cycles_for(gap / chunks)
        for _ in range(3):
            schedule(kind, cyc, chunks)
        torch.cuda.synchronize()
        reps = 5
        evs = []
        e_all0, e_all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e_all0.record(stream)
        for _ in range(reps):
            schedule(kind, cyc, chunks, evs)
        e_all1.record(stream)
        torch.cuda.synchronize()
        total = e_all0.elapsed_time(e_all1) / reps
        fa_ms = sum(a.elapsed_time(b) for t, a, b in evs if t == "fa") / reps
        gap_total = sum(a.elapsed_time(b) for t, a, b in evs if t == "gap") / reps
        sustained = sustained_clock_power(lambda: schedule(kind, cyc, chunks), total, seconds=seconds)
        flop = 4.0 * D * B * N * S * S
        line = {"study": "power_cap", "schedule": kind, "chunks": chunks, "gap_ms_per_layer": gap, "S": S, "N": N,
                "launches": 1 if kind == "baseline" else chunks * (1 if kind == "insertcomm" else 2),
                "ms_per_layer": round(total, 3), "attention_ms": round(fa_ms, 3), "gap_ms": round(gap_total, 3),
                "attention_tflops": round(flop / fa_ms / 1e9, 1)}
        if sustained:
            line["sclk_mhz"] = sustained["sclk_mhz"]
            line["socket_power_w"] = sustained["socket_power_w"]
            line["energy_j_per_layer"] = round(sustained["socket_power_w"] * total * 1e-3, 3)
        print(json.dumps(line), flush=True)
    return 0


def backward_bench(a):
    """The attention backward (dQ, dK, dV) on a dense BNSD config: the forward runs once, untimed,
    then W warm-up and K timed backward calls (all three kernels) between HIP events. Flops: the
    usual 6 D + 4 Dv per (q, k) pair (five products: S and dK, dQ over D, dP and dV over Dv; 10 D
    when Dv = D, 2.5 times the forward's 4 D), and the executed 8 D + 6 Dv of these kernels (S and
    dP are formed once for dQ and once for dK / dV); causal counts the pairs at or below the
    diagonal. --head-dim and --dv set D and Dv. Prints one JSON line."""
    import torch
    import quantized_attention_tiled_amd as qa
    from workloads import CONFIGS, make_workload
    qa.load()
    if CONFIGS[a.config]["kind"] != "dense":
        log("--backward takes a dense config (BNSD or TND)")
        return 2
    w = make_workload(a.config, S=a.seq, D=a.head_dim)
    Dv = a.dv or w.D
    if not 0 < Dv <= w.D:
        log(f"--dv must lie in [1, D = {w.D}]")
        return 2
    w.v = np.ascontiguousarray(w.v[..., :Dv])  # the first Dv channels of the same draw
    dev = torch.device("cuda:0")

    def up(bits):
        if a.dtype == "fp16":  # the same values as float16 (bf16 -> fp16 is exact in this range)
            from workloads import bf16_bits_to_f32
            return torch.from_numpy(bf16_bits_to_f32(bits).astype(np.float16)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(w.q), up(w.k), up(w.v)
    gen = torch.Generator(device=dev).manual_seed(77)
    do = torch.randn(q.shape[:-1] + (Dv,), generator=gen, device=dev).to(q.dtype)
    tnd = w.layout == "TND"
    mode = w.sparse_mode if tnd else a.bwd_mode
    kw = dict(scale=w.scale, sparse_mode=mode)
    if tnd:
        kw.update(layout="TND", cu_seqlens_q=w.cu_seqlens_q.tolist(), cu_seqlens_kv=w.cu_seqlens_kv.tolist())
    o, m, l = qa.attn_fwd(q, k, v, **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(2 * m.numel(), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        qa.attn_bwd(q, k, v, o, do, m, l, dq=dq, dk=dk, dv=dv, workspace=ws, **kw)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    ev[0].record(stream)
    for i in range(a.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(a.steps)])
    ms = ev[0].elapsed_time(ev[a.steps]) / a.steps
    if tnd:  # equal query and key lengths per sequence, so both causal modes keep L (L + 1) / 2 pairs
        lens = np.diff(w.cu_seqlens_q)
        pairs = w.Nq * int(sum(int(L) * (int(L) + 1) // 2 if mode in (2, 3) else int(L) * int(L) for L in lens))
    else:
        pairs = w.B * w.Nq * (w.Sq * (w.Sq + 1) // 2 if mode == 2 else w.Sq * w.Skv)
    std, exe = (6 * w.D + 4 * Dv) * pairs, (8 * w.D + 6 * Dv) * pairs
    line = {"metric": "attention bwd TFLOP/s (dQ, dK, dV; 6 D + 4 Dv flops per pair), % bf16 MFMA peak",
            "value": round(std / ms / 1e9, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
            "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "dtype": a.dtype,
            "data": "synthetic (seeded forward inputs; dO N(0,1) drawn on the GPU)",
            "config": {"workload": f"{a.config}: {w.description}" + (f" (S {w.Sq})" if a.seq else "") +
                       (f" (D {w.D})" if a.head_dim else ""), "D": w.D, "Dv": Dv, "sparse_mode": mode},
            "detail": {"executed_tflops": round(exe / ms / 1e9, 2), "pct_mfma_peak_executed":
                       round(100 * exe / ms / 1e9 / PEAK_BF16, 2), "median_ms": round(float(np.median(per)), 4),
                       "cv": round(float(per.std() / per.mean()), 4), "kernel_source_sha": source_hash("backward")}}
    print(json.dumps(line), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="untimed whole steps run before the warm-up until this many seconds (and at least 16 "
                         "steps) have passed: the first launches of a process run slow while code loads and the "
                         "clock and power settle")
    ap.add_argument("--config", default="c2_dense_8k")
    ap.add_argument("--seq", type=int, default=None, help="override S (dense BNSD configs)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=int, default=None)
    ap.add_argument("--no-smi", action="store_true", help="skip the sustained clock / power sample")
    ap.add_argument("--sweep", action="store_true", help="operator sweep (S x sparsity x kernel) instead of one line")
    ap.add_argument("--sweep-seqs", default="8192,16384,32768,65536")
    ap.add_argument("--backward", action="store_true", help="time the attention backward on the config instead")
    ap.add_argument("--bwd-mode", type=int, default=0, choices=[0, 2], help="sparse_mode of the backward bench")
    ap.add_argument("--power-study", action="store_true",
                    help="power-cap schedules (one call vs head chunks vs head chunks x 2 q-blocks, with gaps)")
    ap.add_argument("--power-seq", type=int, default=75600, help="S of the power-cap study")
    ap.add_argument("--power-gaps", default="0,2.5,10", help="idle ms per layer (the communication), comma separated")
    ap.add_argument("--power-chunks", default="10", help="head-chunk counts of the study, comma separated")
    ap.add_argument("--dtype", choices=["bf16", "fp16"], default="bf16",
                    help="input / output type of the dense and block-sparse configs (fp16: the same values in float16)")
    ap.add_argument("--dv", type=int, default=None, help="value head dimension below D (dense / block-sparse configs)")
    ap.add_argument("--head-dim", type=int, default=None,
                    help="query/key head dimension D in place of the config's (dense / block-sparse BNSD configs; "
                         "scale 1/sqrt(D))")
    ap.add_argument("--mask", choices=["none", "bytes", "bits"], default="none",
                    help="dense BNSD configs: an SS atten_mask [S, S], one byte per key or bit-packed")
    ap.add_argument("--mask-density", type=float, default=0.0, help="fraction of masked keys of --mask (i.i.d.)")
    ap.add_argument("--no-qblock-order", action="store_true",
                    help="block-sparse and quantised configs: launch the q-blocks of each head in index order "
                         "instead of by kept count (build_qblock_order)")
    ap.add_argument("--q-gain", type=float, default=1.0,
                    help="dense configs: multiply Q by this factor (a peaked softmax: rows whose max outgrows the "
                         "16-bit kernel's reference take its second key pass)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {a.gpus}).",
              file=sys.stderr)
        return 2
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py runs as a single process on one GPU.", file=sys.stderr)
        return 2
    import torch
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return 0
    if a.sweep:
        return operator_sweep([int(x) for x in a.sweep_seqs.split(",") if x], qblock_order=not a.no_qblock_order)
    if a.backward:
        return backward_bench(a)
    if a.power_study:
        return power_study(a.power_seq, [float(x) for x in a.power_gaps.split(",") if x],
                           [int(x) for x in a.power_chunks.split(",") if x])

    import quantized_attention_tiled_amd as qa
    from workloads import CONFIGS, make_workload

    qa.load()
    cfg = CONFIGS[a.config]
    kind = cfg["kind"]
    if (a.dtype != "bf16" or a.dv or a.head_dim) and kind == "qbsa":
        log("--dtype / --dv / --head-dim apply to the dense and block-sparse configs only")
        return 2
    if a.head_dim and cfg["layout"] != "BNSD":
        log("--head-dim applies to the BNSD configs")
        return 2
    log(f"generating {a.config} {'S=' + str(a.seq) if a.seq else ''} {'D=' + str(a.head_dim) if a.head_dim else ''}")
    w = make_workload(a.config, S=a.seq, D=a.head_dim)
    name = a.config if not a.seq else f"{a.config}_S{a.seq}"
    if a.head_dim:
        name += f"_d{a.head_dim}"
    if a.dv:
        if not 0 < a.dv <= w.D:
            log(f"--dv must lie in [1, D = {w.D}]")
            return 2
        w.v = np.ascontiguousarray(w.v[..., :a.dv])  # the first Dv channels of the same draw
        name += f"_dv{a.dv}"
    if a.dtype != "bf16":
        name += f"_{a.dtype}"
    if a.q_gain != 1.0:
        if kind != "dense":
            log("--q-gain applies to the dense configs")
            return 2
        from workloads import bf16_bits_to_f32, f32_to_bf16_bits
        w.q = f32_to_bf16_bits(bf16_bits_to_f32(w.q) * np.float32(a.q_gain))
        name += f"_qgain{a.q_gain:g}"
    if a.no_qblock_order and kind != "dense":
        name += "_unordered"
    dev = torch.device("cuda:0")

    def up(bits):
        if a.dtype == "fp16":  # the same values (bf16 -> fp16 is exact in this range) as float16
            from workloads import bf16_bits_to_f32
            return torch.from_numpy(bf16_bits_to_f32(bits).astype(np.float16)).to(dev)
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = up(w.q), up(w.k), up(w.v)
    o = torch.empty(q.shape[:-1] + (v.shape[-1],), dtype=q.dtype, device=dev)
    ml_shape = (w.B, w.Nq, w.Sq) if w.layout == "BNSD" else (w.Nq, w.Sq)
    m = torch.empty(ml_shape, dtype=torch.float32, device=dev)
    l = torch.empty(ml_shape, dtype=torch.float32, device=dev)
    # every launch goes to torch's current stream of cuda:0, which the binding passes to the library
    stream = torch.cuda.current_stream(dev)
    amask = None
    if a.mask != "none":
        if kind != "dense" or w.layout != "BNSD":
            log("--mask applies to the dense BNSD configs")
            return 2
        # seeded i.i.d. SS mask (1 = masked); every row keeps at least its first key
        mk = (np.random.default_rng(77).random((w.Sq, w.Skv)) < a.mask_density).astype(np.uint8)
        mk[:, 0] = 0
        if a.mask == "bits":
            W = (w.Skv + 31) // 32
            pad = np.zeros((w.Sq, 32 * W), np.uint8)
            pad[:, :w.Skv] = mk
            mk = np.ascontiguousarray(np.packbits(pad, axis=-1, bitorder="little")).view("<i4")
        amask = torch.from_numpy(mk).to(dev)
        name += f"_mask{a.mask}{a.mask_density:g}"
    if kind == "dense":
        cu = w.cu_seqlens_q.tolist() if w.layout == "TND" else None

        def step(ka=None, kb=None):
            if ka is not None:
                ka.record(stream)
            qa.attn_fwd(q, k, v, scale=w.scale, layout=w.layout, sparse_mode=w.sparse_mode, cu_seqlens_q=cu,
                        cu_seqlens_kv=cu, out=o, softmax_max=m, softmax_sum=l, atten_mask=amask)
            if kb is not None:
                kb.record(stream)
        dtype, peak = a.dtype, PEAK_BF16
    elif kind == "blocksparse":
        keep = torch.from_numpy(w.keep).to(dev)
        counts = torch.empty(w.keep.shape[:3], dtype=torch.int32, device=dev)
        idx = torch.empty(w.keep.shape, dtype=torch.int32, device=dev)
        order = None if a.no_qblock_order else torch.empty(w.keep.shape[:3], dtype=torch.int32, device=dev)

        def step(ka=None, kb=None):
            qa.build_kv_block_list(keep, counts, idx)
            if order is not None:
                qa.build_qblock_order(counts, order)
            if ka is not None:
                ka.record(stream)
            qa.attn_fwd_blocksparse(q, k, v, counts, idx, scale=w.scale, out=o, softmax_max=m, softmax_sum=l,
                                    qblock_order=order)
            if kb is not None:
                kb.record(stream)
        dtype, peak = a.dtype, PEAK_BF16
    else:
        keep = torch.from_numpy(w.keep).to(dev)
        counts = torch.empty(w.keep.shape[:3], dtype=torch.int32, device=dev)
        idx = torch.empty(w.keep.shape, dtype=torch.int32, device=dev)
        qq = torch.empty(q.shape, dtype=torch.int8, device=dev)
        kq = torch.empty(k.shape, dtype=torch.int8, device=dev)
        vq = torch.empty(v.shape, dtype=torch.uint8, device=dev)
        nb = (w.Sq + 127) // 128
        qs = torch.empty((w.B, w.Nq, nb), dtype=torch.float32, device=dev)
        ks = torch.empty((w.B, w.Nkv, nb), dtype=torch.float32, device=dev)
        vs = torch.empty((w.B, w.Nkv, w.D), dtype=torch.float32, device=dev)
        order = None if a.no_qblock_order else torch.empty(w.keep.shape[:3], dtype=torch.int32, device=dev)

        def step(ka=None, kb=None):
            qa.quantize_qk_perblock_int8(q, qq, qs)
            qa.quantize_qk_perblock_int8(k, kq, ks)
            qa.quantize_v_perchannel_fp8(v, vq, vs)
            qa.build_kv_block_list(keep, counts, idx)
            if order is not None:
                qa.build_qblock_order(counts, order)
            if ka is not None:
                ka.record(stream)
            qa.attn_fwd_qbsa(qq, kq, vq, qs, ks, vs, counts, idx, scale=w.scale, out=o, softmax_max=m,
                             softmax_sum=l, qblock_order=order)
            if kb is not None:
                kb.record(stream)
        dtype, peak = "int8/fp8", PEAK_FP8

    # Settling: the first launches of a process run slower (code loading, then about a dozen launches
    # while the clock and power settle), so whole steps run untimed for a fixed time before the W
    # warm-up steps; the timed region is unchanged.
    settle_n, settle_t0 = 0, time.perf_counter()
    while settle_n < 16 or time.perf_counter() - settle_t0 < a.settle_s:
        for _ in range(8):
            step()
        settle_n += 8
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - settle_t0
    log(f"settled after {settle_n} steps ({settle_s:.2f} s); warmup {a.warmup}")
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    kev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
    log(f"timing {a.steps} steps")
    torch.cuda.synchronize()
    # amd-smi readings lag the load by up to a second: a timed region shorter than about two seconds
    # gets none, and the sampling thread's process launches would only disturb the host's launches
    expect_s = a.steps * settle_s / max(settle_n, 1)
    sampler = None if a.no_smi or expect_s < 2.0 else ClockSampler().start()
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(a.steps):
        step(*kev[i])
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    clock = sampler.stop() if sampler is not None else None
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(a.steps)])
    kper = np.array([ka.elapsed_time(kb) for ka, kb in kev])
    total_ms = ev[0].elapsed_time(ev[a.steps])
    ms = total_ms / a.steps
    kms = float(kper.mean())
    ex, useful, dense = flop_counts(w)
    value = ex / (ms * 1e-3) / 1e12
    kvalue = ex / (kms * 1e-3) / 1e12
    alg_bytes = algorithmic_bytes(w, kind)
    traffic = load_traffic(name, kind)
    # the dominant kernel: algorithmic flops of one launch / its mean launch duration (HIP events on the
    # launch stream, bracketing that launch alone)
    roof = {"bound": "mfma", "achieved": round(kvalue, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(kvalue / peak, 4), "traffic": traffic, "kernel": "attn_fwd_kernel" if kind != "qbsa"
            else "attn_qbsa_kernel", "flop_per_launch": ex, "launch_ms": round(kms, 4)}
    if clock:
        # the published peak assumes 2400 MHz; at the clock measured during the timed steps the
        # matrix cores can deliver peak * clock / 2400
        roof["clock_mhz_during_timed"] = clock["median_mhz"]
        roof["clock_limited_peak"] = round(peak * clock["median_mhz"] / 2400.0, 1)
        roof["frac_of_clock_limited_peak"] = round(kvalue / roof["clock_limited_peak"], 4)
    cpu = None
    if not a.no_cpu:
        log(f"cpu oracle baseline (~{a.cpu_seconds:.0f} s)")
        cpu = run_cpu_baseline(w, kind, a.cpu_seconds)
    if w.layout == "TND":
        wl = f"{a.config}: {w.description}; T={w.Sq}"
        conf = {"workload": wl, "layout": "TND", "sequences": int(w.B), "lengths": np.diff(w.cu_seqlens_q).tolist(),
                "Nq": w.Nq, "Nkv": w.Nkv, "D": w.D, "sparse_mode": w.sparse_mode}
    else:
        wl = f"{name}: {w.description}" + (f" (S overridden to {w.Sq})" if a.seq else "") + \
            (f" (D overridden to {w.D})" if a.head_dim else "")
        conf = {"workload": wl, "layout": "BNSD", "B": w.B, "N": w.Nq, "Nkv": w.Nkv, "S": w.Sq, "D": w.D}
        if a.dv:
            conf["Dv"] = a.dv
        if a.q_gain != 1.0:
            conf["q_gain"] = a.q_gain
        if amask is not None:
            conf["atten_mask"] = {"kind": "SS", "format": a.mask, "density": a.mask_density,
                                  "bytes": int(amask.numel() * amask.element_size())}
        if w.keep is not None:
            conf["kept_fraction"] = round(float(w.keep.mean()), 4)
            conf["qblock_order"] = "index" if a.no_qblock_order else "by kept count (build_qblock_order)"
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic (seeded, shapes of the pages' workloads)",
        "config": conf, "roofline": roof, "cpu_baseline": cpu,
        "detail": {"executed_tflops": round(value, 2), "dense_equiv_tflops": round(dense / (ms * 1e-3) / 1e12, 2),
                   "useful_tflops": round(useful / (ms * 1e-3) / 1e12, 2),
                   "pct_mfma_peak": round(100 * value / peak, 2), "median_ms": round(float(np.median(per)), 4),
                   "min_ms": round(float(per.min()), 4), "cv": round(float(per.std() / per.mean()), 4),
                   "algorithmic_bytes": alg_bytes, "algorithmic_gbps": round(alg_bytes / (ms * 1e-3) / 1e9, 1),
                   "wall_s_timed": round(wall, 3), "kernel_source_sha": source_hash(kind),
                   "clock_during_timed": clock,
                   "settle": {"untimed_steps": settle_n, "seconds": round(settle_s, 3)}},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
