"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-widened] [--no-sweep]

One step runs every kernel of the path once on the headline workload
(B=2, H=16, N=8192, d=128, causal), inputs already resident in HBM:
  fa_fwd (bf16)  ->  fa_bwd (bf16, recomputing P from the saved LSE)
  ->  fa_quant_fp8 on Q, K (random-sign Hadamard rotation) and V  ->  fa_fwd_fp8.
Kernels that are not built yet are left out of the step and listed as such.

Prints ONE JSON line on stdout. "value" is the metric exactly: the bf16
forward + backward rate, algorithmic causal FLOPs (forward 4 B H N^2 d / 2,
backward 2.5x that) over the two calls' own times inside the timed steps (HIP
events on the stream they run on), with its fraction of the 2516.6 TFLOP/s
dense bf16 MFMA peak. The fp8 leg (quantiser and e4m3 forward) runs in every
step too and is reported on its own in "breakdown" (against the 5033.2 TFLOP/s
e4m3 peak, and HBM for the quantiser). Also: the roofline of the dominant
kernel, the shader clock sampled from sysfs while the bf16 kernels run (with
the utilisation normalised to it), and the fp64 CPU oracle timed on a bounded
sample of the same workload. After the timed steps (and outside them) the
widened rows are timed on their own shapes ("widened") and a sequence-length
sweep ("sweep"), each as median / min / max over repeated calls.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOPS (bf16, causal, d=128, N=8k) + % of MFMA peak, 1 GPU"
PEAK_BF16 = 2516.6   # TFLOP/s, dense MFMA, 256 CUs x 4096 FLOP/clk x 2.4 GHz
PEAK_FP8 = 5033.2    # TFLOP/s
PEAK_HBM = 8000.0    # GB/s
B, H, N, D = 2, 16, 8192, 128


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fwd_flops(b, h, n, d, causal=True):
    f = 4.0 * b * h * n * n * d
    return f / 2 if causal else f


def fwd_bytes(b, h, n, d, elt=2):
    # Q, K, V in and O out (elt bytes each) plus the fp32 LSE
    return 4.0 * b * h * n * d * elt + 4.0 * b * h * n


def bwd_bytes(b, h, n, d):
    # reads Q, K, V, O, dO (bf16) and LSE; writes dQ, dK, dV (bf16); D written once, read once
    return 8.0 * b * h * n * d * 2 + 4.0 * b * h * n * 3


def visible_pairs(n_q, n_k, causal, window=(-1, -1)):
    """Number of (query, key) pairs a mask leaves visible in one head, counted
    row by row: query i sees keys c - left .. c + right of 0 .. n_k - 1, with
    c = i + n_k - n_q (right capped at 0 when causal; -1 = unbounded)."""
    import numpy as np
    left, right = window
    c = np.arange(n_q, dtype=np.int64) + (n_k - n_q)
    lo = np.zeros(n_q, dtype=np.int64) if left < 0 else np.maximum(0, c - left)
    hi = np.full(n_q, n_k - 1, dtype=np.int64) if right < 0 else np.minimum(n_k - 1, c + right)
    if causal:
        hi = np.minimum(hi, c)
    return int(np.maximum(0, hi - lo + 1).sum())


def quant_bytes(b, h, n, d):
    return b * h * n * d * (2 + 1) + 4.0 * b * h * ((n + 127) // 128)


def measured_traffic(path: str):
    """Bytes per launch from a committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary,
    or None when the kernel sources listed there changed since it was taken."""
    import hashlib
    try:
        fields = {}
        for line in open(path):
            if ":" in line and line.split(":", 1)[0] in ("traffic_bytes_per_launch", "source_sha1", "sources"):
                k, v = line.split(":", 1)
                fields[k] = v.strip()
        h = hashlib.sha1()
        for src in fields["sources"].split():
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != fields["source_sha1"]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_model() -> str | None:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def call_stats(times):
    """median / min / max (ms) of repeated calls; the individual times too when
    the slowest is more than twice the median (a stall, not the kernel)."""
    import numpy as np
    t = np.asarray(times, dtype=np.float64)
    med = float(np.median(t))
    out = {"ms_median": med, "ms_min": float(t.min()), "ms_max": float(t.max()), "calls": int(t.size)}
    if t.max() > 2.0 * med:
        out["ms_each"] = [float(x) for x in t]
    return out


def sclk_file():
    """The sysfs file that lists the shader clock levels of this GPU (the
    current one marked '*'), or None."""
    import glob
    cands = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    if not cands:
        return None
    try:
        import torch
        p = torch.cuda.get_device_properties(0)
        bus = "%04x:%02x:%02x" % (getattr(p, "pci_domain_id", 0), p.pci_bus_id, p.pci_device_id)
        for c in cands:
            if bus in os.path.realpath(os.path.dirname(c)):
                return c
    except Exception:
        pass
    return cands[0] if len(cands) == 1 else None


def read_sclk_mhz(path):
    try:
        for line in open(path):
            if line.strip().endswith("*"):
                v = line.split(":", 1)[1].strip().rstrip("*").strip().lower()
                return float(v.replace("mhz", ""))
    except (OSError, ValueError, IndexError):
        pass
    return None


def sample_sclk(run, seconds=1.5):
    """Run `run` (one bf16 forward + backward) back to back for about `seconds`
    while a thread reads the current shader clock every 10 ms."""
    import threading
    import numpy as np
    import torch
    path = sclk_file()
    if path is None:
        return {"mhz_median": None, "reason": "no pp_dpm_sclk in sysfs for this GPU"}
    vals, stop = [], threading.Event()

    def reader():
        while not stop.is_set():
            v = read_sclk_mhz(path)
            if v is not None:
                vals.append(v)
            time.sleep(0.01)

    th = threading.Thread(target=reader, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(5):
            run()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not vals:
        return {"mhz_median": None, "reason": "sysfs clock unreadable", "file": path}
    v = np.asarray(vals)
    return {"mhz_median": float(np.median(v)), "mhz_min": float(v.min()), "mhz_max": float(v.max()),
            "samples": int(v.size), "file": path,
            "how": "sysfs pp_dpm_sclk current level, every 10 ms while bf16 fa_fwd + fa_bwd run back to back"}


def cpu_baseline(sample_heads: int):
    """The fp64 oracle (as it stands) on `sample_heads` heads of the bf16
    workload: one forward and one backward per head."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import fa_inputs
    from oracle import attention as A

    rng = np.random.Generator(np.random.PCG64(3))
    q, k, v, do = (rng.standard_normal((sample_heads, N, D), dtype=np.float32) for _ in range(4))
    q, k, v, do = (fa_inputs.to_bf16_values(x) for x in (q, k, v, do))
    scale = 1.0 / math.sqrt(D)
    t0 = time.perf_counter()
    for i in range(sample_heads):
        A.forward_head(q[i], k[i], v[i], True, scale)
        A.backward_head(q[i], k[i], v[i], do[i], True, scale)
    dt = time.perf_counter() - t0
    flops = 3.5 * fwd_flops(1, sample_heads, N, D)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    cores = len(os.sched_getaffinity(0))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": min(cores, int(threads)),
            "host_cores": cores, "blas_threads": int(threads), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": "fp64 forward + backward by definition on %d of the %d heads of the "
                      "B=%d H=%d N=%d d=%d causal workload (%.1f s); algorithmic causal FLOPs / wall time"
                      % (sample_heads, B * H, B, H, N, D, dt),
            "seconds": dt}


def widened(fa, dev, q, k, v, do, steps=10, warmup=5):
    """The widened rows (grouped heads, [B, N, H, d] layout, sliding window,
    ALiBi, cross-attention, d = 64 and 256) on shapes of the headline's size:
    bf16 forward and backward, each timed with HIP events on the current
    stream, algorithmic FLOPs = 4 d x (visible pairs) per head (backward 2.5x).
    """
    import numpy as np
    import torch

    import fa_inputs

    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(warmup):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return call_stats([a.elapsed_time(b) for a, b in evs])

    def case(qq, kk, vv, dd, causal=True, window=None, slopes=None, cfg=""):
        b_, h_, nq, d_ = qq.shape
        nk = kk.shape[2]
        o_, l_ = fa.fwd(qq, kk, vv, causal=causal, window=window, alibi_slopes=slopes)
        need = fa.bwd_workspace_bytes(b_, h_, nq, d_, H_kv=kk.shape[1], causal=causal, N_k=nk,
                                      window=window)
        ws_ = torch.empty(need, dtype=torch.uint8, device=dev)
        sf = timed(lambda: fa.fwd(qq, kk, vv, causal=causal, window=window, alibi_slopes=slopes, out=o_, lse=l_))
        sb = timed(lambda: fa.bwd(qq, kk, vv, o_, dd, l_, causal=causal, workspace=ws_, window=window,
                                  alibi_slopes=slopes))
        tf, tb = sf["ms_median"], sb["ms_median"]
        flops = 4.0 * d_ * visible_pairs(nq, nk, causal, window if window is not None else (-1, -1)) * b_ * h_
        ent = {"config": cfg, "fwd_ms": tf, "bwd_ms": tb, "fwd_calls": sf, "bwd_calls": sb,
               "fwd_tflops": flops / (tf * 1e-3) / 1e12, "bwd_tflops": 2.5 * flops / (tb * 1e-3) / 1e12}
        ent["fwd_frac"] = ent["fwd_tflops"] / PEAK_BF16
        ent["bwd_frac"] = ent["bwd_tflops"] / PEAK_BF16
        log("widened %-8s fwd %.3f ms (%.3f..%.3f) %.0f TFLOP/s, bwd %.3f ms (%.3f..%.3f) %.0f TFLOP/s"
            % (cfg.split(":")[0], tf, sf["ms_min"], sf["ms_max"], ent["fwd_tflops"], tb, sb["ms_min"],
               sb["ms_max"], ent["bwd_tflops"]))
        return ent

    out = {}
    hkv = 2
    kg, vg = k[:, :hkv].contiguous(), v[:, :hkv].contiguous()
    out["gqa"] = case(q, kg, vg, do, cfg="gqa: B=2 H=16 H_kv=2 N=8192 d=128 causal")
    qt, kt, vt, dt = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v, do))
    out["bnhd"] = case(qt, kt, vt, dt, cfg="bnhd: [B, N, H, d] storage, B=2 H=16 N=8192 d=128 causal")
    del qt, kt, vt, dt
    out["window"] = case(q, k, v, do, window=(1024, 0),
                         cfg="window: B=2 H=16 N=8192 d=128 causal, 1024 keys back")
    slopes = torch.from_numpy(fa_inputs.alibi_slopes(q.shape[1])).to(dev)
    out["alibi"] = case(q, k, v, do, slopes=slopes, cfg="alibi: B=2 H=16 N=8192 d=128 causal")
    nq = q.shape[2] // 4
    out["cross"] = case(q[:, :, -nq:], k, v, do[:, :, -nq:].contiguous(),
                        cfg="cross: B=2 H=16 N_q=2048 N_k=8192 d=128 causal (last queries on last keys)")
    for d_ in (64, 256):
        x = fa_inputs.attention_inputs(1, 16, 8192, d_, seed=7, with_do=True)
        qd, kd, vd, dd = (torch.from_numpy(x[n]).to(torch.bfloat16).to(dev) for n in ("q", "k", "v", "do"))
        del x
        out["d%d" % d_] = case(qd, kd, vd, dd, cfg="d%d: B=1 H=16 N=8192 d=%d causal" % (d_, d_))
        del qd, kd, vd, dd
    return out


def fp8_exp_modes(fa, q8, k8, v8, qs, ks, vs, flops, rounds=10, warmup=3):
    """The fp8 forward with its softmax exponentials on the hardware unit
    (exp_mode 0, the step's form) and in the software 2^x for one in four
    (1) or all (2) of them: the three modes interleaved call by call, so each
    sees the same clock, each timed with HIP events on the current stream."""
    import torch

    stream = torch.cuda.current_stream()
    fns = [lambda m=m: fa.fwd_fp8(q8, k8, v8, qs, ks, vs, causal=True, exp_mode=m) for m in range(3)]
    for _ in range(warmup):
        for fn in fns:
            fn()
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
           for _ in range(rounds)]
    torch.cuda.synchronize()
    for r in range(rounds):
        for i, fn in enumerate(fns):
            evs[r][i][0].record(stream)
            fn()
            evs[r][i][1].record(stream)
    torch.cuda.synchronize()
    out = {}
    for i in range(3):
        st = call_stats([evs[r][i][0].elapsed_time(evs[r][i][1]) for r in range(rounds)])
        st["tflops"] = flops / (st["ms_median"] * 1e-3) / 1e12
        st["frac"] = st["tflops"] / PEAK_FP8
        out["exp_mode%d" % i] = st
        log("fp8 exp_mode %d: %.3f ms (%.3f..%.3f) %.0f TFLOP/s"
            % (i, st["ms_median"], st["ms_min"], st["ms_max"], st["tflops"]))
    return out


def sweep(fa, dev, steps=10, warmup=5):
    """Sequence-length sweep at a fixed token count: N = 512 .. 16384 with
    B = 16384 / N, H = 16, d = 64 and 128, causal and not; forward and backward
    timed with HIP events (inputs: seeded normal bf16 drawn on the GPU). Points
    whose forward is HBM-bound (N / 4 FLOP per byte causal, N / 2 not, below
    the 314.6 FLOP/B ridge) also get a cold-cache forward time, with a 512 MiB
    write before each call to evict L2 and the memory-side cache."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    ridge = PEAK_BF16 * 1e12 / (PEAK_HBM * 1e9)

    def timed(fn, cold=False):
        for _ in range(warmup):
            fn()
        times = []
        for _ in range(steps):
            if cold:
                flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        return call_stats(times)

    g = torch.Generator(device=dev)
    pts = []
    for d in (64, 128):
        for n in (512, 1024, 2048, 4096, 8192, 16384):
            b = 16384 // n
            g.manual_seed(100 + int(round(math.log2(n))))
            q, k, v, do = (torch.randn((b, 16, n, d), generator=g, device=dev).to(torch.bfloat16) for _ in range(4))
            ws = torch.empty(fa.bwd_workspace_bytes(b, 16, n, d), dtype=torch.uint8, device=dev)
            for causal in (True, False):
                o, lse = fa.fwd(q, k, v, causal=causal)
                sf = timed(lambda: fa.fwd(q, k, v, causal=causal, out=o, lse=lse))
                sb = timed(lambda: fa.bwd(q, k, v, o, do, lse, causal=causal, workspace=ws))
                tf, tb = sf["ms_median"], sb["ms_median"]
                fl = fwd_flops(b, 16, n, d, causal)
                by = fwd_bytes(b, 16, n, d)
                ent = {"N": n, "B": b, "H": 16, "d": d, "causal": causal,
                       "fwd_ms": tf, "fwd_tflops": fl / (tf * 1e-3) / 1e12, "fwd_gbps": by / (tf * 1e-3) / 1e9,
                       "bwd_ms": tb, "bwd_tflops": 2.5 * fl / (tb * 1e-3) / 1e12, "fwd_calls": sf, "bwd_calls": sb}
                ent["fwd_frac"] = ent["fwd_tflops"] / PEAK_BF16
                ent["bwd_frac"] = ent["bwd_tflops"] / PEAK_BF16
                ent["fwd_bound"] = "hbm" if fl / by < ridge else "mfma"
                if ent["fwd_bound"] == "hbm":
                    sc_ = timed(lambda: fa.fwd(q, k, v, causal=causal, out=o, lse=lse), cold=True)
                    tc = sc_["ms_median"]
                    ent["fwd_ms_cold"] = tc
                    ent["fwd_cold_calls"] = sc_
                    ent["fwd_gbps_cold"] = by / (tc * 1e-3) / 1e9
                    ent["fwd_hbm_frac_cold"] = ent["fwd_gbps_cold"] / PEAK_HBM
                log("sweep d=%d N=%5d B=%2d causal=%d: fwd %.3f ms %.0f TFLOP/s, bwd %.3f ms %.0f TFLOP/s%s"
                    % (d, n, b, causal, tf, ent["fwd_tflops"], tb, ent["bwd_tflops"],
                       (", cold fwd %.0f GB/s" % ent["fwd_gbps_cold"]) if "fwd_gbps_cold" in ent else ""))
                pts.append(ent)
            del q, k, v, do, ws, o, lse
    return pts


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-heads", type=int, default=12)
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the sequence-length sweep (N = 512 .. 16384 at 16384 tokens, d = 64 / 128)")
    ap.add_argument("--no-widened", action="store_true",
                    help="skip the widened rows (GQA, layout, window, ALiBi, cross-attention, d=64/256)")
    ap.add_argument("--only", default=None,
                    help="time only this kernel (fa_fwd, fa_bwd, fa_quant_fp8, fa_fwd_fp8) or 'copy[MiB]', "
                         "a plain device copy (default 256 MiB) used to calibrate rocprofv3 byte counters")
    ap.add_argument("--seq", type=int, default=None,
                    help="with --only: run the timed kernel at sequence length SEQ and batch 16384 // SEQ "
                         "(the sweep's token count) instead of the headline shape, for profiling the short, "
                         "bandwidth-bound shapes")
    ap.add_argument("--head-dim", type=int, default=None,
                    help="with --only: run the timed kernel at this head dim (64 or 128) instead of 128")
    args = ap.parse_args()
    if args.head_dim is not None:
        if args.only is None or args.only.startswith("copy") or args.head_dim not in (64, 128):
            ap.error("--head-dim profiles one kernel at d = 64 or 128: give --only as well")
        global D
        D = args.head_dim
    if args.seq is not None:
        if args.only is None or args.only.startswith("copy"):
            ap.error("--seq profiles one kernel: give --only fa_fwd, fa_bwd, fa_quant_fp8 or fa_fwd_fp8")
        global B, N
        N, B = args.seq, max(1, 16384 // args.seq)
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(the (batch, head) pairs would shard with no communication)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_104_amd as fa
    import fa_inputs

    fa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating inputs B=%d H=%d N=%d d=%d" % (B, H, N, D))
    host = fa_inputs.attention_inputs(B, H, N, D, seed=3, with_do=True)
    q, k, v, do = (torch.from_numpy(host[n]).to(torch.bfloat16).to(dev) for n in ("q", "k", "v", "do"))
    h8 = fa_inputs.attention_inputs(B, H, N, D, seed=5, outliers=True)
    q5, k5, v5 = (torch.from_numpy(h8[n]).to(torch.bfloat16).to(dev) for n in ("q", "k", "v"))
    signs = torch.from_numpy(fa_inputs.hadamard_signs()).to(dev)
    del host, h8
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, D), dtype=torch.uint8, device=dev)

    # which kernels exist
    def available(fn):
        try:
            fn()
            torch.cuda.synchronize()
            return True
        except fa.FAError as e:
            log("left out of the step: %s" % e)
            return False

    have_fwd = available(lambda: fa.fwd(q, k, v, causal=True, out=o, lse=lse))
    have_bwd = have_fwd and available(lambda: fa.bwd(q, k, v, o, do, lse, causal=True, workspace=ws))
    have_q8 = available(lambda: fa.quant_fp8(q5, signs))
    have_f8 = False
    if have_q8:
        q8, qs = fa.quant_fp8(q5, signs)
        k8, ks = fa.quant_fp8(k5, signs)
        v8, vs = fa.quant_fp8(v5, None)
        have_f8 = available(lambda: fa.fwd_fp8(q8, k8, v8, qs, ks, vs, causal=True))

    stream = torch.cuda.current_stream()
    kernels = []  # (name, callable, flops, bytes, peak)
    if have_fwd:
        kernels.append(("fa_fwd", lambda: fa.fwd(q, k, v, causal=True, out=o, lse=lse),
                        fwd_flops(B, H, N, D), fwd_bytes(B, H, N, D), PEAK_BF16))
    if have_bwd:
        kernels.append(("fa_bwd", lambda: fa.bwd(q, k, v, o, do, lse, causal=True, workspace=ws),
                        2.5 * fwd_flops(B, H, N, D), bwd_bytes(B, H, N, D), PEAK_BF16))
    if have_q8:
        def quant3():
            fa.quant_fp8(q5, signs)
            fa.quant_fp8(k5, signs)
            fa.quant_fp8(v5, None)
        kernels.append(("fa_quant_fp8 x3", quant3, 0.0, 3 * quant_bytes(B, H, N, D), None))
    if have_f8:
        kernels.append(("fa_fwd_fp8", lambda: fa.fwd_fp8(q8, k8, v8, qs, ks, vs, causal=True),
                        fwd_flops(B, H, N, D), fwd_bytes(B, H, N, D, 1), PEAK_FP8))
    if args.only is not None and args.only.startswith("copy"):
        mib = int(args.only[4:] or 256)
        src = torch.full((mib << 20,), 7, dtype=torch.uint8, device=dev)  # written, so its reads are real
        dst = torch.zeros_like(src)
        kernels = [("copy %d MiB" % mib, lambda: dst.copy_(src), 0.0, 2.0 * src.numel(), None)]
    elif args.only is not None:
        kernels = [k for k in kernels if k[0].startswith(args.only)]
    if not kernels:
        raise RuntimeError("no kernel of the path is available")

    for _ in range(args.warmup):
        for _, fn, *_r in kernels:
            fn()
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in kernels] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        for i, (_, fn, *_r) in enumerate(kernels):
            ev[s][i][0].record(stream)
            fn()
            ev[s][i][1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps

    breakdown = {}
    dom = None
    for i, (name, _, flops, nbytes, peak) in enumerate(kernels):
        times = [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)]
        avg = float(np.mean(times))
        ent = {"ms_avg": avg, "ms_median": float(np.median(times)), "ms_min": float(np.min(times))}
        if flops:
            ent["tflops"] = flops / (avg * 1e-3) / 1e12
            ent["pct_of_peak"] = 100.0 * ent["tflops"] / peak
        ent["gbps"] = nbytes / (avg * 1e-3) / 1e9
        if not flops:
            ent["pct_of_hbm_peak"] = 100.0 * ent["gbps"] / PEAK_HBM
        breakdown[name] = ent
        if dom is None or avg > breakdown[dom[0]]["ms_avg"]:
            dom = (name, flops, nbytes, peak)

    name, flops, nbytes, peak = dom
    if peak:
        achieved = breakdown[name]["tflops"]
        traffic = None
        if name == "fa_bwd":  # one C-ABI call: dq_kernel (which also forms D), dkdv_kernel
            traffic = measured_traffic(os.path.join(ROOT, "profiles", "fa_bwd_n8192_d128_causal_hbm_bytes.md"))
        roofline = {"kernel": name, "bound": "mfma", "achieved": achieved, "peak": peak,
                    "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic,
                    "per_launch_flops": flops, "avg_launch_ms": breakdown[name]["ms_avg"],
                    "algorithmic_bytes": nbytes,
                    "how": "per-launch algorithmic FLOPs / average of the launch's HIP-event times on its "
                           "stream over the timed steps"}
    else:
        achieved = breakdown[name]["gbps"]
        roofline = {"kernel": name, "bound": "hbm", "achieved": achieved, "peak": PEAK_HBM,
                    "unit": "GB/s", "frac": achieved / PEAK_HBM, "traffic": None}

    # The metric: bf16 forward + backward only, from their own times in the steps.
    value, frac_bf16 = None, None
    if "fa_fwd" in breakdown and "fa_bwd" in breakdown:
        bf16_ms = breakdown["fa_fwd"]["ms_avg"] + breakdown["fa_bwd"]["ms_avg"]
        value = 3.5 * fwd_flops(B, H, N, D) / (bf16_ms * 1e-3) / 1e12
        frac_bf16 = value / PEAK_BF16

    # Shader clock while the bf16 kernels run (outside the timed steps), and the
    # utilisation against the MFMA peak at that clock (the 2516.6 TFLOP/s spec
    # assumes 2.4 GHz).
    sclk = None
    if args.only is None and value is not None:
        sclk = sample_sclk(lambda: (fa.fwd(q, k, v, causal=True, out=o, lse=lse),
                                    fa.bwd(q, k, v, o, do, lse, causal=True, workspace=ws)))
        if sclk.get("mhz_median"):
            sclk["frac_of_peak_at_this_clock"] = frac_bf16 * 2400.0 / sclk["mhz_median"]
            sclk["roofline_frac_at_this_clock"] = roofline["frac"] * 2400.0 / sclk["mhz_median"]
        log("sclk: %s" % sclk)

    # Context, outside the timed step: the rate of a large bf16 GEMM from the
    # vendor library on this machine, a practical ceiling for dense bf16 MFMA work.
    gemm = None
    if args.only is None:
        a_ = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        b_ = torch.randn(8192, 8192, device=dev).to(torch.bfloat16)
        for _ in range(3):
            torch.matmul(a_, b_)
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(10):
            torch.matmul(a_, b_)
        g1.record(stream)
        torch.cuda.synchronize()
        gms = g0.elapsed_time(g1) / 10
        gemm = {"what": "torch.matmul bf16 8192x8192x8192 (hipBLASLt), 10 calls after 3 warm-ups",
                "ms": gms, "tflops": 2.0 * 8192 ** 3 / (gms * 1e-3) / 1e12,
                "frac_of_peak": 2.0 * 8192 ** 3 / (gms * 1e-3) / 1e12 / PEAK_BF16}
        del a_, b_

    wid = None
    if not args.no_widened and args.only is None and have_bwd:
        wid = widened(fa, dev, q, k, v, do)
    f8x = None
    if not args.no_widened and args.only is None and have_f8:
        f8x = fp8_exp_modes(fa, q8, k8, v8, qs, ks, vs, fwd_flops(B, H, N, D))
    swp = None
    if not args.no_sweep and args.only is None and have_bwd:
        swp = sweep(fa, dev)

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on %d heads" % args.cpu_heads)
        cpu = cpu_baseline(args.cpu_heads)

    out = {
        "metric": METRIC,
        "value": value,
        "pct_of_peak": None if frac_bf16 is None else 100.0 * frac_bf16,
        "value_definition": "bf16 fa_fwd + fa_bwd: 3.5 x 4 B H N^2 d / 2 algorithmic causal FLOPs over the sum "
                            "of the two calls' average HIP-event times inside the timed steps; the step also "
                            "runs the fp8 leg (3 x fa_quant_fp8 + fa_fwd_fp8), reported under breakdown",
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal attention B=%d H=%d N=%d d=%d (bf16; fp8 leg with 0.1%% x20 "
                               "outliers, Hadamard-rotated Q/K)" % (B, H, N, D),
                   "B": B, "H": H, "N": N, "d": D, "causal": True,
                   "step": [k[0] for k in kernels]},
        "breakdown": breakdown,
        "roofline": roofline,
        "sclk": sclk,
        "cpu_baseline": cpu,
        "context": {"library_bf16_gemm": gemm},
        "widened": wid,  # each row: median of 10 calls, with min / max
        "fp8_exp_modes": f8x,  # software 2^x in the fp8 forward's softmax: none, 1 in 4, all
        "sweep": swp,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
