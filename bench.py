"""Benchmark of the int8-state gated delta-rule decode step on one MI355X.

Workload (the one the headline metric is quoted on): one decode token for
each of B=64 sequences x H=32 heads, d_k = d_v = 128, window W = 64, bf16
q/k/v, int8 state (N(0, 0.5) entries quantized per row) and per-sequence
window fills drawn from U{0..63} holding fp32 (k, v, alpha, beta).

A "step" is one gdnq_decode_step launch over the whole batch.  The state of
one step (codes, scales, buffer: ~106 MB) fits in the 256 MB Infinity Cache,
so steps rotate over `--replicas` copies of it (16 by default, ~1.7 GB).
With the buffer read by nontemporal loads, the codes alone (35 MB per
replica) would otherwise stay in that cache across a short rotation (with 4
replicas a step took 25 us instead of 28); 16 replicas hold 550 MB of codes,
so every step reads its state cold from HBM, as a step of one layer of a
model does between the other layers' work.  Fills advance by one per step
per replica (f -> f+1, or 0 after a window close), as in a real decode loop.

Prints ONE JSON line.  `value` = tokens/s (B tokens per step); the roofline
object uses the algorithmic bytes of each launch (computed from the realized
fills) divided by the measured launch time; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload.  The GDN and SSD
chunked-prefill measurements follow as secondary objects (`--no-prefill`
skips them).
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

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2516.6

B, H, DK, DV, W = 64, 32, 128, 128, 64


def decode_bytes_per_head(f, W=W, dk=DK, dv=DV, e_in=2, e_out=2, e_buf=4, state_bits=8):
    """Algorithmic HBM bytes of one decode token for one head with fill f:
    the state's code rows (dk * state_bits / 8 bytes each) + scales read, f
    buffered writes read (k, v at e_buf bytes per entry, alpha and beta fp32,
    plus two fp32 scales per write with the FP8 buffer, e_buf = 1), the
    token's q, k, v, alpha, beta read, o written, and either the token's
    write appended (window open) or the requantized rows + scales written
    (window close)."""
    w = e_buf * (dk + dv) + 8 + (8 if e_buf == 1 else 0)
    state = dv * dk * state_bits // 8 + 4 * dv
    rd = state + w * f + e_in * (2 * dk + dv) + 8
    wr = e_out * dv + (w if f + 1 < W else state)
    return rd + wr


def decode_bytes(fills, heads=H, e_buf=4, state_bits=8):
    per_seq_fill = 8  # fill_in read + fill_out write
    table = np.array([decode_bytes_per_head(f, e_buf=e_buf, state_bits=state_bits) for f in range(W)],
                     np.int64)
    return int(heads * table[np.asarray(fills, np.int64)].sum() + per_seq_fill * len(fills))


def decode_schedule_bytes(fills0, n_steps, heads=H, e_buf=4, state_bits=8):
    """Algorithmic bytes of each of n_steps consecutive launches of one state
    whose fills start at fills0 and advance by one per step (0 after a
    window close); computed before anything is timed."""
    fills = np.asarray(fills0, np.int64).copy()
    out = []
    for _ in range(n_steps):
        out.append(decode_bytes(fills, heads=heads, e_buf=e_buf, state_bits=state_bits))
        fills = np.where(fills + 1 == W, 0, fills + 1)
    return out


# the sources of the decode kernel (a traffic summary is stale once they change)
DECODE_SOURCES = ["decode.hip", "decode_impl.h", "device_common.h"]
SLIDING_SOURCES = ["decode_sliding.hip", "decode_impl.h", "device_common.h"]


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "quantized_recurrent_state_gdnq_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(name, kernel_sources, per_launch_units):
    """Measured HBM bytes per launch from a committed rocprofv3 counter summary,
    or None when the summary is absent or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != source_hash(*kernel_sources):
        return None
    return d.get("bytes_per_launch")


def host_cpu_info():
    """The host the CPU oracle runs on: model, cores this process may use,
    logical CPUs, and the BLAS threads numpy runs with."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
    except Exception:
        pass
    return {"cpu_model": model, "affinity_cores": affinity, "cpu_count": os.cpu_count(),
            "blas_threads": blas}


def _cores_used(info):
    """Threads the oracle can use: numpy's BLAS threads, within the affinity."""
    b = info["blas_threads"] or 1
    return min(b, info["affinity_cores"] or b)


def cpu_baseline_prefill(kind, seconds_cap=20.0):
    """The CPU oracle on one whole sequence of a prefill workload (all heads,
    every token): GDN B=4 T=8192 H=16 (one of the 4 sequences), SSD B=2
    T=4096 H=80 with rotated int8 q/k (one of the 2 sequences)."""
    import oracle
    import workloads as wl

    if kind == "gdn":
        x = wl.gdn_prefill(B=1, T=8192, H=16, dk=128, dv=128, seed=0)
        t0 = time.perf_counter()
        oracle.prefill(x["q"], x["k"], x["v"], x["alpha"], x["beta"], W=64)
        el = time.perf_counter() - t0
        T, sample = 8192, "1 of 4 sequences (all 16 heads, all 8192 tokens)"
    else:
        x = wl.ssd_prefill(B=1, T=4096, H=80, dk=128, dv=64, seed=0)
        t0 = time.perf_counter()
        oracle.prefill(x["q"], x["k"], x["v"], x["alpha"], None, W=None, kind="ssd", rot=True,
                       qk_int8=True)
        el = time.perf_counter() - t0
        T, sample = 4096, "1 of 2 sequences (all 80 heads, all 4096 tokens)"
    info = host_cpu_info()
    return {"value": round(T / el, 1), "unit": "tokens/s", "cores": _cores_used(info), "kind": "oracle",
            "sample": f"{sample}, numpy fp32 oracle token by token ({el:.1f} s)", **info}


def cpu_baseline_decode(seconds=12.0):
    """The CPU oracle on a bounded sample: the first sequences of the same
    workload, one decode call at a time, until `seconds` have elapsed."""
    import oracle
    import workloads as wl

    nseq = 4
    d = wl.decode_batch(B=nseq, H=H, dk=DK, dv=DV, W=W, seed=0)
    codes, scales = oracle.quantize_rows(d["state"])
    bufs = [d["buf_k"], d["buf_v"], d["buf_alpha"], d["buf_beta"]]
    fill = d["fill"]
    t0 = time.perf_counter()
    steps = 0
    while True:
        x = wl.decode_tokens(B=nseq, H=H, dk=DK, dv=DV, step=steps, seed=1)
        out = oracle.decode_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], codes, scales,
                                 *bufs, fill, W)
        _, codes, scales, *bufs, fill = out
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    info = host_cpu_info()
    return {"value": nseq * steps / el, "unit": "tokens/s", "cores": _cores_used(info), "kind": "oracle",
            "sample": f"{nseq} of {B} sequences x {H} heads, {steps} consecutive decode steps "
                      f"({el:.1f} s), numpy fp32 oracle", **info}


def bench_decode(args, torch, ops, wl, rep_count, buf_dtype=None, state_bits=8, wht=False):
    """Timed decode steps; buf_dtype torch.bfloat16 runs the low-precision
    window buffer (writes stored as bf16) on the same workload; state_bits 4
    the uniform 4-bit state; wht=True the rotation of q and k (the state and
    buffered keys taken as in the rotated basis)."""
    buf_dtype = buf_dtype or torch.float32
    e_buf = {torch.float32: 4, torch.bfloat16: 2, torch.float8_e4m3fn: 1}[buf_dtype]
    dev = torch.device("cuda:0")
    d = wl.decode_batch(B=B, H=H, dk=DK, dv=DV, W=W, seed=0)
    state = torch.from_numpy(d["state"]).to(dev)
    codes0, scales0 = ops.quantize_state(state, state_bits=state_bits)  # the library's own codec
    del state
    reps = []
    for i in range(rep_count):
        rep = ops.DecodeState(codes0.clone(), scales0.clone(), W,
                              fill=torch.from_numpy(d["fill"]).to(dev), buf_dtype=buf_dtype,
                              state_bits=state_bits, wht=wht)
        if buf_dtype == torch.float8_e4m3fn:  # E4M3 vector pairs: scale absmax/448, codes by torch's cast
            for dst, sdst, x in ((rep.buf_k, rep.buf_k_scale, d["buf_k"]), (rep.buf_v, rep.buf_v_scale, d["buf_v"])):
                t = torch.nan_to_num(torch.from_numpy(x).to(dev))
                sc = t.abs().amax(dim=-1) / 448.0
                dst.copy_((t / torch.where(sc > 0, sc, 1.0)[..., None]).to(torch.float8_e4m3fn))
                sdst.copy_(sc)
        else:
            rep.buf_k.copy_(torch.from_numpy(d["buf_k"]).to(buf_dtype))
            rep.buf_v.copy_(torch.from_numpy(d["buf_v"]).to(buf_dtype))
        rep.buf_alpha.copy_(torch.from_numpy(d["buf_alpha"]))
        rep.buf_beta.copy_(torch.from_numpy(d["buf_beta"]))
        reps.append(rep)
    host_fills = [d["fill"].astype(np.int64).copy() for _ in range(rep_count)]
    # per replica, token input buffers (bf16 q/k/v, fp32 alpha/beta) bound once:
    # the launch path then only passes prebuilt arguments, as a serving loop would
    o = torch.empty((B, H, DV), dtype=torch.bfloat16, device=dev)
    launchers = []
    for s in range(rep_count):
        x = wl.decode_tokens(B=B, H=H, dk=DK, dv=DV, step=s, seed=1)
        tok = [torch.from_numpy(x["q"]).to(dev).bfloat16(),
               torch.from_numpy(x["k"]).to(dev).bfloat16(),
               torch.from_numpy(x["v"]).to(dev).bfloat16(),
               torch.from_numpy(x["alpha"]).to(dev), torch.from_numpy(x["beta"]).to(dev)]
        launchers.append((reps[s].bind(*tok, o=o), tok))

    # every launch's algorithmic bytes, from the fills each replica will have,
    # before anything is timed: the timed loop only launches
    n_all = args.warmup + args.steps
    per_rep = [decode_schedule_bytes(host_fills[r], (n_all + rep_count - 1 - r) // rep_count,
                                     e_buf=e_buf, state_bits=state_bits) for r in range(rep_count)]
    step_bytes = [per_rep[i % rep_count][i // rep_count] for i in range(n_all)]
    total_bytes = sum(step_bytes[args.warmup:])
    launch = [lc[0] for lc in launchers]

    for i in range(args.warmup):
        launch[i % rep_count]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.warmup, n_all):
        launch[i % rep_count]()
    e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ms_step = ms / args.steps
    tokens_s = B * args.steps / (ms / 1e3)
    bytes_launch = total_bytes / args.steps
    gbps = bytes_launch / (ms_step * 1e-3) / 1e9
    return {"ms_per_step": ms_step, "tokens_s": tokens_s, "bytes_per_launch": bytes_launch,
            "gbps": gbps}


def bench_decode_long(torch, ops, wl, B2=256, steps=1024, warmup=16, n_tok=8, n_rep=4):
    """Large-batch decode: B2 sequences x H heads, `steps` consecutive decode
    steps of each of n_rep copies of one state (every sequence crosses window
    ends), the copies taken in turn so that a step reads its state cold (one
    copy, 675 MB, would keep its 138 MB of codes in the Infinity Cache from
    one step to the next); all n_rep * steps launches timed end to end.
    n_tok token sets are bound once per copy and reused in turn."""
    dev = torch.device("cuda:0")
    d = wl.decode_batch(B=B2, H=H, dk=DK, dv=DV, W=W, seed=2)
    codes, scales = ops.quantize_state(torch.from_numpy(d["state"]).to(dev))
    fill0 = torch.from_numpy(d["fill"]).to(dev)
    sts = []
    for r in range(n_rep):
        st = ops.DecodeState(codes.clone(), scales.clone(), W, fill=fill0.clone())
        if r == 0:
            st.buf_k.copy_(torch.from_numpy(d["buf_k"]))
            st.buf_v.copy_(torch.from_numpy(d["buf_v"]))
            st.buf_alpha.copy_(torch.from_numpy(d["buf_alpha"]))
            st.buf_beta.copy_(torch.from_numpy(d["buf_beta"]))
        else:
            for name in ("buf_k", "buf_v", "buf_alpha", "buf_beta"):
                getattr(st, name).copy_(getattr(sts[0], name))
        sts.append(st)
    fills = d["fill"].astype(np.int64)
    del d, codes, scales
    o = torch.empty((B2, H, DV), dtype=torch.bfloat16, device=dev)
    launchers = []  # [replica][token set]
    toks = []
    for s in range(n_tok):
        x = wl.decode_tokens(B=B2, H=H, dk=DK, dv=DV, step=s, seed=3)
        toks.append([torch.from_numpy(x["q"]).to(dev).bfloat16(), torch.from_numpy(x["k"]).to(dev).bfloat16(),
                     torch.from_numpy(x["v"]).to(dev).bfloat16(), torch.from_numpy(x["alpha"]).to(dev),
                     torch.from_numpy(x["beta"]).to(dev)])
    for st in sts:
        launchers.append([st.bind(*tok, o=o) for tok in toks])
    # every copy advances through the same fills
    step_bytes = decode_schedule_bytes(fills, warmup + steps)
    total = n_rep * sum(step_bytes[warmup:])
    for i in range(warmup):
        for r in range(n_rep):
            launchers[r][i % n_tok]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        for r in range(n_rep):
            launchers[r][i % n_tok]()
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1)
    n_launch = n_rep * steps
    gbps = total / (ms * 1e-3) / 1e9
    del sts, launchers, toks, o
    torch.cuda.empty_cache()
    return {
        "workload": f"{steps} consecutive decode steps of each of {n_rep} copies of one state (taken in "
                    f"turn: every step reads its state cold), B={B2} H={H} d_k=d_v={DK} W={W}, int8 state, "
                    "fp32 window buffer, fills from U{0..63} advancing (every sequence crosses window "
                    "ends), timed end to end",
        "ms_total": round(ms, 3), "ms_per_step": round(ms / n_launch, 5),
        "tokens_s": round(B2 * n_launch / (ms * 1e-3), 1), "gbps": round(gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic("decode_b256_h32_1024steps_traffic.json", DECODE_SOURCES, 1),
                     "algorithmic_bytes_per_launch": int(total / n_launch)},
    }


def sliding_bytes_per_head(fill, W, dk=DK, dv=DV, e_in=2, e_out=2):
    """Algorithmic HBM bytes of one sliding-window decode token for one head:
    the historical rows + scales read and rewritten (requantized every
    token), the n = min(fill, W) window writes read (fp32 k, v, alpha,
    beta), the token's q, k, v, alpha, beta read, o written, and the token's
    write stored in the ring."""
    n = min(fill, W)
    state = dv * dk + 4 * dv
    w = 4 * (dk + dv) + 8
    return 2 * state + n * w + e_in * (2 * dk + dv) + 8 + e_out * dv + w


def bench_decode_sliding(args, torch, ops, wl, rep_count, Ws=8):
    """The Pure-Write sliding-window decode (GDNQ_FLAG_SLIDING) on the decode
    batch: B=64, H=32, d=128, window of Ws writes, ring fills drawn
    U{0..2Ws-1} (about half the sequences with a full window), bf16 q/k/v,
    rotating state replicas.  Every token rewrites every head's codes."""
    dev = torch.device("cuda:0")
    g = np.random.default_rng(70)
    fills0 = g.integers(0, 2 * Ws, B).astype(np.int32)
    d = wl.decode_batch(B=B, H=H, dk=DK, dv=DV, W=Ws, seed=71, fill=np.minimum(fills0, Ws - 1), poison=False)
    state = torch.from_numpy(d["state"]).to(dev)
    codes0, scales0 = ops.quantize_state(state)
    del state
    o = torch.empty((B, H, DV), dtype=torch.bfloat16, device=dev)
    launchers, fills = [], []
    for r in range(rep_count):
        st = ops.DecodeState(codes0.clone(), scales0.clone(), Ws, fill=torch.from_numpy(fills0).to(dev),
                             sliding=True)
        for name in ("buf_k", "buf_v", "buf_alpha", "buf_beta"):
            getattr(st, name).copy_(torch.from_numpy(d[name]))
        x = wl.decode_tokens(B=B, H=H, dk=DK, dv=DV, step=r, seed=72)
        tok = [torch.from_numpy(x["q"]).to(dev).bfloat16(), torch.from_numpy(x["k"]).to(dev).bfloat16(),
               torch.from_numpy(x["v"]).to(dev).bfloat16(), torch.from_numpy(x["alpha"]).to(dev),
               torch.from_numpy(x["beta"]).to(dev)]
        launchers.append((st.bind(*tok, o=o), tok))
        fills.append(fills0.astype(np.int64).copy())
    n_all = args.warmup + args.steps
    step_bytes = []
    for i in range(n_all):
        f = fills[i % rep_count]
        step_bytes.append(int(sum(H * sliding_bytes_per_head(int(x), Ws) + 8 for x in f)))
        fills[i % rep_count] = np.where(f < Ws, f + 1, Ws + (f - Ws + 1) % Ws)
    total = sum(step_bytes[args.warmup:])
    launch = [lc[0] for lc in launchers]
    for i in range(args.warmup):
        launch[i % rep_count]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.warmup, n_all):
        launch[i % rep_count]()
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    gbps = total / args.steps / (ms * 1e-3) / 1e9
    return {
        "workload": f"Pure-Write sliding-window decode step B={B} H={H} d_k=d_v={DK} window of {Ws} writes, "
                    f"ring fills U{{0..{2 * Ws - 1}}}, bf16 q/k/v, int8 historical state requantized every "
                    f"token, fp32 window, {rep_count} state replicas",
        "ms_per_step": round(ms, 5), "tokens_s": round(B / (ms * 1e-3), 1), "gbps": round(gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "traffic": load_traffic("decode_b64_h32_sliding_traffic.json", SLIDING_SOURCES, 1),
                     "algorithmic_bytes_per_launch": int(total / args.steps)},
    }


def gdn_prefill_flops(B, T, H, dk=DK, dv=DV, C=64):
    """Useful FLOPs of the chunked GDN prefill, counted as full C x C tiles as
    MFMA executes them: per token-head 6 dk dv (K S0^T, Q S0^T and the state
    update U^T K, one multiply-add each) + C (6 dk + 4 dv) (K K^T, T K and
    Q K^T over dk; T V and (L o Q K^T) U over dv).  180,224 at d = 128,
    C = 64."""
    return 2.0 * B * T * H * (3 * dk * dv + C * (3 * dk + 2 * dv))


def gdn_prefill_flops_triangular(B, T, H, dk=DK, dv=DV, C=64):
    """The same products counted over their causal (triangular) parts only,
    plus the C^3/6 of the inverse: what the algorithm needs at the least."""
    tri, tri0 = C * (C + 1) // 2, C * (C - 1) // 2
    macs = dk * tri0 + C ** 3 / 6 + 3 * C * dk * dv + dv * tri + dk * tri + dv * tri
    return 2.0 * macs * B * (T // C) * H


def ssd_prefill_flops(B, T, H, dk=128, dv=64, C=64):
    """Useful FLOPs of the chunked SSD prefill as full tiles: per token-head
    4 dk dv (Q S0^T and the state update) + C (2 dk + 2 dv) (Q K^T and
    M V).  57,344 at dk = 128, dv = 64, C = 64 (the rotation and operand
    quantization are O(d log d) per row and not counted)."""
    return 2.0 * B * T * H * (2 * dk * dv + C * (dk + dv))


def gdn_prefill_bytes(B, T, H, dk=DK, dv=DV):
    """Algorithmic HBM bytes: bf16 q, k, v and fp32 alpha, beta read, bf16 o
    written, the final int8 rows + scales written (zero initial state)."""
    return B * T * H * (2 * (2 * dk + dv) + 8 + 2 * dv) + B * H * dv * (dk + 4)


def ssd_prefill_bytes(B, T, H, dk=128, dv=64):
    """bf16 q, k, v and fp32 a read, bf16 o written, the final fp32 state written."""
    return B * T * H * (2 * (2 * dk + dv) + 4 + 2 * dv) + B * H * dv * dk * 4


# the sources of each prefill's kernels (GDN, SSD)
PREFILL_SOURCES = {False: ["prefill_gdn.hip", "device_common.h", "mfma.h"],
                   True: ["prefill_ssd.hip", "device_common.h", "mfma.h"]}


W_LONG = 128  # the long-window prefill line


def bench_prefill(torch, ops, wl, steps=20, warmup=3, with_cpu=True):
    """Secondary: GDN chunked prefill B=4, T=8192, H=16, d=128, C=W=64 (bf16
    output, zero initial state); SSD prefill B=2, T=4096, H=80, d_k=128,
    d_v=64 with WHT-rotated int8 q/k (bf16 output); the GDN hand-over to
    decode (T = 8192 + 37); a packed batch of 32 sequences of seeded lengths
    U{1..2047} (H=16); resuming 4 decode states at fills U{0..63} with
    8192 new tokens each; the GDN prefill with q, k rotated; and with
    windows of 128 tokens.  Inputs and workspace are resident before timing;
    each call is timed whole (all its kernels)."""
    dev = torch.device("cuda:0")
    res = {}
    names = ["gdn_prefill", "ssd_prefill", "gdn_prefill_handoff", "gdn_prefill_varlen",
             "gdn_prefill_resume", "gdn_prefill_wht", "gdn_prefill_w128"]
    H16, d = 16, 128
    state_bytes = d * (d + 4)  # int8 rows + fp32 scales of one head

    def t(x, bf16=False):
        y = torch.from_numpy(x).to(dev)
        return y.bfloat16() if bf16 else y

    for name in names:
        ssd = name == "ssd_prefill"
        if name == "gdn_prefill_varlen":
            lengths = np.random.default_rng(5).integers(1, 2048, 32)
            x = wl.gdn_prefill_varlen(lengths, H=H16, dk=d, dv=d, seed=0)
        elif name == "ssd_prefill":
            x = wl.ssd_prefill(B=2, T=4096, H=80, dk=128, dv=64, seed=0)
        else:
            T = 8192 + 37 if name == "gdn_prefill_handoff" else 8192
            x = wl.gdn_prefill(B=4, T=T, H=H16, dk=d, dv=d, seed=0)
        q, k, v = t(x["q"], True), t(x["k"], True), t(x["v"], True)
        a = t(x["alpha"])
        bt = None if ssd else t(x["beta"])
        dk, dv = q.shape[-1], v.shape[-1]
        Hh = q.shape[-2]
        extra_bytes = 0
        if name == "gdn_prefill_varlen":
            cu = t(x["cu_seqlens"])
            N, nseq = int(q.shape[0]), len(lengths)
            chunks = int(sum((int(n) + 63) // 64 for n in lengths))
            o = torch.empty((N, Hh, dv), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(ops.prefill_varlen_workspace_size(q, v, nseq), dtype=torch.uint8, device=dev)
            _, st = ops.prefill_varlen(q, k, v, a, bt, cu, o=o, workspace=ws)

            def call():
                ops.prefill_varlen(q, k, v, a, bt, cu, o=o, state=st, workspace=ws)
            workload = (f"{nseq} packed sequences of seeded lengths U{{1..2047}} ({N} tokens), H={Hh} "
                        f"d_k={dk} d_v={dv} chunk=window=64, int8 state, each handed over to decode")
            tokens = N
        elif name == "gdn_prefill_resume":
            Bq, T = q.shape[0], q.shape[1]
            nseq, N = Bq, Bq * T
            g = np.random.default_rng(6)
            fills = g.integers(0, 64, Bq).astype(np.int32)
            S = (g.standard_normal((Bq, Hh, dv, dk)) * 0.5).astype(np.float32)
            codes = torch.empty((Bq, Hh, dv, dk), dtype=torch.int8, device=dev)
            scales = torch.empty((Bq, Hh, dv), dtype=torch.float32, device=dev)
            ops.quantize_state(t(S), codes, scales)
            st = ops.DecodeState(codes, scales, 64, fill=t(fills))
            for buf in (st.buf_k, st.buf_v):  # bf16 values, as decode stores from bf16 inputs
                buf.copy_(torch.nn.functional.normalize(torch.randn(buf.shape, device=dev), dim=-1)
                          .bfloat16().float())
            st.buf_alpha.fill_(0.95)
            st.buf_beta.fill_(0.5)
            chunks = int(sum((int(f) + T + 63) // 64 for f in fills))
            o = torch.empty((Bq, T, Hh, dv), dtype=torch.bfloat16, device=dev)
            ws = torch.empty(ops.prefill_resume_workspace_size(q, v, Bq), dtype=torch.uint8, device=dev)

            def call():  # T is whole windows, so every call starts at the same fills
                ops.prefill_resume(st, q, k, v, a, bt, o=o, workspace=ws)
            extra_bytes = nseq * Hh * state_bytes + int(fills.sum()) * Hh * (4 * (dk + dv) + 8)
            workload = (f"B={Bq} decode states at fills U{{0..63}} resumed with T={T} new tokens each, "
                        f"H={Hh} d_k={dk} d_v={dv} chunk=window=64, int8 state")
            tokens = N
        else:
            Bq, T = q.shape[0], q.shape[1]
            nseq, N = Bq, Bq * T
            chunks = Bq * ((T + 63) // 64)
            o = torch.empty((Bq, T, Hh, dv), dtype=torch.bfloat16, device=dev)
            if name == "gdn_prefill_handoff":  # the open last window (T mod 64 writes) goes to decode's buffer
                ws = torch.empty(ops.prefill_handoff_workspace_size(q, v), dtype=torch.uint8, device=dev)
                _, st = ops.prefill_handoff(q, k, v, a, bt, o=o, workspace=ws)

                def call():
                    ops.prefill_handoff(q, k, v, a, bt, o=o, state=st, workspace=ws)
            else:
                kw = dict(ssd=True, wht=True, int8_qk=True) if ssd else dict(window=W_LONG if name == "gdn_prefill_w128" else 64)
                if name == "gdn_prefill_wht":
                    kw["wht"] = True
                kw["workspace"] = torch.empty(ops.prefill_workspace_size(q, v, **kw), dtype=torch.uint8,
                                              device=dev)
                kw["o"] = o
                if ssd:
                    kw["state_f32"] = torch.empty((Bq, Hh, dv, dk), dtype=torch.float32, device=dev)
                else:
                    kw["codes"] = torch.empty((Bq, Hh, dv, dk), dtype=torch.int8, device=dev)
                    kw["scales"] = torch.empty((Bq, Hh, dv), dtype=torch.float32, device=dev)

                def call():
                    ops.prefill_chunked(q, k, v, a, bt, **kw)
            workload = (f"B={Bq} T={T} H={Hh} d_k={dk} d_v={dv} chunk=64"
                        + (" WHT+int8 q/k, fp32 state" if ssd else f" window={kw.get('window', 64)}, int8 state"
                           if name != "gdn_prefill_handoff" else " window=64, int8 state")
                        + (" (two chunks per window: the state stays fp32 at the chunk between window ends)"
                           if name == "gdn_prefill_w128" else "")
                        + (", q and k rotated (WHT) and rounded to bf16" if name == "gdn_prefill_wht" else "")
                        + (f", the last {T % 64} tokens' writes handed to decode's window buffer"
                           if name == "gdn_prefill_handoff" else ""))
            tokens = N
        del x
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            call()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1) / steps
        if ssd:
            flops = ssd_prefill_flops(1, 64 * chunks, Hh, dk, dv)
            nbytes = ssd_prefill_bytes(1, N, Hh, dk, dv) + (nseq - 1) * Hh * dv * dk * 4
        else:
            flops = gdn_prefill_flops(1, 64 * chunks, Hh, dk, dv)
            nbytes = gdn_prefill_bytes(1, N, Hh, dk, dv) + (nseq - 1) * Hh * state_bytes + extra_bytes
        tflops = flops / (ms * 1e-3) / 1e12
        gbps = nbytes / (ms * 1e-3) / 1e9
        res[name] = {
            "workload": workload,
            "ms": round(ms, 4), "tokens_s": round(tokens / (ms * 1e-3), 1),
            "tflops": round(tflops, 2), "gbps": round(gbps, 1),
            "flops_per_call": flops, "bytes_per_call": nbytes,
            "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                         "traffic": load_traffic(f"{name}_traffic.json", PREFILL_SOURCES[ssd], 1)},
            "roofline_mfma": {"bound": "mfma", "achieved": round(tflops, 2), "peak": BF16_PEAK_TFLOPS,
                              "unit": "TFLOP/s", "frac": round(tflops / BF16_PEAK_TFLOPS, 4)},
        }
        if not ssd:
            res[name]["flops_triangular_per_call"] = gdn_prefill_flops_triangular(1, 64 * chunks, Hh, dk, dv)
        if with_cpu and name in ("gdn_prefill", "ssd_prefill"):
            res[name]["cpu_baseline"] = cpu_baseline_prefill("ssd" if ssd else "gdn")
        del q, k, v, a, bt, o, call
        torch.cuda.empty_cache()
    return res


def copy_probe(torch, mib):
    """One plain device copy of `mib` MiB (read + write), the reference the
    HBM byte counters are scaled by."""
    dev = torch.device("cuda:0")
    src = torch.empty(mib * 1024 * 1024 // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replicas", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill measurements")
    ap.add_argument("--no-fp8-buffer", action="store_true", help="skip the FP8 window-buffer line")
    ap.add_argument("--no-state4", action="store_true", help="skip the 4-bit state line")
    ap.add_argument("--no-long-decode", action="store_true", help="skip the B=256, 1024-step decode line")
    ap.add_argument("--no-wht", action="store_true", help="skip the decode line with the rotation")
    ap.add_argument("--no-sliding", action="store_true", help="skip the sliding-window decode line")
    ap.add_argument("--no-bf16-buffer", action="store_true",
                    help="skip the decode measurement with the bf16 window buffer")
    ap.add_argument("--skip-decode", action="store_true",
                    help="profiling aid: time only the prefills (the printed line then has no decode value)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="profiling aid: run one plain copy of MIB MiB first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (this build runs on "
              "one GPU only).", file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as wl
    from quantized_recurrent_state_gdnq_amd import ops

    if args.copy_probe:
        copy_probe(torch, args.copy_probe)
    if args.skip_decode:
        print(json.dumps({"prefill": bench_prefill(torch, ops, wl, with_cpu=False)}), flush=True)
        return

    r = bench_decode(args, torch, ops, wl, max(1, args.replicas))
    traffic = load_traffic("decode_b64_h32_traffic.json", DECODE_SOURCES, 1)
    line = {
        "metric": "int8-state GDN decode tokens/s + achieved HBM GB/s; prefill tokens/s",
        "value": round(r["tokens_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"decode step B={B} H={H} d_k=d_v={DK} W={W} bf16 q/k/v, int8 "
                               f"state, fills U{{0..{W - 1}}}, {args.replicas} state replicas "
                               "(cold HBM and Infinity Cache)",
                   "state": "int8 codes + fp32 per-row scales", "window_buffer": "fp32"},
        "hbm_gbps": round(r["gbps"], 1),
        "roofline": {"bound": "hbm", "achieved": round(r["gbps"], 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(r["gbps"] / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(r["bytes_per_launch"])},
    }
    if not args.no_bf16_buffer:
        rb = bench_decode(args, torch, ops, wl, max(1, args.replicas), buf_dtype=torch.bfloat16)
        line["decode_bf16_buffer"] = {
            "workload": "the same decode step with the window buffer's keys and values stored "
                        "as bf16 (GDNQ_FLAG_BUF_BF16; lossless for bf16 inputs without WHT)",
            "ms_per_step": round(rb["ms_per_step"], 5),
            "tokens_s": round(rb["tokens_s"], 1),
            "gbps": round(rb["gbps"], 1),
            "roofline": {"bound": "hbm", "achieved": round(rb["gbps"], 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(rb["gbps"] / HBM_PEAK_GBPS, 4),
                         "traffic": load_traffic("decode_b64_h32_bf16buf_traffic.json",
                                                 DECODE_SOURCES, 1),
                         "algorithmic_bytes_per_launch": int(rb["bytes_per_launch"])},
        }
    if not args.no_fp8_buffer:
        rf = bench_decode(args, torch, ops, wl, max(1, args.replicas), buf_dtype=torch.float8_e4m3fn)
        line["decode_fp8_buffer"] = {
            "workload": "the same decode step with the window buffer's keys and values stored "
                        "as FP8 vector pairs (GDNQ_FLAG_BUF_FP8: OCP E4M3 codes, one fp32 scale "
                        "per vector)",
            "ms_per_step": round(rf["ms_per_step"], 5),
            "tokens_s": round(rf["tokens_s"], 1),
            "gbps": round(rf["gbps"], 1),
            "roofline": {"bound": "hbm", "achieved": round(rf["gbps"], 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(rf["gbps"] / HBM_PEAK_GBPS, 4),
                         "traffic": load_traffic("decode_b64_h32_fp8buf_traffic.json",
                                                 DECODE_SOURCES, 1),
                         "algorithmic_bytes_per_launch": int(rf["bytes_per_launch"])},
        }
    if not args.no_state4:
        r4 = bench_decode(args, torch, ops, wl, max(1, args.replicas), state_bits=4)
        line["decode_state4"] = {
            "workload": "the same decode step with the uniform 4-bit state (GDNQ_FLAG_STATE_4BIT: "
                        "codes in [-7, 7], two per byte, scale absmax/7) and the fp32 window buffer",
            "ms_per_step": round(r4["ms_per_step"], 5),
            "tokens_s": round(r4["tokens_s"], 1),
            "gbps": round(r4["gbps"], 1),
            "roofline": {"bound": "hbm", "achieved": round(r4["gbps"], 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(r4["gbps"] / HBM_PEAK_GBPS, 4),
                         "traffic": load_traffic("decode_b64_h32_state4_traffic.json",
                                                 DECODE_SOURCES + ["decode_q4.hip"], 1),
                         "algorithmic_bytes_per_launch": int(r4["bytes_per_launch"])},
        }
    if not args.no_wht:
        rw = bench_decode(args, torch, ops, wl, max(1, args.replicas), wht=True)
        line["decode_wht"] = {
            "workload": "the same decode step with q and k rotated by the normalised Walsh-Hadamard "
                        "matrix inside the kernel (GDNQ_FLAG_WHT; state and buffered keys in the "
                        "rotated basis)",
            "ms_per_step": round(rw["ms_per_step"], 5),
            "tokens_s": round(rw["tokens_s"], 1),
            "gbps": round(rw["gbps"], 1),
            "roofline": {"bound": "hbm", "achieved": round(rw["gbps"], 1), "peak": HBM_PEAK_GBPS,
                         "unit": "GB/s", "frac": round(rw["gbps"] / HBM_PEAK_GBPS, 4),
                         "traffic": load_traffic("decode_b64_h32_wht_traffic.json", DECODE_SOURCES, 1),
                         "algorithmic_bytes_per_launch": int(rw["bytes_per_launch"])},
        }
    if not args.no_sliding:
        line["decode_sliding_window"] = bench_decode_sliding(args, torch, ops, wl, max(1, args.replicas))
    if not args.no_long_decode:
        line["decode_b256_1024_steps"] = bench_decode_long(torch, ops, wl)
    if not args.no_prefill:
        line["prefill"] = bench_prefill(torch, ops, wl, with_cpu=not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
