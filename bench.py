#!/usr/bin/env python3
"""Benchmark of the fused RoPE + FlashAttention forward on one MI355X.

One step = the whole hot path on one batch of synthetic inputs already resident in HBM:
rope_tables (cos/sin for positions 0..S-1) followed by the fused forward
(rope_flash_attn_fwd_ws: Q rotated in registers; K rotated in the kernel's staging or, where
that repeats the rotation of a key many times, once per key by a pre-pass into the
workspace; causal attention).  The host inverse frequencies are computed once at
set-up (a model-load-time quantity).  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5]

The default workload is the largest single-GPU one: B1, 64 q heads over 8 kv heads,
head_dim 128, S 16384, bf16, linear position scaling 2.  The value is TFLOP/s of causal
attention (4*B*Hq*S^2*D/2 per step) over the timed steps.  The roofline object reports
the fused call's own time (its k' pre-pass included), measured with HIP events on the
stream it runs on, against the dense bf16 MFMA peak.  Extra measurements (after the timed
region): the fusion ablation (the fused call, the fused kernel rotating K in-loop, and
rope_qk + attention without rotation, timed in alternating rounds after the same warm-up)
on every 16-bit workload, rope_tables GB/s at
the op's size limits, rope_qk GB/s, the RoPE variants of the fused kernel, the backward
pass, the fused RMSNorm + RoPE + KV-cache write GB/s on a paged-cache prefill, and
decode-step attention GB/s over a paged cache.  The cpu_baseline leg times the fp64 CPU
oracle on a bounded sample of the same workload, phase by phase.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused RoPE+FlashAttn fwd TFLOP/s and % bf16 MFMA peak; rope_tables GB/s"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # dense MFMA peaks (f32: matrix fp32)
PEAK_HBM_GBS = 8000.0
EXTRAS = ("ablation", "backward", "variants", "tables", "kvcache", "decode")
KERNEL_SOURCES = ["rope_flashattention_amd/csrc/flash_fwd.h", "rope_flashattention_amd/csrc/common.h",
                  "rope_flashattention_amd/csrc/rope_qk.hip"]


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def gpu_max_clock_mhz():
    """The GPU agent's maximum engine clock as rocminfo reports it (MHz), or None."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=20).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for agent in txt.split("Agent ")[1:]:
        if "gfx950" not in agent:
            continue
        for ln in agent.splitlines():
            if "Max Clock Freq" in ln:
                try:
                    return int(ln.split(":")[1].split()[0])
                except (IndexError, ValueError):
                    return None
    return None


def read_traffic(workload_key):
    """HBM bytes per launch from the committed counter summary, if it matches the source."""
    path = os.path.join(ROOT, "profiles", f"traffic_flash_fwd_{workload_key}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for ln in fh:
            if ":" in ln:
                k, v = ln.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_hash(KERNEL_SOURCES):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def time_events(fn, reps, torch):
    """Device time (ms) per call of fn: reps back-to-back calls between two HIP events on the
    current stream (an event pair around every call adds a few microseconds of queue work,
    a sizeable share for the HBM-bound kernels of 40-150 us)."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def cpu_baseline(inp, budget_s):
    """The oracle as it stands, one (sequence, q head) at a time, until the budget is spent.

    Each phase is timed on its own: the tables of the sequence (oracle.rope_tables), the
    rotation of the head's queries and of its kv head's keys (oracle.rotate_tokens) and the
    attention with the full N x N score matrix (oracle.attention)."""
    import numpy as np
    import oracle as orc
    try:
        from threadpoolctl import threadpool_info
        blas = max([int(i.get("num_threads", 1)) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing
        blas = None
    cores = len(os.sched_getaffinity(0))
    w = inp.workload
    q, k, v = inp.packed()
    starts = orc.segment_starts(inp.seq_lens)
    g = w.hq // w.hkv
    phase = {"tables_s": 0.0, "rotation_s": 0.0, "attention_s": 0.0}
    t0 = time.perf_counter()
    flops, done = 0.0, 0
    for b in range(w.batch):
        s0, S = int(starts[b]), int(inp.seq_lens[b])
        sl = slice(s0, s0 + S)
        ta = time.perf_counter()
        f = orc.inv_freq_per_sequence(w.base, inp.seq_lens[b:b + 1], w.head_dim, w.trained_len)
        sn, cs = orc.rope_tables(inp.pos[sl], f, inp.seq_lens[b:b + 1], w.pos_scale)
        sn, cs = orc.round_rne(sn, w.dtype), orc.round_rne(cs, w.dtype)
        phase["tables_s"] += time.perf_counter() - ta
        for h in range(w.hq):
            ta = time.perf_counter()
            qr = orc.rotate_tokens(q[sl, h:h + 1], cs, sn)[:, 0]
            kr = orc.rotate_tokens(k[sl, h // g:h // g + 1], cs, sn)[:, 0]
            tb = time.perf_counter()
            orc.attention(qr, kr, v[sl, h // g], w.softmax_scale, w.causal)
            tc = time.perf_counter()
            phase["rotation_s"] += tb - ta
            phase["attention_s"] += tc - tb
            flops += 4.0 * S * S * w.head_dim / (2.0 if w.causal else 1.0)
            done += 1
            if tc - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "blas_threads": blas, "phases_s": {k2: round(v2, 3) for k2, v2 in phase.items()},
            "sample": f"{done} of {w.batch * w.hq} (sequence, q head) pairs of {w.name} in order, full causal "
                      f"rows, tables and rotation included; {dt:.1f} s wall on {cores} usable cores, numpy "
                      f"float64 with {blas} BLAS threads (the exponentials run on one core)"}


def attention_setup(w, inp, dev, rfa, wl, np, torch):
    """Inputs resident in HBM, the host inverse frequencies, table and output buffers."""
    D = w.head_dim
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    if w.varlen:
        f = torch.from_numpy(rfa.inv_freq(w.base, D, inp.seq_lens, w.trained_len)).to(dev)
        pos = torch.from_numpy(inp.pos).to(dev)
        tab_lens = inp.seq_lens
        cu = torch.from_numpy(wl.cu_seqlens(inp.seq_lens)).to(dev)
        akw = dict(layout="TND", cu_seqlens=cu, max_seqlen=int(inp.seq_lens.max()))
    else:
        f = torch.from_numpy(rfa.inv_freq(w.base, D, [w.seqlen], w.trained_len)).to(dev)
        pos = torch.arange(w.seqlen, dtype=torch.int32, device=dev)   # one table shared by the batch
        tab_lens = np.array([w.seqlen], dtype=np.int32)
        akw = dict(layout="BNSD")
    T_tab = int(tab_lens.sum())
    sin = torch.empty((T_tab, D), dtype=w.torch_dtype, device=dev)
    cos = torch.empty((T_tab, D), dtype=w.torch_dtype, device=dev)
    out = torch.empty_like(q)
    # the fused call's workspace (k' rows of the pre-pass), allocated once
    need = rfa.flash_attn_fwd_workspace_size(q, k, v, cos, sin, causal=w.causal, **akw)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    return dict(q=q, k=k, v=v, f=f, pos=pos, tab_lens=tab_lens, sin=sin, cos=cos, out=out, akw=akw, ws=ws)


def fusion_ablation(w, st, rfa, torch, rounds=5, reps=10):
    """The fused call (k' pre-pass where the library plans one), the fused kernel rotating K
    in-loop, and the unfused path (rope_qk, then attention without rotation), timed in
    alternating rounds of back-to-back calls after the same warm-up, so that every leg sees
    the same clock state.  Returns medians over the rounds (ms)."""
    q, k, v, cos, sin, out, akw = st["q"], st["k"], st["v"], st["cos"], st["sin"], st["out"], st["akw"]
    ws = st["ws"] if st["ws"] is not None else "auto"
    qkw = {kk: vv for kk, vv in akw.items()}
    oq, ok = torch.empty_like(q), torch.empty_like(k)
    kw = dict(causal=w.causal, softmax_scale=w.softmax_scale, out=out, **akw)
    fused = lambda: rfa.rope_flash_attn_fwd(q, k, v, cos, sin, workspace=ws, **kw)
    inloop = lambda: rfa.rope_flash_attn_fwd(q, k, v, cos, sin, workspace=None, **kw)
    rot = lambda: rfa.rope_qk(q, k, cos, sin, table_seq_rows=0, out_q=oq, out_k=ok, **qkw)
    plain = lambda: rfa.rope_flash_attn_fwd(oq, ok, v, None, None, workspace=None, **kw)
    rot()
    for _ in range(reps):
        fused()
        inloop()
        plain()
    tf, ti, tr, tp = [], [], [], []
    for _ in range(rounds):
        tf.append(time_events(fused, reps, torch))
        ti.append(time_events(inloop, reps, torch))
        tr.append(time_events(rot, reps, torch))
        tp.append(time_events(plain, reps, torch))
    del oq, ok
    mf, mi, mr, mp = median(tf), median(ti), median(tr), median(tp)
    return {"fused_ms": round(mf, 4), "k_prepass": st["ws"] is not None, "fused_in_loop_ms": round(mi, 4),
            "rope_qk_ms": round(mr, 4), "plain_attention_ms": round(mp, 4), "unfused_ms": round(mr + mp, 4),
            "fused_over_unfused": round(mf / (mr + mp), 4), "in_loop_over_unfused": round(mi / (mr + mp), 4)}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU reaches its steady clocks only after ~100 ms of sustained work: 50 untimed
    # steps of the default workload (about 0.2 s) before the K timed ones
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=5,
                    help="workload 1..5 (default 5: B1 H64/8 S16384, the largest single-GPU workload)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the measurements after the timed region")
    ap.add_argument("--ablation-configs", default="2,3,4,5",
                    help="workloads of the fusion ablation besides the benchmarked one (comma list, may be empty)")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="comma list of the measurements after the timed region (default all): " + ", ".join(EXTRAS))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (scales HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import rope_flashattention_amd as rfa
    from rope_flashattention_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": a.numel() * 4,
                          "copy_calibration_bytes_written_per_launch": b.numel() * 4}), flush=True)
        return
    rfa.lib()
    w = wl.CONFIGS[args.config]
    inp = wl.generate(w)
    D = w.head_dim

    # ---- set-up: inputs resident in HBM, host inverse frequencies, output buffers
    st = attention_setup(w, inp, dev, rfa, wl, np, torch)
    q, k, v, f, pos, tab_lens = st["q"], st["k"], st["v"], st["f"], st["pos"], st["tab_lens"]
    sin, cos, out, akw = st["sin"], st["cos"], st["out"], st["akw"]
    ws = st["ws"] if st["ws"] is not None else "auto"

    def step():
        rfa.rope_tables(pos, f, tab_lens, D, w.pos_scale, w.torch_dtype, sin, cos)
        rfa.rope_flash_attn_fwd(q, k, v, cos, sin, causal=w.causal, softmax_scale=w.softmax_scale, out=out,
                                workspace=ws, **akw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps; each fused call (k' pre-pass and attention kernel)
    # bracketed by events on its stream
    # (two events per step: each recorded event adds a few microseconds of queue work, so
    # the table pass is timed on its own after this region)
    K = args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        rfa.rope_tables(pos, f, tab_lens, D, w.pos_scale, w.torch_dtype, sin, cos)
        ev[i][0].record()
        rfa.rope_flash_attn_fwd(q, k, v, cos, sin, causal=w.causal, softmax_scale=w.softmax_scale, out=out,
                                workspace=ws, **akw)
        ev[i][1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    flops = wl.causal_flops(w, inp.seq_lens)
    ms_per_step = (t1 - t0) * 1e3 / K
    value = flops / (ms_per_step * 1e-3) / 1e12
    att_all = sorted(e[0].elapsed_time(e[1]) for e in ev)
    att_ms = sum(att_all) / K
    # the table pass alone: 50 back-to-back launches between two events
    t_a, t_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_a.record()
    for _ in range(50):
        rfa.rope_tables(pos, f, tab_lens, D, w.pos_scale, w.torch_dtype, sin, cos)
    t_b.record()
    torch.cuda.synchronize()
    tab_ms = t_a.elapsed_time(t_b) / 50
    achieved = flops / (att_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    wkey = f"cfg{args.config}"
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to the dtype, positions 0..L-1 per sequence",
        "config": {"workload": w.name, "batch": w.batch, "hq": w.hq, "hkv": w.hkv, "head_dim": D,
                   "seq_len": (int(inp.seq_lens.max()) if w.varlen else w.seqlen),
                   "ntokens": inp.ntokens, "causal": w.causal, "rope_base": w.base,
                   "ntk_trained_len": w.trained_len, "pos_scale": w.pos_scale, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": read_traffic(wkey),
                     "kernel": ("rope_qk_kernel (k' pre-pass) + flash_fwd16_kernel, timed together"
                                if st["ws"] is not None else "flash_fwd16_kernel"),
                     "avg_launch_ms": round(att_ms, 4)},
        "components": {"rope_tables_ms": round(tab_ms, 5), "attention_ms": round(att_ms, 4),
                       "attention_ms_p10_median_p90": [round(att_all[int(0.1 * (K - 1))], 4),
                                                       round(median(att_all), 4),
                                                       round(att_all[int(0.9 * (K - 1))], 4)],
                       "attention_tflops": round(achieved, 2)},
    }
    # the dense peak at the clock the agent reports: 256 CUs x 4096 bf16/fp16 FLOP per clock
    mhz = gpu_max_clock_mhz()
    if mhz and w.dtype in ("bf16", "f16"):
        pk = 256 * 4096 * mhz * 1e6 / 1e12
        result["components"]["max_clock_mhz"] = mhz
        result["components"]["peak_at_max_clock_tflops"] = round(pk, 1)
        result["components"]["frac_of_peak_at_max_clock"] = round(achieved / pk, 4)

    extras = set(args.extras.split(","))
    if not args.no_extras:
        comp = result["components"]
        if "ablation" in extras:
            # rope_qk on the workload (reads Q, K; writes Q', K'; table rows read once)
            oq, ok = torch.empty_like(q), torch.empty_like(k)
            qk_fn = lambda: rfa.rope_qk(q, k, cos, sin, table_seq_rows=0, out_q=oq, out_k=ok, **akw)
            for _ in range(3):
                qk_fn()
            ms = time_events(qk_fn, 20, torch)
            qk_bytes = 2 * (q.numel() + k.numel()) * q.element_size() + 2 * sin.numel() * sin.element_size()
            comp["rope_qk_ms"] = round(ms, 4)
            comp["rope_qk_gbps"] = round(qk_bytes / (ms * 1e-3) / 1e9, 1)
            comp["rope_qk_hbm_frac"] = round(qk_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            del oq, ok
            # fusion ablation on every 16-bit workload (this one first), and the attention
            # throughput of the others
            abl = {}
            others = [int(c) for c in args.ablation_configs.split(",") if c and int(c) != args.config]
            for c in [args.config] + others:
                wc = wl.CONFIGS[c]
                if wc.dtype == "f32":
                    continue
                if c == args.config:
                    sc, fl = st, flops
                else:
                    ic = wl.generate(wc)
                    sc = attention_setup(wc, ic, dev, rfa, wl, np, torch)
                    rfa.rope_tables(sc["pos"], sc["f"], sc["tab_lens"], wc.head_dim, wc.pos_scale, wc.torch_dtype,
                                    sc["sin"], sc["cos"])
                    fl = wl.causal_flops(wc, ic.seq_lens)
                r = fusion_ablation(wc, sc, rfa, torch)
                r["fused_tflops"] = round(fl / (r["fused_ms"] * 1e-3) / 1e12, 2)
                r["plain_attention_tflops"] = round(fl / (r["plain_attention_ms"] * 1e-3) / 1e12, 2)
                abl[f"cfg{c}"] = r
                if c != args.config:
                    del sc
                    torch.cuda.empty_cache()
            comp["fusion_ablation"] = abl
        if "backward" in extras:
            # backward on the same workload (delta, dk/dv and dq kernels; dO seeded): algorithmic
            # FLOPs 2.5x the forward's (the five products S, dP, dV, dK, dQ; the dq kernel's
            # recomputation of S and dP is overhead, not counted)
            if w.dtype != "f32":
                out_f, lse_f = rfa.rope_flash_attn_fwd(q, k, v, cos, sin, causal=w.causal, softmax_scale=w.softmax_scale,
                                                       return_lse=True, workspace=ws, **akw)
                bdo = wl.generate_dout(inp, 9001).to(dev)
                if not w.varlen and akw.get("layout") == "BSND":
                    bdo = bdo.transpose(1, 2).contiguous()
                bdq, bdk, bdv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
                bfn = lambda: rfa.rope_flash_attn_bwd(q, k, v, out_f, lse_f, bdo, cos, sin, causal=w.causal,
                                                      softmax_scale=w.softmax_scale, dq=bdq, dk=bdk, dv=bdv, **akw)
                bfn()
                bms = time_events(bfn, 10, torch)
                comp["bwd_ms"] = round(bms, 4)
                comp["bwd_tflops"] = round(2.5 * flops / (bms * 1e-3) / 1e12, 2)
                del out_f, lse_f, bdo, bdq, bdk, bdv
        if "variants" in extras:
            # RoPE variants of the fused kernel on the same workload: interleaved pairs (tables
            # from rope_tables_ex), and table values formed inside the kernel (no table read, no
            # table pass) for both pairings
            if not w.varlen:
                vpos = torch.arange(w.seqlen, dtype=torch.int32, device=dev)
                vf = torch.from_numpy(rfa.inv_freq(w.base, w.head_dim, [w.seqlen], w.trained_len)).to(dev)
                isin, icos = rfa.rope_tables(vpos, vf, [w.seqlen], w.head_dim, w.pos_scale, w.torch_dtype,
                                             pairing="interleaved")
                vkw = dict(causal=w.causal, softmax_scale=w.softmax_scale, out=out, **akw)
                for name, fn in (
                        ("interleaved_tables", lambda: rfa.rope_flash_attn_fwd(q, k, v, icos, isin, pairing="interleaved",
                                                                               **vkw)),
                        ("formed_tables_half", lambda: rfa.rope_flash_attn_fwd(q, k, v, None, None, pos=vpos, inv_freq=vf,
                                                                               pos_scale=w.pos_scale, **vkw)),
                        ("formed_tables_interleaved", lambda: rfa.rope_flash_attn_fwd(
                            q, k, v, None, None, pos=vpos, inv_freq=vf, pos_scale=w.pos_scale, pairing="interleaved",
                            **vkw))):
                    fn()
                    vms = time_events(fn, 10, torch)
                    comp[f"fused_{name}_ms"] = round(vms, 4)
                    comp[f"fused_{name}_tflops"] = round(flops / (vms * 1e-3) / 1e12, 2)
        if "tables" in extras:
            # rope_tables at the op's limits: batch 16, ntokens 256000 (sequences of 16000 tokens),
            # head_size 2048 (2.1 GB written) and 512
            lens = np.full(16, 16000, dtype=np.int32)
            tpos = torch.arange(16000, dtype=torch.int32, device=dev).repeat(16)
            for Dt in (2048, 512, 128):
                tf = torch.from_numpy(rfa.inv_freq(1e4, Dt, lens, 4096)).to(dev)
                variants = []
                for dt_name, dt in (("f16", torch.float16), ("bf16", torch.bfloat16)):
                    ts = torch.empty((256000, Dt), dtype=dt, device=dev)
                    tc = torch.empty((256000, Dt), dtype=dt, device=dev)
                    variants.append((dt_name, (lambda ts=ts, tc=tc, dt=dt: rfa.rope_tables(tpos, tf, lens, Dt, 1.0, dt, ts,
                                                                                          tc))))
                # the dtypes are timed in turn, three times each, and the median taken: the first
                # variant timed after the matrix-bound runs above otherwise reads up to 15% slow
                times = {name: [] for name, _ in variants}
                for _ in range(3):
                    for name, fn in variants:
                        for _ in range(10):
                            fn()
                        times[name].append(time_events(fn, 20, torch))
                tb = 2 * 256000 * Dt * 2 + 4 * 256000 + 4 * 16 * (Dt // 2)
                for name, _ in variants:
                    ms = median(times[name])
                    comp[f"rope_tables_{name}_T256000_D{Dt}_gbps"] = round(tb / (ms * 1e-3) / 1e9, 1)
                    comp[f"rope_tables_{name}_T256000_D{Dt}_hbm_frac"] = round(tb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
                del variants
            torch.cuda.empty_cache()
        if "kvcache" in extras:
            # fused RMSNorm + RoPE + KV-cache write on a 16 x 4096-token prefill into a paged cache:
            # reads K, V and the table rows, writes K', V into the cache (slots, gamma are small)
            cw = wl.CACHE_CONFIGS["prefill"]
            ci = wl.generate_cache(cw)
            ck, cv = ci.k.to(dev), ci.v.to(dev)
            kc, vc = ci.k_cache.to(dev), ci.v_cache.to(dev)
            cgam, cslots = ci.gamma.to(dev), torch.from_numpy(ci.slots).to(dev)
            clens = np.full(cw.batch, cw.new_tokens, dtype=np.int32)
            cf = torch.from_numpy(rfa.inv_freq(cw.base, cw.head_dim, clens)).to(dev)
            csin, ccos = rfa.rope_tables(torch.from_numpy(ci.pos).to(dev), cf, clens, cw.head_dim, 1.0, cw.torch_dtype)
            fn = lambda: rfa.rope_kv_rms_norm_rope_cache(ck, cv, ccos, csin, cslots, kc, vc, gamma=cgam, eps=1e-6)
            for _ in range(3):
                fn()
            ms = time_events(fn, 20, torch)
            esz = ck.element_size()
            cb = 4 * ck.numel() * esz + 2 * csin.numel() * esz + 8 * cslots.numel() + 4 * cgam.numel()
            comp["kv_cache_workload"] = cw.name
            comp["kv_cache_ms"] = round(ms, 4)
            comp["kv_cache_gbps"] = round(cb / (ms * 1e-3) / 1e9, 1)
            comp["kv_cache_hbm_frac"] = round(cb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            del ck, cv, kc, vc, ci
            torch.cuda.empty_cache()
        if "decode" in extras:
            # decode step over a paged cache: 32 sequences with 1024..8192 cached tokens, Hq 64 / Hkv 8;
            # both launches (split partials and their merge) inside the timed call
            dw = wl.CACHE_CONFIGS["decode"]
            di = wl.generate_cache(dw)
            dlens = (di.ctx + 1).astype(np.int32)
            dq = di.q.to(dev)
            dkc, dvc = di.k_cache.to(dev), di.v_cache.to(dev)
            dbt = torch.from_numpy(di.block_table.astype(np.int32)).to(dev)
            dsl = torch.from_numpy(dlens).to(dev)
            dfr = torch.from_numpy(rfa.inv_freq(dw.base, dw.head_dim)).to(dev)
            dsin, dcos = rfa.rope_tables(torch.from_numpy(di.pos).to(dev), dfr, [dw.batch], dw.head_dim, 1.0,
                                         dw.torch_dtype)
            dkw = dict(max_seqlen=int(dlens.max()), block_table=dbt)
            dws = torch.empty(rfa.decode_workspace_size(dq, dkc, dvc, dsl, **dkw), dtype=torch.uint8, device=dev)
            dout = torch.empty_like(dq)
            fn = lambda: rfa.rope_decode_attn_fwd(dq, dkc, dvc, dsl, dcos, dsin, out=dout, workspace=dws, **dkw)
            for _ in range(3):
                fn()
            ms = time_events(fn, 20, torch)
            db = wl.decode_bytes(dw, dlens)
            comp["decode_workload"] = dw.name
            comp["decode_ms"] = round(ms, 4)
            comp["decode_gbps"] = round(db / (ms * 1e-3) / 1e9, 1)
            comp["decode_hbm_frac"] = round(db / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            del dq, dkc, dvc, dws, di
            torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
