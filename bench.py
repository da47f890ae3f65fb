#!/usr/bin/env python3
"""KDA benchmark on one MI355X: chunked prefill throughput (headline) plus decode bandwidth.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one kda_chunked_forward call over the largest single-GPU prefill
workload: one sequence of 1,048,576 tokens x 8 heads, bf16 q/k/v/g/beta,
d_k = d_v = 128, chunk 64, fp32 state from zero.  The call runs, on the
caller's stream, the intra-chunk kernel (gate cumsum, UT/WY transform and the
chunk-local products of every (chunk, head), in parallel, into per-chunk
records) and the state chain (for this shape: 32 segments of 512 chunks per
head; a summary pass over each segment's value and identity columns, the fp32
combine of segment start states, then the chain of every segment on whole
128-column states, writing o and hT).  Inputs are resident in HBM before the timed
region; the timed region is exactly K back-to-back steps between two HIP events
on the launch stream, bracketed by synchronisation (ms_per_step = event time /
K; a step moves tens of GB, far beyond the 256 MB Infinity Cache).  A pass
through kda_chunked_forward_profiled gives the two stages' durations.

The JSON line carries:
  roofline       -- the whole call against HBM, its binding roof: achieved = the
                    call's algorithmic bytes (q, k, v, g, beta in, o out: 1,282 B
                    per token-head at bf16, d = 128; plus the hT write) / ms_per_step;
                    traffic = the call's HBM bytes from the rocprofv3 FETCH_SIZE /
                    WRITE_SIZE counters (summed over its kernels, scaled by a plain
                    copy's reading; profiles/hbm_traffic.json), null unless taken on
                    the current kernel sources; traffic_ratio = traffic / algorithmic
  roofline_mfma  -- the call's algorithmic flops against dense bf16 MFMA (the
                    headline metric's "% of MFMA peak")
  stages         -- intra-chunk kernel and state-chain durations (profiled entry point)
  stream         -- plain device copy / fill / read rates on this GPU, and the call's
                    counter-measured HBM bytes (whole call and per kernel) at the copy
                    rate: the least time any kernel moving those bytes could take
  workloads      -- the other seeded prefill workloads (fp32 2 x 256 tokens; 4 x 16
                    heads x 4096 tokens; 32 heads x 65,536 tokens; 16 packed
                    sequences), each timed over a few calls with the cache evicted
                    before each: tokens/s, the chain layout, the two stages'
                    durations, and the call's algorithmic bytes / flops against
                    HBM / MFMA
  states, fused, mxfp8, backward -- on the 4 x 16 x 4096 workload: the call keeping
                    the state every 1024 tokens; the fused gate / q-k norm / output
                    gate; MXFP8 q, k, v; the backward (training) call, and a
                    training step (forward + backward) with and without the
                    forward's records and states saved for the backward
  decode         -- 1000 sequential kda_decode_step calls on the 256-sequence x
                    32-head state (512 MiB fp32), bytes and fraction of HBM
  cpu_baseline   -- the fp64 oracle on this host's cores, whole passes over the first
                    65,536 tokens x 8 heads of the headline workload for at least 10 s
                    (a baseline, not a target); cores = the threads it used
Algorithmic work per token and head (d_k = d_v = d, chunk C):
  flops 6 d^2 + (C-1) d + 2 (C+1) d + 2 (C+1) d + C^2/3 ; bytes (3 d_k + d_v) s_in + s_beta + d_v s_out,
  plus 4 d_k d_v per (sequence, head) for each of h0 (when given) and hT.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2516.6  # MI355X dense bf16 MFMA
CSRC = os.path.join(ROOT, "gated_delta_rule_94_amd", "csrc")
# the sources each measured launch group is built from (a counter reading is valid for these exact
# sources only)
KERNEL_SOURCES = {
    "prefill": ("kda_intra.hip", "kda_chain.hip", "kda_prefill.hip", "kda_device.h", "kda_record.h", "kda_internal.h"),
    "decode": ("kda_decode.hip", "kda_device.h"),
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
HEADLINE = "cfg4_bf16_b1_h8_t1048576_d128"


def prefill_flops_per_token_head(dk, dv, C):
    return 6 * dk * dv + (C - 1) * dk + 2 * (C + 1) * dk + 2 * (C + 1) * dv + C * C / 3.0


def backward_flops_per_token_head(dk, dv, C):
    """Products the backward computes per (token, head), masked halves counted as half: the forward
    recompute; the adjoint chain (P^T dO, Kd dS, (Q Gamma)^T dO, W^T dU); the state products (U, dU,
    dP, d(Q Gamma), dKd, dW); the transform (Ekk, dT, T^T dW, T^T dU, L^T dL L^T, and the four
    Ekk / Eqk products)."""
    chain = C * dv + 6 * dk * dv
    state = 2 * C * dv + 10 * dk * dv
    transform = 7 * C * dk + 2 * C * dv + 2 * C * C // 3
    return prefill_flops_per_token_head(dk, dv, C) + chain + state + transform


def prefill_bytes(B, T, H, dk, dv, s_in, s_out, with_h0=True, with_hT=True):
    per_th = (3 * dk + dv) * s_in + s_in + dv * s_out
    return B * T * H * per_th + B * H * 4 * dk * dv * (int(with_h0) + int(with_hT))


def decode_bytes(B, H, dk, dv, s_in):
    return B * H * (2 * 4 * dk * dv + (3 * dk + dv) * s_in + s_in + dv * s_in)


def sources_sha256(kernel_key):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel_key]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_entry(entry, kernel_key):
    """The committed rocprofv3 counter summary of a workload (or "decode"): HBM bytes per call and
    per kernel, if taken on the current sources of kernel_key, else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[entry]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("source_sha256") != sources_sha256(kernel_key):
        return None
    return t


def measured_traffic(entry, kernel_key):
    t = traffic_entry(entry, kernel_key)
    return None if t is None else t["bytes_per_call"]


def stream_rates(reps=5):
    """Rates of plain device streams on this GPU (torch's own copy, fill and max-reduction over 4 GiB,
    far beyond the 256 MB Infinity Cache): what a kernel that only moves bytes reaches here, the
    practical ceiling the kernels' HBM traffic is held against."""
    import torch

    n = 1 << 30  # 4 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    rates = {}
    for name, fn, moved in (("copy_GBps", lambda: b.copy_(a), 8 * n), ("fill_GBps", lambda: b.fill_(2.0), 4 * n),
                            ("read_GBps", lambda: torch.amax(a), 4 * n)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        rates[name] = moved / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return rates


def world_size():
    return int(os.environ.get("WORLD_SIZE", "1"))


def copy_calibration():
    """One plain copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    n = 1 << 28  # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n}))


def time_launches(fn, steps, flush=None):
    """Mean duration of `fn` over `steps` launches, each bracketed by events on the current stream."""
    import torch

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush()
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return sum(ms) / len(ms), wall


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true", help="skip the other prefill workloads")
    ap.add_argument("--no-states", action="store_true", help="skip the state-snapshot leg")
    ap.add_argument("--no-fused", action="store_true", help="skip the fused-steps leg")
    ap.add_argument("--no-mxfp8", action="store_true", help="skip the MXFP8-input leg")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward (training) leg")
    ap.add_argument("--workloads", default="", help="comma-separated subset of the other prefill workloads")
    ap.add_argument("--no-flush", action="store_true", help="do not evict the Infinity Cache between steps")
    ap.add_argument("--copy-calibration", action="store_true", help="run one 1 GiB copy (counter scaling) and exit")
    ap.add_argument("--no-stream", action="store_true", help="skip the plain-stream rates")
    args = ap.parse_args()

    if args.gpus != 1 or world_size() != 1:
        print("bench.py runs on one GPU only: the KDA path here is the single-GPU kernel "
              "(multi-GPU sharding is a design note, not built); got --gpus %d, WORLD_SIZE=%d"
              % (args.gpus, world_size()), file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    import datagen
    import gated_delta_rule_94_amd as kda

    dev = torch.device("cuda:0")

    def to_dev(a):
        if a is None:
            return None
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    scratch = None if args.no_flush else torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def flush():
        scratch.fill_(1)

    def prefill_case(wl):
        """Device inputs, outputs and workspace of a seeded prefill workload, and its call."""
        tdt = torch.float32 if wl.dtype == datagen.DT_F32 else torch.bfloat16
        c = {"wl": wl, "tdt": tdt, "s_io": 4 if tdt == torch.float32 else 2}
        if wl.kind == "varlen":
            lens = datagen.varlen_lengths(wl.seed, wl.num_seqs, wl.len_lo, wl.len_hi)
            cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
            dl = datagen.prefill_inputs(wl.seed, 1, int(cu[-1]), wl.H, wl.dk, wl.dv, wl.dtype, None)
            c.update(n_tok=int(cu[-1]), n_seq=wl.num_seqs, maxlen=int(lens.max()), cu=to_dev(cu), with_h0=False)
        else:
            dl = datagen.prefill_inputs(wl.seed, wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.dtype, wl.h0_std)
            c.update(n_tok=wl.B * wl.T, n_seq=wl.B, with_h0=wl.h0_std is not None)
        c["host"] = dl
        c["g"] = {key: to_dev(val) for key, val in dl.items()}
        c["o"] = torch.empty(c["g"]["v"].shape, dtype=tdt, device=dev)
        c["hT"] = torch.empty((c["n_seq"], wl.H, wl.dk, wl.dv), dtype=torch.float32, device=dev)
        gg = c["g"]
        if wl.kind == "varlen":
            c["ws"] = torch.empty(kda.varlen_workspace_bytes(wl.num_seqs, c["n_tok"], c["maxlen"], wl.H, wl.dk, wl.dv,
                                                             wl.chunk, tdt), dtype=torch.uint8, device=dev)

            def call(_i):
                kda.kda_chunked_forward_varlen(gg["q"], gg["k"], gg["v"], gg["g"], gg["beta"], c["cu"], c["maxlen"],
                                               None, chunk=wl.chunk, o=c["o"], hT=c["hT"], workspace=c["ws"])
        else:
            c["ws"] = torch.empty(kda.workspace_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.chunk, tdt),
                                  dtype=torch.uint8, device=dev)

            def call(_i):
                kda.kda_chunked_forward(gg["q"], gg["k"], gg["v"], gg["g"], gg["beta"], gg["h0"], chunk=wl.chunk,
                                        o=c["o"], hT=c["hT"], workspace=c["ws"])
        c["call"] = call
        c["alg_bytes"] = prefill_bytes(1, c["n_tok"], wl.H, wl.dk, wl.dv, c["s_io"], c["s_io"], with_h0=False,
                                       with_hT=False) + c["n_seq"] * wl.H * 4 * wl.dk * wl.dv * (int(c["with_h0"]) + 1)
        c["alg_flops"] = c["n_tok"] * wl.H * prefill_flops_per_token_head(wl.dk, wl.dv, wl.chunk)
        return c

    def stages(c):
        """(intra-chunk kernel ms, state chain ms) of one call, cache evicted before it."""
        wl, gg = c["wl"], c["g"]
        if not args.no_flush:
            flush()
        return kda.kda_chunked_forward_profiled(gg["q"], gg["k"], gg["v"], gg["g"], gg["beta"], gg["h0"], c["o"],
                                                c["hT"], chunk=wl.chunk, workspace=c["ws"])

    def plan_of(wl, tdt):
        vs, nseg, segc = kda.chain_plan(wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.chunk, tdt)
        return {"value_slice": vs, "segments": nseg, "segment_chunks": segc,
                "summary_slice": kda.summary_slice(wl.B, wl.T, wl.H, wl.dk, wl.dv, wl.chunk, tdt)}

    # ---------------- prefill (headline): one 1,048,576-token sequence x 8 heads
    w = datagen.WORKLOADS[HEADLINE]
    hc = prefill_case(w)
    step = hc["call"]
    for _ in range(args.warmup):
        step(0)
    torch.cuda.synchronize()
    # the timed region: exactly K back-to-back steps, bracketed by synchronisation
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    # the two stages of the call, through the profiling entry point
    st_ms = [0.0, 0.0]
    n_prof = max(1, min(args.steps, 5))
    for _ in range(n_prof):
        a_ms, b_ms = stages(hc)
        st_ms[0] += a_ms / n_prof
        st_ms[1] += b_ms / n_prof

    tokens = hc["n_tok"]
    alg_bytes, alg_flops = hc["alg_bytes"], hc["alg_flops"]
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    tfs = alg_flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic(HEADLINE, "prefill")
    out = {
        "metric": "KDA prefill tokens/s (% bf16 MFMA peak); decode GB/s (% HBM peak)",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded SplitMix64/Box-Muller inputs with the workload's distributions",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "d_k": w.dk, "d_v": w.dv, "chunk": w.chunk,
                   "state": "fp32", "h0": "zero", "tokens_per_step": tokens,
                   "chain_plan": plan_of(w, hc["tdt"]),
                   "timing": "K back-to-back steps between two HIP events on the launch stream"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "traffic_ratio": None if traffic is None else traffic / alg_bytes,
                     "scope": "whole call (intra-chunk kernel, segment summaries, combine, chain)",
                     "alg_bytes_per_call": alg_bytes, "ms_per_call": ms},
        "roofline_mfma": {"achieved": tfs, "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                          "frac": tfs / MFMA_BF16_PEAK_TFS, "alg_flops_per_call": alg_flops, "scope": "whole call"},
        "stages": {"intra_ms": st_ms[0], "chain_ms": st_ms[1],
                   "note": "mean of %d calls through kda_chunked_forward_profiled (events between the stages)"
                           % n_prof},
        "wall_s_timed_region": wall,
        "ms_per_step_wall": 1e3 * wall / args.steps,
    }
    cpu_sample = {key: np.ascontiguousarray(hc["host"][key][:, :65536]) for key in ("q", "k", "v", "g", "beta")}
    del hc, step
    torch.cuda.empty_cache()

    # ---------------- plain streams: the call's measured HBM traffic at a plain device copy's rate is
    # the least time any kernel moving those bytes could take on this GPU
    if not args.no_stream:
        rates = stream_rates()
        tr = traffic_entry(HEADLINE, "prefill")
        floor = {"rates": rates, "call_floor_ms": None, "kernel_floor_ms": None, "call_frac_of_floor": None}
        if tr is not None:
            floor["call_floor_ms"] = tr["bytes_per_call"] / (rates["copy_GBps"] * 1e6)
            floor["call_frac_of_floor"] = floor["call_floor_ms"] / ms
            floor["kernel_floor_ms"] = {k: v["bytes"] / (rates["copy_GBps"] * 1e6) for k, v in tr["kernels"].items()}
        floor["note"] = ("floor = the call's HBM bytes (rocprofv3 counters, profiles/hbm_traffic.json) at the rate of "
                         "a plain device copy (read + write) on this GPU")
        out["stream"] = floor

    # ---------------- the 4 x 16 x 4096 workload: its own line in `workloads`, and the legs below
    # (skipped when none of them runs, so that a profile of the headline holds the headline only)
    if args.no_workloads and args.no_states and args.no_fused and args.no_mxfp8 and args.no_backward:
        args.no_states = args.no_fused = args.no_mxfp8 = args.no_backward = True
        c1 = None
    else:
        w = datagen.WORKLOADS["cfg1_bf16_b4_h16_t4096_d128"]
        c1 = prefill_case(w)
        g, o, hT = c1["g"], c1["o"], c1["hT"]
        tokens = c1["n_tok"]
        c1["call"](0)
        torch.cuda.synchronize()
        ms, _ = time_launches(c1["call"], args.steps, None if args.no_flush else flush)
    # ---------------- the same call keeping the state every 1024 tokens (prefix states for a cache)
    if not args.no_states:
        every = 1024
        st_buf = torch.empty((w.B, w.H, w.T // every, w.dk, w.dv), dtype=torch.float32, device=dev)

        def sstep(_i):
            kda.kda_chunked_forward_with_states(g["q"], g["k"], g["v"], g["g"], g["beta"], g["h0"], state_every=every,
                                                chunk=w.chunk, o=o, hT=hT, states=st_buf)

        sstep(0)
        torch.cuda.synchronize()
        sms, _ = time_launches(sstep, args.steps, None if args.no_flush else flush)
        out["states"] = {"state_every": every, "states_per_call": w.B * w.H * (w.T // every),
                         "state_bytes_per_call": st_buf.numel() * 4, "ms_per_call": sms,
                         "tokens_per_s": tokens / (sms * 1e-3), "overhead_vs_plain": sms / ms - 1.0}
        del st_buf

    # ---------------- the same workload through the fused entry point: the log-decay from its gate
    # pre-activation, q and k normalised in the kernel, an output gate on o
    if not args.no_fused:
        dr = datagen.prefill_preactivations(w.seed, w.B, w.T, w.H, w.dk, w.dv, w.dtype, w.h0_std)
        gr = {key: to_dev(dr[key]) for key in ("q", "k", "v", "x", "beta", "z")}
        del dr

        def fstep(_i):
            kda.kda_chunked_forward_fused(gr["q"], gr["k"], gr["v"], None, gr["beta"], g["h0"], gate_x=gr["x"],
                                          gate_scale=5.0, normalize_qk=True, out_gate=gr["z"], chunk=w.chunk, o=o,
                                          hT=hT)

        fstep(0)
        torch.cuda.synchronize()
        fms, _ = time_launches(fstep, args.steps, None if args.no_flush else flush)
        out["fused"] = {"gate": "-5 sigmoid(x) in the kernel", "normalize_qk": True, "out_gate": True,
                        "ms_per_call": fms, "tokens_per_s": tokens / (fms * 1e-3), "overhead_vs_plain": fms / ms - 1.0}
        del gr

    # ---------------- the same workload with MXFP8 q, k, v (quantised from the bf16 inputs)
    if not args.no_mxfp8:
        dm = datagen.mxfp8_prefill_inputs(w.seed, w.B, w.T, w.H, w.dk, w.dv, w.h0_std)
        gm = {key: to_dev(dm[key]) for key in ("q8", "qs", "k8", "ks", "v8", "vs")}
        del dm

        def mstep(_i):
            kda.kda_chunked_forward_mxfp8(gm["q8"], gm["qs"], gm["k8"], gm["ks"], gm["v8"], gm["vs"], g["g"], g["beta"],
                                          g["h0"], chunk=w.chunk, o=o, hT=hT)

        mstep(0)
        torch.cuda.synchronize()
        mms, _ = time_launches(mstep, args.steps, None if args.no_flush else flush)
        # q, k, v one byte per element plus a scale byte per 32; g, beta, o bf16; h0 and hT fp32
        per_th = (2 * w.dk + w.dv) * (1 + 1 / 32) + 2 * w.dk + 2 + 2 * w.dv
        mbytes = w.B * w.T * w.H * per_th + w.B * w.H * 4 * w.dk * w.dv * 2
        out["mxfp8"] = {"format": "E4M3 elements, E8M0 scale per 32 channels (q, k, v)", "ms_per_call": mms,
                        "tokens_per_s": tokens / (mms * 1e-3), "ratio_to_bf16_call": mms / ms,
                        "alg_bytes_per_call": mbytes, "hbm_frac": mbytes / (mms * 1e-3) / 8e12}
        del gm

    # ---------------- backward of the same call (training): gradients of <do, o> + <dhT, hT>, the
    # forward recomputed inside
    if not args.no_backward:
        do, dhT = datagen.backward_adjoints(w.seed, w.B, w.T, w.H, w.dk, w.dv, w.dtype, 0.5)
        do, dhT = to_dev(do), to_dev(dhT)
        bws = torch.empty(kda.backward_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.chunk, g["q"].dtype),
                          dtype=torch.uint8, device=dev)
        grads = kda.kda_chunked_backward(g["q"], g["k"], g["v"], g["g"], g["beta"], g["h0"], do, dhT, chunk=w.chunk,
                                         workspace=bws)

        def bstep(_i):
            kda.kda_chunked_backward(g["q"], g["k"], g["v"], g["g"], g["beta"], g["h0"], do, dhT, chunk=w.chunk,
                                     grads=grads, workspace=bws)

        torch.cuda.synchronize()
        bms, _ = time_launches(bstep, max(3, args.steps // 4), None if args.no_flush else flush)
        bflops = backward_flops_per_token_head(w.dk, w.dv, w.chunk) * tokens * w.H
        out["backward"] = {"ms_per_call": bms, "tokens_per_s": tokens / (bms * 1e-3), "ratio_to_forward": bms / ms,
                           "flops_per_token_head": backward_flops_per_token_head(w.dk, w.dv, w.chunk),
                           "tflops": bflops / (bms * 1e-3) / 1e12, "peak_tflops": MFMA_BF16_PEAK_TFS,
                           "mfma_frac": bflops / (bms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS,
                           "workspace_bytes": bws.numel(),
                           "note": "forward recompute + adjoint chain + state products + UT-transform backward"}
        # a training step: forward + backward, the backward recomputing the forward, or using what
        # kda_chunked_forward_train saved (the same gradients bitwise)
        saved = torch.empty(kda.train_saved_bytes(w.B, w.T, w.H, w.dk, w.dv, w.chunk, g["q"].dtype), dtype=torch.uint8,
                            device=dev)
        sws = torch.empty(kda.backward_saved_workspace_bytes(w.B, w.T, w.H, w.dk, w.dv, w.chunk, g["q"].dtype),
                          dtype=torch.uint8, device=dev)

        def step_recompute(_i):
            c1["call"](0)
            bstep(0)

        def step_saved(_i):
            kda.kda_chunked_forward_train(g["q"], g["k"], g["v"], g["g"], g["beta"], g["h0"], chunk=w.chunk, o=o, hT=hT,
                                          saved=saved)
            kda.kda_chunked_backward_saved(g["q"], g["k"], g["v"], g["g"], g["beta"], g["h0"], do, dhT, saved,
                                           chunk=w.chunk, grads=grads, workspace=sws)

        def bstep_saved(_i):  # the backward alone, from the buffer the last training forward filled
            kda.kda_chunked_backward_saved(g["q"], g["k"], g["v"], g["g"], g["beta"], g["h0"], do, dhT, saved,
                                           chunk=w.chunk, grads=grads, workspace=sws)

        step_saved(0)
        torch.cuda.synchronize()
        rms, _ = time_launches(step_recompute, max(3, args.steps // 4), None if args.no_flush else flush)
        tms, _ = time_launches(step_saved, max(3, args.steps // 4), None if args.no_flush else flush)
        step_saved(0)
        torch.cuda.synchronize()
        bsms, _ = time_launches(bstep_saved, max(3, args.steps // 4), None if args.no_flush else flush)
        out["train_step"] = {"ms_recompute": rms, "ms_saved": tms, "saved_bytes": saved.numel(),
                             "workspace_bytes_saved_backward": sws.numel(),
                             "tokens_per_s_saved": tokens / (tms * 1e-3),
                             "ms_backward_saved": bsms,
                             "note": "forward + backward per step; 'saved': kda_chunked_forward_train + "
                                     "kda_chunked_backward_saved (no forward recompute); ms_backward_saved: "
                                     "kda_chunked_backward_saved alone"}
        del bws, grads, do, dhT, saved, sws

    # ---------------- decode
    if not args.no_decode:
        wd = datagen.WORKLOADS["cfg3_decode_b256_h32_d128"]
        state = to_dev(datagen.decode_state0(wd.seed, wd.B, wd.H, wd.dk, wd.dv))
        pool = []
        for s in range(8):  # distinct inputs, used round-robin (decode time does not depend on values)
            dd = datagen.decode_inputs(wd.seed, s, wd.B, wd.H, wd.dk, wd.dv, wd.dtype)
            pool.append([to_dev(dd[key]) for key in ("q", "k", "v", "g", "beta")])
        od = torch.empty((wd.B, wd.H, wd.dv), dtype=torch.bfloat16, device=dev)

        def dstep(i):
            kda.kda_decode_step(*pool[i % len(pool)], state, o=od)

        for i in range(3):
            dstep(i)
        torch.cuda.synchronize()
        dms, dwall = time_launches(dstep, args.decode_steps)
        dbytes = decode_bytes(wd.B, wd.H, wd.dk, wd.dv, 2)
        dgbs = dbytes / (dms * 1e-3) / 1e9
        out["decode"] = {
            "workload": wd.name, "steps": args.decode_steps, "us_per_step": dms * 1e3,
            "tokens_per_s": wd.B / (dms * 1e-3), "wall_s": dwall,
            "roofline": {"bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dgbs / HBM_PEAK_GBS, "traffic": measured_traffic("decode", "decode"),
                         "kernel": "decode_step_kernel<bf16, 128, 128>", "alg_bytes_per_launch": dbytes},
        }
        del state, pool

    # ---------------- the other prefill workloads: tokens/s on one GPU
    def workload_entry(c, lms, reps):
        wl = c["wl"]
        entry = {"ms_per_call": lms, "tokens_per_s": c["n_tok"] / (lms * 1e-3),
                 "token_heads_per_s": c["n_tok"] * wl.H / (lms * 1e-3), "calls": reps,
                 "dtype": "f32" if c["tdt"] == torch.float32 else "bf16",
                 "alg_bytes_per_call": c["alg_bytes"],
                 "hbm_frac": c["alg_bytes"] / (lms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "mfma_frac": None if c["tdt"] == torch.float32
                 else c["alg_flops"] / (lms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS}
        if wl.kind == "varlen":
            entry["sequences"] = int(wl.num_seqs)
        else:
            entry["chain_plan"] = plan_of(wl, c["tdt"])
            a_ms, b_ms = stages(c)
            entry.update({"intra_ms": a_ms, "chain_ms": b_ms})
        return entry

    if not args.no_workloads:
        out["workloads"] = {}
        chosen = set(x for x in args.workloads.split(",") if x)
        out["workloads"]["cfg1_bf16_b4_h16_t4096_d128"] = workload_entry(c1, ms, args.steps)
        for name, reps in (("cfg0_f32_b1_h2_t256_d64", 20), ("cfg2_bf16_b1_h32_t65536_d128", 5),
                           ("cfg4v_varlen_n16_h8_d128", 3)):
            if chosen and name not in chosen:
                continue
            cl = prefill_case(datagen.WORKLOADS[name])
            cl["call"](0)
            torch.cuda.synchronize()
            lms, _ = time_launches(cl["call"], reps, None if args.no_flush else flush)
            out["workloads"][name] = workload_entry(cl, lms, reps)
            print("workload %s: %.3f ms" % (name, lms), file=sys.stderr, flush=True)
            del cl
            torch.cuda.empty_cache()

    # ---------------- CPU baseline: the fp64 oracle on this host's cores, on a bounded sample of the
    # headline workload (its first 65,536 tokens, all 8 heads; the oracle runs one thread per head)
    if not args.no_cpu_baseline:
        import oracle

        wh = datagen.WORKLOADS[HEADLINE]
        threads = max(1, min(16, os.cpu_count() or 1, wh.H))  # the oracle's work units are the 8 heads
        n_tok = cpu_sample["q"].shape[1]
        passes, t0 = 0, time.perf_counter()
        while True:  # whole passes over the sample, for at least 10 s
            oracle.forward(cpu_sample["q"], cpu_sample["k"], cpu_sample["v"], cpu_sample["g"], cpu_sample["beta"],
                           None, nthreads=threads)
            passes += 1
            secs = time.perf_counter() - t0
            if secs >= 10.0:
                break
        out["cpu_baseline"] = {"value": passes * n_tok / secs, "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "host_cpu_count": os.cpu_count(),
                               "sample": "%d passes over the first %d tokens x %d heads of the %s workload (fp64, "
                                         "token by token, one thread per head), %.1f s wall on %d threads"
                                         % (passes, n_tok, wh.H, wh.name, secs, threads)}

    print(json.dumps(out))


if __name__ == "__main__":
    main()
