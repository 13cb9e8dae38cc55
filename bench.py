"""Benchmark of the Falcon recurrence on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-errors]
                    [--only SECTIONS] [--copy-calibration]

A step is one falcon_chunk_fwd call for Falcon-1 over the whole batch B=8,
H=16, T=4096, d_k=d_v=128, bf16 q/k/v, fp32 state, chunk 64, with the inputs
resident in HBM: the intra-chunk kernel (norms, decay scan, masked Gram
blocks, diagonal-block inverses) and the state-passing kernel (residuals,
blocked forward substitution, outputs, state update).  `value` is tokens
(B*T) per second over the K timed steps.  The same line reports Falcon-1A on
the same batch, Falcon-1 with same-step pairs (k_t, v_t), Falcon-1 with
L2-normalized keys and queries, Falcon-1 over 16 packed sequences of mixed
lengths with the same token count, the backward of Falcon-1 and Falcon-1A on
the same batch, a Falcon-1 training step (forward keeping the backward's
checkpoints, backward from them), Falcon-2 / Falcon-2A at B=4, H=32, T=8192
and Falcon-3 / Falcon-3A (window 4) at B=2, H=16, T=32768, the decode step
(256 sequences x 32 heads, d=128, 1024 consecutive steps) and the Falcon-3
decode step at the same shape with a window of four, each with its roofline
and its max relative error against the fp64 oracle (per (batch, head) slice,
max|gpu - oracle| / max|oracle| for o and for the final state, the maximum
over every slice; decode: a sample of 64 heads followed through all 1024
steps), and the fp64 CPU oracle timed on this host over a bounded sample of
the Falcon-1 workload.

Timing: each timed region records a HIP event on the launch stream before
the first step and after every step, so the line gives the mean over the K
steps (ms_per_step, which `value` uses) and the median and minimum per call.
Every timed region starts with untimed calls of its own step, back to back
for at least 0.3 s and at least --warmup of them, so the device's clocks are
at their sustained state when the timed steps begin: a fresh process times
its first ~100 calls up to 10% slow, and after the host has checked the
previous region's errors (the device idle for a second or more) a region
with only a few warm-up calls ran up to 20% slow.  The decode lines time the 1024 steps captured once as a HIP
graph (one launch per replay, as a serving loop would run them), after
checking that a replay leaves the eager steps' state bit for bit, and give
the eager loop's time (one launch per step) beside it.

roofline.achieved is the algorithmic HBM bytes of one call (q, k, v, o once,
alpha, eta, final state) over the call's mean HIP-event time; roofline.traffic
is the HBM bytes the PMC counters measured for the same call (profiles/), or
null when the kernel sources changed since.  The flops of each workload are
counted on the chunk form's contractions (Falcon-3/3A: the window form of
64-step chunks, E = C + W - 1 distinct keys, CW virtual examples).

--only takes a comma-separated subset of the sections f1, f1a, f1_same,
f1_l2, f1_varlen, bwd, f2, f3, decode, decode3 (for profiler runs; `value`
is null unless f1 runs).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Falcon-1 chunk fwd tokens/s (B8 H16 T4096 d128) + decode tok/s; % roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
SETTLE_S = 0.3               # untimed back-to-back calls before every timed region
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
SECTIONS = ("f1", "f1a", "f1_same", "f1_l2", "f1_varlen", "bwd", "f2", "f3", "decode", "decode3")


def chunk_bytes(B, H, T, D, elem=2, with_state_out=True):
    """Algorithmic HBM bytes of one chunk-forward call: q, k, v and o once
    (elem bytes each element), alpha and eta (fp32), final state (fp32)."""
    per_token_head = 3 * D * elem + 2 * 4 + D * elem
    return B * H * T * per_token_head + (B * H * D * D * 4 if with_state_out else 0)


def bwd_bytes(B, H, T, D, elem=2):
    """Algorithmic HBM bytes of one backward call: q, k, v, d_o read and dq,
    dk, dv written once (elem bytes each), alpha and eta read and their
    gradients written (fp32), dS_final read and dS0 written (fp32)."""
    per_token_head = 7 * D * elem + 4 * 4
    return B * H * T * per_token_head + 2 * B * H * D * D * 4


def chunk_flops(B, H, T, D, C, delta=True):
    """Algorithmic flops of the chunk form per call, counted on full C x C
    tiles: Grams, the triangular solve, the two C x d products per side of the
    state, and the state update (delta family); A family without the solve."""
    if delta:
        per = 2 * C * C * (3 * D + 2 * D) + 6 * C * D * D + 2 * C ** 3 / 3
    else:
        per = 2 * C * C * (D + D) + 4 * C * D * D
    return B * H * (T // C) * per


def window_flops(B, H, T, D, C, W, delta=True):
    """Algorithmic flops of the window rules (Falcon-3 / Falcon-3A) per call,
    on chunks of C steps: E = C + W - 1 distinct keys serve the C W virtual
    examples.  Falcon-3: the extended key Gram (2 E^2 d) and the query-key
    products (2 C E d), the CW x CW triangular solve (2 (CW)^3 / 3), the
    transformed keys and targets (2 (CW)^2 (d_k + d_v)), the residual
    product (2 CW d_k d_v), the state read by the queries (2 C d_k d_v), the
    intra-chunk outputs (2 C CW d_v) and the state update over the E keys
    (2 E d_k d_v).  Falcon-3A: banded outputs 2 C E (d_k + d_v), the state
    read 2 C d_k d_v and the update 2 E d_k d_v."""
    E, Cv = C + W - 1, C * W
    if delta:
        per = (2 * E * E * D + 2 * C * E * D + 2 * Cv ** 3 / 3 + 2 * Cv * Cv * (D + D)
               + 2 * Cv * D * D + 2 * C * D * D + 2 * C * Cv * D + 2 * E * D * D)
    else:
        per = 2 * C * E * (D + D) + 2 * C * D * D + 2 * E * D * D
    return B * H * (T // C) * per


def decode_bytes(N, H, D, elem=2):
    """Per step: state read + write (fp32), q, k, v, the key cache read and
    rewritten, alpha, eta, and o."""
    return N * H * (2 * D * D * 4 + 3 * D * elem + 2 * D * elem + 2 * 4 + D * elem)


def decode_window_bytes(N, H, D, W, elem=2):
    """Per Falcon-3 step: state read + write (fp32), q, k, v, o, the key cache
    (W slots) and the value cache (W - 1 slots) each read and rewritten,
    alpha, eta."""
    return N * H * (2 * D * D * 4 + 4 * D * elem + 2 * W * D * elem + 2 * (W - 1) * D * elem
                    + 2 * 4)


def measured_traffic(entry):
    """HBM bytes per call from profiles/traffic.json, if the kernel sources
    still hash to what the counters were taken on; else None."""
    import hashlib
    try:
        t = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
        e = t["entries"][entry]
        m = hashlib.sha256()
        for f in e["sources"]:
            m.update(open(os.path.join(ROOT, "weight_recurrent_sequence_amd", "csrc", f), "rb").read())
        if m.hexdigest() != e["sources_sha256"]:
            return None
        return sum(k["fetch_kib"] * 1024 * t["fetch_scale"] + k["write_kib"] * 1024 * t["write_scale"]
                   for k in e["kernels"].values())
    except (OSError, KeyError, ValueError):
        return None


def settle(fn, seconds, min_calls=0):
    """Untimed calls of fn, back to back, for at least `seconds` and at least
    `min_calls` calls; returns their number.  The device lowers its clocks
    while it idles (the host checking a region's errors against the oracle,
    for one) and takes a few hundred milliseconds under load to bring them
    back, so a few warm-up calls alone leave the next region's timed calls
    up to 20% slow.  Synchronizes every four calls, so the queue stays short."""
    import torch
    t_end = time.perf_counter() + seconds
    n = 0
    while n < min_calls or time.perf_counter() < t_end:
        for _ in range(4):
            fn()
        n += 4
        torch.cuda.synchronize()
    return n


def timed(fn, steps, warmup, settle_s=SETTLE_S):
    """Mean, median and minimum milliseconds per call of `steps` calls, from
    HIP events on the current stream (one before the first call, one after
    each); synchronized before and after.  Before them, untimed calls for at
    least `settle_s` seconds and at least `warmup` calls."""
    import torch
    settle(fn, settle_s, warmup)
    st = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(st)
    for i in range(steps):
        fn()
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    mid = steps // 2
    median = per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])
    return {"mean": ev[0].elapsed_time(ev[steps]) / steps, "median": median, "min": per[0],
            "wall": wall}


def slice_rel_err(got, ref, axes):
    """Max over slices of max|got - ref| / max|ref| (a slice = the leading
    axes not in `axes`)."""
    import numpy as np
    num = np.abs(np.asarray(got, np.float64) - ref).max(axis=axes)
    den = np.abs(ref).max(axis=axes)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max()) if num.size else 0.0


def to_f64(t):
    import numpy as np
    return t.float().cpu().numpy().astype(np.float64)


def chunk_errors(inp, variant, W, o, S, align="prefix", phi="identity"):
    """Max relative error of o and S_final against the fp64 oracle over every
    (batch, head) sequence of the call."""
    import oracle
    o_np, S_np = to_f64(o), to_f64(S)
    d = inp.f64()
    o_ref, S_ref = oracle.recurrent(variant, d["q"], d["k"], d["v"], d["alpha"], d["eta"],
                                    window=W, align=align, phi=phi)
    del d
    B, H = o_np.shape[:2]
    return {"o": slice_rel_err(o_np, o_ref, (2, 3)), "S": slice_rel_err(S_np, S_ref, (2, 3)),
            "sequences": B * H, "tolerance": 2e-2 if inp.dtype == "bf16" else 1e-4}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, budget_s=12.0):
    """fp64 oracle on this host's cores over a bounded sample of whole
    sequences of the Falcon-1 workload."""
    import numpy as np

    import oracle
    B, H, T, D = inp.k.shape
    cores = oracle.num_cpus()
    # calibrate on one sequence
    d1 = inp.f64((np.array([0]), np.array([0])))
    t0 = time.perf_counter()
    oracle.recurrent("F1", *(d1[x][None] for x in ("q", "k", "v", "alpha", "eta")), nthreads=1)
    t_one = time.perf_counter() - t0
    n = int(max(1, min(B * H, budget_s * cores / max(t_one, 1e-6))))
    n = max(min(n, B * H), 1)
    idx = np.arange(n)
    bs, hs = idx // H, idx % H
    d = inp.f64((bs, hs))
    t0 = time.perf_counter()
    used = oracle.recurrent_threads_used(1, n)
    oracle.recurrent("F1", *(d[x][None] for x in ("q", "k", "v", "alpha", "eta")))
    wall = time.perf_counter() - t0
    token_heads_per_s = n * T / wall
    return {"value": token_heads_per_s / H, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"Falcon-1 fp64 recurrent oracle on {n} of {B * H} (batch, head) "
                      f"sequences, full T={T}, d={D}; {wall:.1f} s wall; token-heads/s "
                      f"divided by H={H} to give tokens/s of the full workload"}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-errors", action="store_true",
                    help="skip the oracle comparisons of the full-size outputs")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--only", default=",".join(SECTIONS),
                    help="comma-separated sections to run: " + ", ".join(SECTIONS))
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(every (batch, head) sequence is independent; shard batch x head across GPUs)",
              file=sys.stderr)
        sys.exit(2)
    only = set(s.strip() for s in args.only.split(",") if s.strip())
    bad = only - set(SECTIONS)
    if bad:
        ap.error(f"unknown sections {sorted(bad)}")
    if args.no_decode:
        only -= {"decode", "decode3"}
    errors = not args.no_errors

    import numpy as np
    import torch

    import weight_recurrent_sequence_amd as fal
    from weight_recurrent_sequence_amd import inputs as I
    if not os.path.exists(fal.binding.LIB_PATH):
        from weight_recurrent_sequence_amd import _build
        _build.build()
    dev = torch.device("cuda:0")

    name = "falcon1_bf16_B8H16T4096d128"
    w = I.WORKLOADS[name]
    B, H, T, D, C = w["B"], w["H"], w["T"], w["d"], w["chunk"]
    inp = I.workload_inputs(name)
    t = inp.to_torch(dev)
    o = torch.empty_like(t["v"])
    S_fin = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(fal.workspace_bytes(B, H, T, D, D, fal.BF16, "F1", 1, C), dtype=torch.uint8,
                     device=dev)
    nbytes = chunk_bytes(B, H, T, D)

    def fwd(variant, **kw):
        return lambda: fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], variant,
                                     chunk=C, o=o, S_final=S_fin, **kw)

    # Clocks settle: in a fresh process the first ~100 calls run up to 10%
    # slower while the device ramps to its sustained state, and after an
    # idle gap it ramps again, so every timed region starts with untimed
    # calls of its own for at least SETTLE_S (and at least `--warmup`).
    step_f1 = fwd("F1", workspace=ws)
    n_settle = settle(step_f1, SETTLE_S, 20)
    log(f"settle {n_settle} Falcon-1 calls, warmup {args.warmup}, steps {args.steps}")

    def rate(tm, nb, tokens):
        return {"tokens_per_s": tokens / (tm["mean"] / 1e3), "ms_per_step": tm["mean"],
                "ms_median": tm["median"], "ms_min": tm["min"],
                "hbm_gbs": nb / (tm["mean"] / 1e3) / 1e9,
                "hbm_frac": nb / (tm["mean"] / 1e3) / 1e9 / HBM_PEAK_GBS}

    line = {"metric": METRIC, "value": None, "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": None,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": name, "variant": "F1", "B": B, "H": H, "T": T, "d_k": D,
                       "d_v": D, "chunk": C, "global_batch": B, "seq_len": T, "state": "fp32",
                       "parallelism": "single GPU"}}

    if "f1" in only:
        log(f"chunk_fwd F1 {name}")
        tm = timed(step_f1, args.steps, args.warmup)
        ms = tm["mean"]
        nflops = chunk_flops(B, H, T, D, C, delta=True)
        gbs = nbytes / (ms / 1e3) / 1e9
        tfs = nflops / (ms / 1e3) / 1e12
        line["value"] = B * T / (ms / 1e3)
        line["ms_per_step"] = ms
        line["ms_median"] = tm["median"]
        line["ms_min"] = tm["min"]
        line["roofline"] = {
            "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic("chunk_fwd_F1_B8H16T4096d128_bf16_c64"),
            "kernel": "chunk_prep2_kernel + chunk_pass_kernel (one falcon_chunk_fwd call)",
            "algorithmic_bytes_per_launch": nbytes,
            "mfma_tflops": tfs, "mfma_frac_bf16": tfs / BF16_PEAK_TFLOPS,
            "algorithmic_flops_per_launch": nflops}
        if errors:
            log("F1 errors against the oracle (every sequence)")
            line["errors"] = chunk_errors(inp, "F1", 1, o, S_fin)

    if "f1a" in only:
        log("F1A")
        tm = timed(fwd("F1A", workspace=ws), args.steps, args.warmup)
        fl = chunk_flops(B, H, T, D, C, delta=False)
        r = rate(tm, nbytes, B * T)
        r.update({"kernels": "fused_kernel<128> (one falcon_chunk_fwd call)",
                  "traffic": measured_traffic("chunk_fwd_F1A_B8H16T4096d128_bf16_c64"),
                  "algorithmic_flops_per_call": fl,
                  "mfma_frac_bf16": fl / (tm["mean"] / 1e3) / 1e12 / BF16_PEAK_TFLOPS})
        if errors:
            r["errors"] = chunk_errors(inp, "F1A", 1, o, S_fin)
        line["falcon1a"] = r

    if "f1_same" in only:
        log("F1 same-step pairs")
        tm = timed(fwd("F1", workspace=ws, align="same"), args.steps, args.warmup)
        r = rate(tm, nbytes, B * T)
        r["pairs"] = "(k_t, v_t), FALCON_SAME_STEP"
        if errors:
            r["errors"] = chunk_errors(inp, "F1", 1, o, S_fin, align="same")
        line["falcon1_same_step"] = r

    if "f1_l2" in only:
        ws_phi = torch.empty(fal.workspace_bytes(B, H, T, D, D, fal.BF16, "F1", 1, C, phi="l2"),
                             dtype=torch.uint8, device=dev)
        log("F1 with L2-normalized keys and queries")
        tm = timed(fwd("F1", workspace=ws_phi, phi="l2"), args.steps, args.warmup)
        r = rate(tm, nbytes, B * T)
        r["phi"] = "L2 normalization of keys and queries, FALCON_PHI_L2"
        if errors:
            r["errors"] = chunk_errors(inp, "F1", 1, o, S_fin, phi="l2")
        line["falcon1_phi_l2"] = r
        del ws_phi

    if "f1_varlen" in only:
        # Falcon-1 over a packed batch of 16 sequences of mixed lengths with
        # the same 32768 tokens per head (falcon_chunk_fwd_varlen)
        rl = np.random.default_rng(5)
        lengths = rl.integers(256, 3840, 15).tolist()
        lengths.append(B * T - sum(lengths))
        vi = I.make_varlen_inputs(lengths, H, D, D, dtype="bf16", seed=980)
        tv = {n: torch.from_numpy(getattr(vi, n)).view(torch.bfloat16).to(dev)
              for n in ("q", "k", "v")}
        av, ev = torch.from_numpy(vi.alpha).to(dev), torch.from_numpy(vi.eta).to(dev)
        cu = torch.from_numpy(vi.cu).to(dev)
        maxT = max(lengths)
        ov = torch.empty_like(tv["v"])
        Sv = torch.empty((len(lengths), H, D, D), dtype=torch.float32, device=dev)
        wsv = torch.empty(fal.varlen_workspace_bytes(len(lengths), H, maxT, D, D, fal.BF16, "F1",
                                                     1, C), dtype=torch.uint8, device=dev)

        def step_varlen():
            fal.chunk_fwd_varlen(tv["q"], tv["k"], tv["v"], av, ev, cu, "F1", max_seqlen=maxT,
                                 chunk=C, o=ov, S_final=Sv, workspace=wsv)

        log(f"F1 packed varlen ({len(lengths)} sequences)")
        tm = timed(step_varlen, args.steps, args.warmup)
        r = rate(tm, nbytes, B * T)
        r["batch"] = (f"{len(lengths)} packed sequences, lengths {min(lengths)}..{maxT}, "
                      f"{B * T} tokens per head, H={H}")
        line["falcon1_varlen"] = r
        del tv, ov, wsv

    if "bwd" in only:
        # Backward (falcon_chunk_bwd) of Falcon-1 and Falcon-1A on the same
        # batch: forward recompute with checkpoints, reverse tile scan,
        # per-tile gradients
        d_o_np, dS_np = I.make_cotangents(B, H, T, D, D, seed=w["seed"])
        d_o = torch.from_numpy(d_o_np).view(torch.bfloat16).to(dev)
        dS_fin = torch.from_numpy(dS_np).to(dev)
        del d_o_np, dS_np
        ws_b = torch.empty(fal.bwd_workspace_bytes(B, H, T, D, D, fal.BF16, "F1", 1, C),
                           dtype=torch.uint8, device=dev)

        def step_bwd(variant):
            return lambda: fal.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o,
                                         variant, dS_final=dS_fin, chunk=C, workspace=ws_b)

        nbytes_b = bwd_bytes(B, H, T, D)
        log("F1 backward")
        tm = timed(step_bwd("F1"), args.steps, args.warmup)
        r = rate(tm, nbytes_b, B * T)
        r.update({"algorithmic_bytes_per_call": nbytes_b,
                  "traffic": measured_traffic("chunk_bwd_F1_B8H16T4096d128_bf16_c64"),
                  "call": "falcon_chunk_bwd: dq, dk, dv, dalpha, deta, dS0 from d_o and "
                          "dS_final (forward recomputed inside)"})
        line["falcon1_bwd"] = r
        log("F1A backward")
        tm = timed(step_bwd("F1A"), args.steps, args.warmup)
        r = rate(tm, nbytes_b, B * T)
        r["traffic"] = measured_traffic("chunk_bwd_F1A_B8H16T4096d128_bf16_c64")
        line["falcon1a_bwd"] = r

        # A training step without the backward's forward re-run: the forward
        # keeps its records and checkpoints (falcon_chunk_fwd_save), the
        # backward reads them (falcon_chunk_bwd_saved)
        def step_train():
            fal.chunk_fwd_save(t["q"], t["k"], t["v"], t["alpha"], t["eta"], "F1", chunk=C, o=o,
                               S_final=S_fin, saved=ws_b)
            fal.chunk_bwd_saved(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o, "F1",
                                dS_final=dS_fin, chunk=C, saved=ws_b)

        log("F1 training step (forward with checkpoints + backward from them)")
        tm = timed(step_train, args.steps, args.warmup)
        line["falcon1_train_step"] = {
            "tokens_per_s": B * T / (tm["mean"] / 1e3), "ms_per_step": tm["mean"],
            "ms_median": tm["median"], "ms_min": tm["min"],
            "call": "falcon_chunk_fwd_save (o, S_final and the backward's checkpoints) + "
                    "falcon_chunk_bwd_saved"}
        del ws_b, d_o, dS_fin

    # The other full-size chunk-forward workloads: Falcon-2 (per-column
    # normalized step, lognormal key scales, long near-one decay spans) and
    # Falcon-3 / Falcon-3A with a window of four prefix-aligned pairs.
    for sec, wname, variants in (("f2", "falcon2_bf16_B4H32T8192d128", ("F2", "F2A")),
                                 ("f3", "falcon3_w4_bf16_B2H16T32768d128", ("F3", "F3A"))):
        if sec not in only:
            continue
        wx = I.WORKLOADS[wname]
        Bx, Hx, Tx, Dx, Wx = wx["B"], wx["H"], wx["T"], wx["d"], wx.get("window", 1)
        ix = I.workload_inputs(wname)
        tx = ix.to_torch(dev)
        ox = torch.empty_like(tx["v"])
        Sx = torch.empty((Bx, Hx, Dx, Dx), dtype=torch.float32, device=dev)
        wsx = torch.empty(max(fal.workspace_bytes(Bx, Hx, Tx, Dx, Dx, fal.BF16, v, Wx, C)
                              for v in variants), dtype=torch.uint8, device=dev)
        nb = chunk_bytes(Bx, Hx, Tx, Dx)
        for v in variants:
            def step_x(v=v):
                fal.chunk_fwd(tx["q"], tx["k"], tx["v"], tx["alpha"], tx["eta"], v, chunk=C,
                              window=Wx, o=ox, S_final=Sx, workspace=wsx)

            log(f"{v} {wname}")
            tm = timed(step_x, args.steps, args.warmup)
            delta = not v.endswith("A")
            fl = (window_flops(Bx, Hx, Tx, Dx, C, Wx, delta) if Wx > 1
                  else chunk_flops(Bx, Hx, Tx, Dx, C, delta))
            tfx = fl / (tm["mean"] / 1e3) / 1e12
            tag = v + (f"W{Wx}" if Wx > 1 else "")
            r = rate(tm, nb, Bx * Tx)
            r.update({"workload": wname, "algorithmic_bytes_per_call": nb,
                      "kernels": (("win_prep_kernel + win_pass_kernel" if delta else
                                   "win_prep_kernel + win_seg_kernel + win_pass_kernel (4 segments)")
                                  if Wx > 1 else ("chunk_prep2_kernel + chunk_pass_kernel" if delta
                                                  else "fused_kernel<128, per-column write vectors>")),
                      "traffic": measured_traffic(f"chunk_fwd_{tag}_B{Bx}H{Hx}T{Tx}d{Dx}_bf16_c64"),
                      "mfma_tflops": tfx, "mfma_frac_bf16": tfx / BF16_PEAK_TFLOPS,
                      "algorithmic_flops_per_call": fl})
            if errors:
                log(f"{v} errors against the oracle (every sequence)")
                r["errors"] = chunk_errors(ix, v, Wx, ox, Sx)
            line[v.lower().replace("f", "falcon")] = r
        del tx, ox, Sx, wsx, ix

    for sec, wn, variant in (("decode", "decode_falcon1_N256H32d128_1024steps", "F1"),
                             ("decode3", "decode_falcon3_w4_N256H32d128_1024steps", "F3")):
        if sec not in only:
            continue
        wd = I.WORKLOADS[wn]
        N, Hd, Dd, steps = wd["N"], wd["H"], wd["d"], args.decode_steps
        Wd = wd.get("window", 1)
        x = I.make_decode_inputs_torch(N, Hd, Dd, Dd, steps, device=dev, seed=wd["seed"],
                                       window=Wd)
        S = x["S0"].clone()
        kc = x["k_cache0"].clone()
        vc = x["v_cache0"].clone() if Wd > 1 else None
        od = torch.empty((N, Hd, Dd), dtype=torch.bfloat16, device=dev)
        # a sample of heads whose outputs are kept at every step of the last
        # repeat, for the oracle comparison
        rs = np.random.default_rng(wd["seed"])
        flat = rs.choice(N * Hd, 64, replace=False)
        ns = torch.from_numpy(flat // Hd).to(dev)
        hs = torch.from_numpy(flat % Hd).to(dev)
        keep = torch.empty((steps, 64, Dd), dtype=torch.bfloat16, device=dev)
        counter = [0]

        def dec():
            s = counter[0] % steps
            counter[0] += 1
            if Wd > 1:
                fal.decode_step_window(S, kc, vc, x["q"][s], x["k"][s], x["v"][s], x["alpha"][s],
                                       x["eta"][s], variant, o=od)
            else:
                fal.decode_step(S, kc, x["q"][s], x["k"][s], x["v"][s], x["alpha"][s],
                                x["eta"][s], variant, o=od)

        def reset():
            S.copy_(x["S0"])
            kc.copy_(x["k_cache0"])
            if vc is not None:
                vc.copy_(x["v_cache0"])
            counter[0] = 0
            torch.cuda.synchronize()

        log(f"decode {variant} window {Wd}, {steps} steps")
        settle(dec, SETTLE_S)
        eager = []
        for rep in range(3):
            reset()
            eager.append(timed(dec, steps, 0, settle_s=0.0)["mean"])
        eager.sort()
        S_eager = S.clone()
        # The same steps captured once as a HIP graph (a serving loop would
        # launch them so): one launch per replay instead of one per step.
        # Each replay starts from the initial state; the first must leave
        # the state the eager run left, bit for bit, or the eager times stand.
        reps, graph_ok = [], False
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                reset()
                for _ in range(2):
                    dec()
            torch.cuda.current_stream().wait_stream(side)
            reset()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(steps):
                    dec()
            for rep in range(3):
                reset()
                st = torch.cuda.current_stream()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(st)
                g.replay()
                e1.record(st)
                torch.cuda.synchronize()
                reps.append(e0.elapsed_time(e1) / steps)
                if rep == 0:
                    graph_ok = bool(torch.equal(S, S_eager))
            del g
        except Exception as ex:  # capture not available: keep the eager times
            log(f"decode graph capture failed: {ex}")
        if not graph_ok:
            reps = eager
        reps.sort()
        db = decode_window_bytes(N, Hd, Dd, Wd) if Wd > 1 else decode_bytes(N, Hd, Dd)
        med, best = reps[1], reps[0]
        dgbs = db / (med / 1e3) / 1e9
        r = {"workload": wn, "tokens_per_s": N / (med / 1e3), "ms_per_step": med,
             "ms_per_step_min": best, "repeats_ms_per_step": reps,
             "timing": "hip graph of the steps" if graph_ok else "one launch per step",
             "ms_per_step_eager": eager[1], "repeats_ms_per_step_eager": eager,
             "steps": steps, "roofline": {
                 "bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": dgbs / HBM_PEAK_GBS,
                 "frac_min_time": db / (best / 1e3) / 1e9 / HBM_PEAK_GBS,
                 "traffic": measured_traffic("decode_F1_N256H32d128_bf16" if Wd == 1
                                             else f"decode_F3W{Wd}_N256H32d128_bf16"),
                 "algorithmic_bytes_per_launch": db,
                 "kernel": (f"decode_window_kernel<EBf16,128,{Wd}>" if Wd > 1
                            else "decode_step_kernel<EBf16,128>")}}
        if errors:
            # one more pass from the initial state, untimed, keeping the
            # sampled heads' outputs; the oracle follows them through every step
            import oracle
            log(f"decode {variant} errors against the oracle (64 sampled heads, {steps} steps)")
            S.copy_(x["S0"])
            kc.copy_(x["k_cache0"])
            if vc is not None:
                vc.copy_(x["v_cache0"])
            counter[0] = 0
            for s in range(steps):
                dec()
                keep[s] = od[ns, hs]
            torch.cuda.synchronize()
            S_o = to_f64(x["S0"][ns, hs])[None]
            kc_o = to_f64(x["k_cache0"][ns, hs])[None]
            vc_o = to_f64(x["v_cache0"][ns, hs])[None] if Wd > 1 else None
            o_ref = np.empty((steps, 64, Dd))
            sel = {n: to_f64(x[n][:, ns, hs]) for n in ("q", "k", "v", "alpha", "eta")}
            for s in range(steps):
                args_s = [sel[n][s][None] for n in ("q", "k", "v", "alpha", "eta")]
                if Wd > 1:
                    o1, S_o, kc_o, vc_o = oracle.decode_step_window(variant, S_o, kc_o, vc_o,
                                                                    *args_s)
                else:
                    o1, S_o, kc_o = oracle.decode_step(variant, S_o, kc_o[:, :, 0], *args_s)
                    kc_o = kc_o[:, :, None]
                o_ref[s] = o1[0]
            r["errors"] = {
                "o": slice_rel_err(np.moveaxis(to_f64(keep), 0, 1), np.moveaxis(o_ref, 0, 1),
                                   (1, 2)),
                "S": slice_rel_err(to_f64(S[ns, hs]), S_o[0], (1, 2)),
                "sequences": 64, "steps": steps, "tolerance": 2e-2}
        line["decode" if Wd == 1 else "decode_falcon3"] = r
        del x, S, kc, vc, keep

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = 1 << 30

    if not args.no_cpu:
        log("cpu baseline (fp64 oracle)")
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
