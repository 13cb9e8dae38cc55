"""Benchmark of the Falcon recurrence on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--copy-calibration]

A step is one falcon_chunk_fwd call for Falcon-1 over the whole batch B=8,
H=16, T=4096, d_k=d_v=128, bf16 q/k/v, fp32 state, chunk 64, with the inputs
resident in HBM: the intra-chunk kernel (norms, decay scan, masked Gram
blocks, diagonal-block inverses) and the state-passing kernel (residuals,
blocked forward substitution, outputs, state update).  `value` is tokens
(B*T) per second.  The same line reports Falcon-1A on the same batch,
Falcon-1 with same-step pairs (k_t, v_t), Falcon-1 with L2-normalized keys
and queries, Falcon-1 over 16 packed sequences
of mixed lengths with the same token count, the backward of Falcon-1 and
Falcon-1A on the same batch, a Falcon-1 training step (forward keeping the
backward's checkpoints, backward from them), Falcon-2 / Falcon-2A at B=4, H=32, T=8192 and
Falcon-3 / Falcon-3A (window 4) at B=2, H=16, T=32768, the decode step (256
sequences x 32 heads, d=128, 1024 consecutive steps) and the
Falcon-3 decode step at the same shape with a window of four, each with its
roofline, and the fp64 CPU oracle timed on this host over a bounded sample of
the Falcon-1 workload.

Before the first timed region, untimed Falcon-1 calls run for 0.3 s so the
device's clocks reach their sustained state (a fresh process otherwise times
its first ~100 calls up to 10% slow); every region then does its own
--warmup steps.

roofline.achieved is the algorithmic HBM bytes of one call (q, k, v, o once,
alpha, eta, final state) over the call's HIP-event time on the launch
stream; roofline.traffic is the HBM bytes the PMC counters measured for the
same call (profiles/), or null when the kernel sources changed since.
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
SETTLE_S = 0.3               # untimed calls before the first timed region
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA


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


def timed(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for _ in range(steps):
        fn()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


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
            "sample": f"Falcon-1 fp64 recurrent oracle on {n} of {B * H} (batch, head) "
                      f"sequences, full T={T}, d={D}; {wall:.1f} s wall; token-heads/s "
                      f"divided by H={H} to give tokens/s of the full workload"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter scaling)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(every (batch, head) sequence is independent; shard batch x head across GPUs)",
              file=sys.stderr)
        sys.exit(2)

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

    def step_f1():
        fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], "F1", chunk=C, o=o,
                      S_final=S_fin, workspace=ws)

    def step_f1a():
        fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], "F1A", chunk=C, o=o,
                      S_final=S_fin, workspace=ws)

    # Clocks settle: in a fresh process the first ~100 calls run up to 10%
    # slower while the device ramps to its sustained state, so untimed calls
    # run for at least SETTLE_S before the first warm-up of the first timed
    # region (each region then does its own `--warmup` steps).
    t_end = time.perf_counter() + SETTLE_S
    n_settle = 0
    while time.perf_counter() < t_end or n_settle < 20:
        for _ in range(10):
            step_f1()
        torch.cuda.synchronize()
        n_settle += 10
    print(f"[bench] chunk_fwd F1 {name}: settle {n_settle} calls, warmup {args.warmup}, "
          f"steps {args.steps}", file=sys.stderr, flush=True)
    ms, wall = timed(step_f1, args.steps, args.warmup)
    tok_s = B * T / (ms / 1e3)
    nbytes = chunk_bytes(B, H, T, D)
    nflops = chunk_flops(B, H, T, D, C, delta=True)
    gbs = nbytes / (ms / 1e3) / 1e9
    tfs = nflops / (ms / 1e3) / 1e12
    print(f"[bench] F1A", file=sys.stderr, flush=True)
    ms_a, _ = timed(step_f1a, args.steps, args.warmup)
    gbs_a = nbytes / (ms_a / 1e3) / 1e9

    def step_f1_same():
        fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], "F1", chunk=C, o=o,
                      S_final=S_fin, workspace=ws, align="same")

    print(f"[bench] F1 same-step pairs", file=sys.stderr, flush=True)
    ms_s, _ = timed(step_f1_same, args.steps, args.warmup)
    gbs_s = nbytes / (ms_s / 1e3) / 1e9

    ws_phi = torch.empty(fal.workspace_bytes(B, H, T, D, D, fal.BF16, "F1", 1, C, phi="l2"),
                         dtype=torch.uint8, device=dev)

    def step_f1_l2():
        fal.chunk_fwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], "F1", chunk=C, o=o,
                      S_final=S_fin, workspace=ws_phi, phi="l2")

    print(f"[bench] F1 with L2-normalized keys and queries", file=sys.stderr, flush=True)
    ms_p, _ = timed(step_f1_l2, args.steps, args.warmup)
    gbs_p = nbytes / (ms_p / 1e3) / 1e9
    del ws_phi

    # Falcon-1 over a packed batch of 16 sequences of mixed lengths with the
    # same 32768 tokens per head (falcon_chunk_fwd_varlen)
    rl = __import__("numpy").random.default_rng(5)
    lengths = rl.integers(256, 3840, 15).tolist()
    lengths.append(B * T - sum(lengths))
    vi = I.make_varlen_inputs(lengths, H, D, D, dtype="bf16", seed=980)
    tv = {n: torch.from_numpy(getattr(vi, n)).view(torch.bfloat16).to(dev) for n in ("q", "k", "v")}
    av, ev = torch.from_numpy(vi.alpha).to(dev), torch.from_numpy(vi.eta).to(dev)
    cu = torch.from_numpy(vi.cu).to(dev)
    maxT = max(lengths)
    ov = torch.empty_like(tv["v"])
    Sv = torch.empty((len(lengths), H, D, D), dtype=torch.float32, device=dev)
    wsv = torch.empty(fal.varlen_workspace_bytes(len(lengths), H, maxT, D, D, fal.BF16, "F1", 1, C),
                      dtype=torch.uint8, device=dev)

    def step_varlen():
        fal.chunk_fwd_varlen(tv["q"], tv["k"], tv["v"], av, ev, cu, "F1", max_seqlen=maxT, chunk=C,
                             o=ov, S_final=Sv, workspace=wsv)

    print(f"[bench] F1 packed varlen ({len(lengths)} sequences)", file=sys.stderr, flush=True)
    ms_v, _ = timed(step_varlen, args.steps, args.warmup)
    gbs_v = nbytes / (ms_v / 1e3) / 1e9
    del tv, ov, wsv

    # Backward (falcon_chunk_bwd) of Falcon-1 and Falcon-1A on the same batch:
    # forward recompute with checkpoints, reverse tile scan, per-tile gradients
    d_o_np, dS_np = I.make_cotangents(B, H, T, D, D, seed=w["seed"])
    d_o = torch.from_numpy(d_o_np).view(torch.bfloat16).to(dev)
    dS_fin = torch.from_numpy(dS_np).to(dev)
    del d_o_np, dS_np
    ws_b = torch.empty(fal.bwd_workspace_bytes(B, H, T, D, D, fal.BF16, "F1", 1, C),
                       dtype=torch.uint8, device=dev)

    def step_bwd(variant):
        return lambda: fal.chunk_bwd(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o, variant,
                                     dS_final=dS_fin, chunk=C, workspace=ws_b)

    print(f"[bench] F1 backward", file=sys.stderr, flush=True)
    ms_b, _ = timed(step_bwd("F1"), args.steps, args.warmup)
    print(f"[bench] F1A backward", file=sys.stderr, flush=True)
    ms_ba, _ = timed(step_bwd("F1A"), args.steps, args.warmup)
    nbytes_b = bwd_bytes(B, H, T, D)

    # A training step without the backward's forward re-run: the forward
    # keeps its records and checkpoints (falcon_chunk_fwd_save), the backward
    # reads them (falcon_chunk_bwd_saved)
    def step_train():
        fal.chunk_fwd_save(t["q"], t["k"], t["v"], t["alpha"], t["eta"], "F1", chunk=C, o=o,
                           S_final=S_fin, saved=ws_b)
        fal.chunk_bwd_saved(t["q"], t["k"], t["v"], t["alpha"], t["eta"], d_o, "F1",
                            dS_final=dS_fin, chunk=C, saved=ws_b)

    print(f"[bench] F1 training step (forward with checkpoints + backward from them)",
          file=sys.stderr, flush=True)
    ms_t, _ = timed(step_train, args.steps, args.warmup)
    del ws_b, d_o, dS_fin

    # The other full-size chunk-forward workloads: Falcon-2 (per-column
    # normalized step, lognormal key scales, long near-one decay spans) and
    # Falcon-3 / Falcon-3A with a window of four prefix-aligned pairs.  A
    # window of W turns each step into W virtual rows, so the chunk's 64 rows
    # hold 64 / W steps and the contraction work scales with T * W.
    extra = {}
    for wname, variants in (("falcon2_bf16_B4H32T8192d128", ("F2", "F2A")),
                            ("falcon3_w4_bf16_B2H16T32768d128", ("F3", "F3A"))):
        wx = I.WORKLOADS[wname]
        Bx, Hx, Tx, Dx, Wx = wx["B"], wx["H"], wx["T"], wx["d"], wx.get("window", 1)
        tx = I.workload_inputs(wname).to_torch(dev)
        ox = torch.empty_like(tx["v"])
        Sx = torch.empty((Bx, Hx, Dx, Dx), dtype=torch.float32, device=dev)
        wsx = torch.empty(max(fal.workspace_bytes(Bx, Hx, Tx, Dx, Dx, fal.BF16, v, Wx, C)
                              for v in variants), dtype=torch.uint8, device=dev)
        nb = chunk_bytes(Bx, Hx, Tx, Dx)
        for v in variants:
            def step_x(v=v):
                fal.chunk_fwd(tx["q"], tx["k"], tx["v"], tx["alpha"], tx["eta"], v, chunk=C,
                              window=Wx, o=ox, S_final=Sx, workspace=wsx)

            print(f"[bench] {v} {wname}", file=sys.stderr, flush=True)
            msx, _ = timed(step_x, args.steps, args.warmup)
            fl = chunk_flops(Bx, Hx, Tx * Wx, Dx, C, delta=not v.endswith("A"))
            gx = nb / (msx / 1e3) / 1e9
            tfx = fl / (msx / 1e3) / 1e12
            tag = v + (f"W{Wx}" if Wx > 1 else "")
            extra[v.lower().replace("f", "falcon")] = {
                "workload": wname, "tokens_per_s": Bx * Tx / (msx / 1e3), "ms_per_step": msx,
                "hbm_gbs": gx, "hbm_frac": gx / HBM_PEAK_GBS, "algorithmic_bytes_per_call": nb,
                "traffic": measured_traffic(f"chunk_fwd_{tag}_B{Bx}H{Hx}T{Tx}d{Dx}_bf16_c64"),
                "mfma_tflops": tfx, "mfma_frac_bf16": tfx / BF16_PEAK_TFLOPS,
                "algorithmic_flops_per_call": fl}
        del tx, ox, Sx, wsx

    line = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "variant": "F1", "B": B, "H": H, "T": T, "d_k": D,
                   "d_v": D, "chunk": C, "global_batch": B, "seq_len": T, "state": "fp32",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS,
                     "traffic": measured_traffic("chunk_fwd_F1_B8H16T4096d128_bf16_c64"),
                     "kernel": "chunk_prep2_kernel + chunk_pass_kernel (one falcon_chunk_fwd call)",
                     "algorithmic_bytes_per_launch": nbytes,
                     "mfma_tflops": tfs, "mfma_frac_bf16": tfs / BF16_PEAK_TFLOPS,
                     "algorithmic_flops_per_launch": nflops},
        "falcon1a": {"tokens_per_s": B * T / (ms_a / 1e3), "ms_per_step": ms_a,
                     "hbm_gbs": gbs_a, "hbm_frac": gbs_a / HBM_PEAK_GBS,
                     "traffic": measured_traffic("chunk_fwd_F1A_B8H16T4096d128_bf16_c64")},
        "falcon1_same_step": {"tokens_per_s": B * T / (ms_s / 1e3), "ms_per_step": ms_s,
                              "hbm_gbs": gbs_s, "hbm_frac": gbs_s / HBM_PEAK_GBS,
                              "pairs": "(k_t, v_t), FALCON_SAME_STEP"},
        "falcon1_phi_l2": {"tokens_per_s": B * T / (ms_p / 1e3), "ms_per_step": ms_p,
                           "hbm_gbs": gbs_p, "hbm_frac": gbs_p / HBM_PEAK_GBS,
                           "phi": "L2 normalization of keys and queries, FALCON_PHI_L2"},
        "falcon1_bwd": {"tokens_per_s": B * T / (ms_b / 1e3), "ms_per_step": ms_b,
                        "hbm_gbs": nbytes_b / (ms_b / 1e3) / 1e9,
                        "hbm_frac": nbytes_b / (ms_b / 1e3) / 1e9 / HBM_PEAK_GBS,
                        "algorithmic_bytes_per_call": nbytes_b,
                        "traffic": measured_traffic("chunk_bwd_F1_B8H16T4096d128_bf16_c64"),
                        "call": "falcon_chunk_bwd: dq, dk, dv, dalpha, deta, dS0 from d_o and "
                                "dS_final (forward recomputed inside)"},
        "falcon1_train_step": {"tokens_per_s": B * T / (ms_t / 1e3), "ms_per_step": ms_t,
                               "fwd_plus_recomputing_bwd_ms": ms + ms_b,
                               "call": "falcon_chunk_fwd_save (o, S_final and the backward's "
                                       "checkpoints) + falcon_chunk_bwd_saved"},
        "falcon1a_bwd": {"tokens_per_s": B * T / (ms_ba / 1e3), "ms_per_step": ms_ba,
                         "hbm_gbs": nbytes_b / (ms_ba / 1e3) / 1e9,
                         "hbm_frac": nbytes_b / (ms_ba / 1e3) / 1e9 / HBM_PEAK_GBS,
                         "traffic": measured_traffic("chunk_bwd_F1A_B8H16T4096d128_bf16_c64")},
        "falcon1_varlen": {"tokens_per_s": B * T / (ms_v / 1e3), "ms_per_step": ms_v,
                           "hbm_gbs": gbs_v, "hbm_frac": gbs_v / HBM_PEAK_GBS,
                           "batch": f"{len(lengths)} packed sequences, lengths {min(lengths)}.."
                                    f"{maxT}, {B * T} tokens per head, H={H}"},
    }
    line.update(extra)

    if not args.no_decode:
        wd = I.WORKLOADS["decode_falcon1_N256H32d128_1024steps"]
        N, Hd, Dd, steps = wd["N"], wd["H"], wd["d"], args.decode_steps
        x = I.make_decode_inputs_torch(N, Hd, Dd, Dd, steps, device=dev, seed=wd["seed"])
        S = x["S0"].clone()
        kc = x["k_cache0"].clone()
        od = torch.empty((N, Hd, Dd), dtype=torch.bfloat16, device=dev)
        counter = [0]

        def dec():
            s = counter[0] % steps
            counter[0] += 1
            fal.decode_step(S, kc, x["q"][s], x["k"][s], x["v"][s], x["alpha"][s],
                            x["eta"][s], "F1", o=od)

        print(f"[bench] decode {steps} steps", file=sys.stderr, flush=True)
        best = None
        for rep in range(3):
            S.copy_(x["S0"])
            kc.copy_(x["k_cache0"])
            counter[0] = 0
            torch.cuda.synchronize()
            ms_d, _ = timed(dec, steps, 0)
            best = ms_d if best is None else min(best, ms_d)
        db = decode_bytes(N, Hd, Dd)
        dgbs = db / (best / 1e3) / 1e9
        line["decode"] = {"workload": "decode_falcon1_N256H32d128_1024steps",
                          "tokens_per_s": N / (best / 1e3), "ms_per_step": best,
                          "steps": steps, "roofline": {
                              "bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                              "traffic": measured_traffic("decode_F1_N256H32d128_bf16"),
                              "algorithmic_bytes_per_launch": db,
                              "kernel": "decode_step_kernel<EBf16,128>"}}
        del x

        wn = "decode_falcon3_w4_N256H32d128_1024steps"
        w3 = I.WORKLOADS[wn]
        N, Hd, Dd, Wd = w3["N"], w3["H"], w3["d"], w3["window"]
        x = I.make_decode_inputs_torch(N, Hd, Dd, Dd, steps, device=dev, seed=w3["seed"],
                                       window=Wd)
        S = x["S0"].clone()
        kc = x["k_cache0"].clone()
        vc = x["v_cache0"].clone()

        def dec3():
            s = counter[0] % steps
            counter[0] += 1
            fal.decode_step_window(S, kc, vc, x["q"][s], x["k"][s], x["v"][s], x["alpha"][s],
                                   x["eta"][s], "F3", o=od)

        print(f"[bench] decode F3 window {Wd}, {steps} steps", file=sys.stderr, flush=True)
        best = None
        for rep in range(3):
            S.copy_(x["S0"])
            kc.copy_(x["k_cache0"])
            vc.copy_(x["v_cache0"])
            counter[0] = 0
            torch.cuda.synchronize()
            ms_d, _ = timed(dec3, steps, 0)
            best = ms_d if best is None else min(best, ms_d)
        db = decode_window_bytes(N, Hd, Dd, Wd)
        dgbs = db / (best / 1e3) / 1e9
        line["decode_falcon3"] = {"workload": wn, "tokens_per_s": N / (best / 1e3),
                                  "ms_per_step": best, "steps": steps, "roofline": {
                                      "bound": "hbm", "achieved": dgbs, "peak": HBM_PEAK_GBS,
                                      "unit": "GB/s", "frac": dgbs / HBM_PEAK_GBS,
                                      "traffic": measured_traffic("decode_F3W4_N256H32d128_bf16"),
                                      "algorithmic_bytes_per_launch": db,
                                      "kernel": "decode_window_kernel<EBf16,128,4>"}}
        del x

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["copy_calibration_bytes"] = 1 << 30

    if not args.no_cpu:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
