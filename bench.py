"""Throughput of the folded multi-branch verification layer on one MI355X.

One step = one pass of the whole hot path -- gate, compaction, fold-source resolution,
sparse QKV, folded attention, output projection, sparse FFN and fold-inherit -- over one
verification batch (main + B drafts), through ``specfold_verify_layer``.

Workload (seeded, synthetic): one layer at 1.5B-class shape (hidden 1536, 12 q / 2 kv heads,
head_dim 128, SwiGLU 8960), block 32, main + 8 drafts in a random tree of depth <= 4, prefix
512 tokens, delta 0.1.  Timing replays a HIP graph of K steps bracketed by events; inputs are
resident in HBM before the timed region.  Regime "cold" rotates through copies of the layer's
weights totalling more than the 256 MB Infinity Cache, so every step streams its weights from
HBM as a layer of a real stack does; "warm" reuses one copy.

Prints one JSON line: the throughput fields (metric, value, unit, steps, ms_per_step, config,
...), the dense (delta 0) path of the same kernels and their ratio, the dominant kernel's
roofline object (achieved against peak, with the counter-measured HBM traffic while the GEMM
sources match the committed record), per-launch stage times, and the CPU oracle's rate on a
bounded sample of the same input (cpu_baseline) with the check of the GPU's output against it.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified branch-tokens/s per layer stack at delta=0.1; speedup vs dense delta=0"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="steps per timed graph replay (exactly this many; the median of --rounds replays is "
                         "reported); a step is one verification pass through the workload's layers (default: "
                         "16 for the 28-layer stacks, 200 for single layers)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rounds", type=int, default=5, help="timed replays of the K-step graph (median reported)")
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="keep replaying (untimed) at least this long before timing, so clocks have ramped")
    ap.add_argument("--workload", default="stack-1.5b",
                    help="stack-1.5b (default: the 28-layer 1.5B-shape stack, with the single 1.5B layer as a "
                         "sub-object), stack-7b, layer-1.5b, sweep-14b, draft-shapes-1.5b")
    ap.add_argument("--no-layer", action="store_true",
                    help="stack-1.5b: skip the single-layer (layer-1.5b) sub-object of the default line")
    ap.add_argument("--regime", choices=["cold", "warm"], default="cold")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--stage-calls", type=int, default=30, help="eager calls timed per launch with events")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration runs)")
    ap.add_argument("--counters", type=int, default=0,
                    help="hardware-counter runs: after the eager reference calls, run this many folded and "
                         "then as many dense layer steps (cold weights), the flat gate and compaction once "
                         "each and a 256 MiB device copy, print the dispatch plan and exit (no timing)")
    ap.add_argument("--layers", type=int, default=0, help="stack workloads: layers (default: the workload's)")
    ap.add_argument("--stack-steps", type=int, default=0, help="stack workloads: steps (default: the workload's)")
    ap.add_argument("--no-gate-flat", action="store_true", help="skip the large flat gate/compaction timing")
    ap.add_argument("--with-head", action="store_true",
                    help="stack workloads: also time whole verification passes from token ids: embedding "
                         "gather, the layer stack and the final RMSNorm + LM head + greedy token")
    ap.add_argument("--vocab", type=int, default=151936, help="vocabulary of the --with-head passes")
    ap.add_argument("--correction", action="store_true",
                    help="also time the pages' attention-state correction (variants/) against the library's merge")
    ap.add_argument("--serialized", action="store_true",
                    help="also time serialized verification (each branch alone, delta 0) and compare it "
                         "with the batched dense layer")
    return ap.parse_args()


# Per-kernel fractions of the vendor peaks (event-timed launches): MFMA for the contractions
# (GEMMs, attention), HBM for every kernel.  Bytes are what each launch must move (weights,
# activations, outputs, prefix cache), not split-K partials or chunk states; the epilogue kernels
# have no algorithmic bytes of their own beyond the rows they write.  Cold, a contraction of
# intensity I = flops/bytes cannot exceed I * 8 TB/s of MFMA work, i.e. a fraction
# mfma_cap_cold = min(1, I * HBM peak / MFMA peak) of the MFMA peak.
def kernel_work(sh, name, m):
    """(flops, bytes) of one launch of stage `name` of a layer of shape sh with m recompute rows."""
    R, D, F = sh.rows, sh.hidden, sh.ffn
    d, Hq, Hkv, P, N = sh.head_dim, sh.n_q_heads, sh.n_kv_heads, sh.prefix_len, sh.block
    Nq, Do = (Hq + 2 * Hkv) * d, Hq * d
    table = {
        "gate_rmsnorm": (0, 2 * R * D + 2 * D + 2 * R * D + 9 * R),
        "qkv_gemm_compact_resolve": (2 * m * Nq * D, 2 * Nq * D + 2 * m * D + 2 * m * Nq),
        "qkv_rope_epilogue": (0, 2 * m * Nq),
        "attention": (4 * d * Hq * (P * m + N * R), 4 * P * Hkv * d + 2 * m * Nq + 2 * R * Do),
        "oproj_gemm": (2 * R * Do * D, 2 * Do * D + 2 * R * Do + 2 * R * D),
        "oproj_residual_rmsnorm": (0, 2 * R * D + 4 * R * D),
        "gate_up_swiglu_gemm": (2 * m * 2 * F * D, 2 * 2 * F * D + 2 * m * D + 2 * m * F),
        "down_gemm": (2 * m * F * D, 2 * F * D + 2 * m * F + 2 * m * D),
        "down_inherit_epilogue": (0, 4 * R * D),
    }
    return table.get(name)


def kernel_pct(sh, st, m):
    """Per-stage event-timed microseconds -> fractions of the vendor peaks (the two attention
    launches are reported together)."""
    st = dict(st)
    attn = sum(v for k, v in st.items() if k.startswith("attn"))
    st = {k: v for k, v in st.items() if not k.startswith("attn")}
    st["attention"] = attn
    out_ = {}
    for k, us in st.items():
        w_ = kernel_work(sh, k, m)
        if w_ is None or us <= 0:
            continue
        flops, byts = w_
        sec = us * 1e-6
        row = {"us": round(us, 2), "hbm_frac": round(byts / sec / (HBM_PEAK_GBS * 1e9), 4), "bytes": byts}
        if flops:
            row["mfma_frac"] = round(flops / sec / (BF16_PEAK_TFLOPS * 1e12), 4)
            row["mfma_cap_cold"] = round(min(1.0, flops / byts * HBM_PEAK_GBS * 1e9 / (BF16_PEAK_TFLOPS * 1e12)), 4)
        out_[k] = row
    return out_


def layer_roof_us(sh, m):
    """Whole-layer roofline time at the vendor peaks: sum over the contractions and the gate of
    max(bytes / BW, flops / MFMA) (the epilogues' rows are written by the kernels they follow in
    a fused design)."""
    t = 0.0
    for k in ("gate_rmsnorm", "qkv_gemm_compact_resolve", "attention", "oproj_gemm", "gate_up_swiglu_gemm",
              "down_gemm"):
        flops, byts = kernel_work(sh, k, m)
        t += max(flops / (BF16_PEAK_TFLOPS * 1e12), byts / (HBM_PEAK_GBS * 1e9))
    return t * 1e6


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "this build has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    from synth import WORKLOADS

    wl = WORKLOADS[args.workload]
    if args.steps <= 0:
        args.steps = 16 if (wl.layers > 1 or args.layers > 1) else 200
    if wl.layers > 1 or args.layers > 1:
        return stack_bench(args, wl)
    if wl.branch_sweep:
        return sweep_bench(args, wl)
    if wl.tree_sweep:
        return tree_bench(args, wl)
    return layer_main(args, wl)


def layer_main(args, wl, emit=True):
    """One layer (layer-1.5b): cold and warm, folded and dense, per-launch event timing, the flat
    gate and compaction; prints the line (emit) and returns it."""
    import numpy as np
    import torch

    from sparse_layer_rho_amd import specfold as sf
    from synth import bf16_round, layer_weights, prefix_kv, step_inputs

    sh = wl.shape
    R, D, F = sh.rows, sh.hidden, sh.ffn
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(torch.bfloat16)

    t0 = time.time()
    w_host = layer_weights(sh, wl.base_seed, 0)
    pk_h, pv_h = prefix_kv(sh, wl.base_seed, 0)
    inp = step_inputs(sh, wl.base_seed, 0, tree=wl.tree, child_law=wl.child_law)
    parent = inp["parent"]
    H_host = bf16_round(inp["H"].astype(np.float32))
    w0 = {k: to_dev(v) for k, v in w_host.items()}
    pk, pv = to_dev(pk_h), to_dev(pv_h)
    H_in = to_dev(H_host.reshape(R, D))
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s: {wl.name}, R={R}, "
          f"weights {sh.weight_bytes_bf16() / 1e6:.1f} MB/layer", file=sys.stderr, flush=True)

    # weight copies for the cold regime: enough of them to overflow the 256 MB cache
    n_copies = max(2, int(np.ceil(600e6 / sh.weight_bytes_bf16())))
    copies = [w0] + [{k: v.clone() for k, v in w0.items()} for _ in range(n_copies - 1)]
    lws = [sf.layer_weights_struct(c) for c in copies]
    pf = sf.prefix_view(pk, pv)
    ws = sf.new_workspace(sh)
    H_out = torch.empty((R, D), dtype=torch.bfloat16, device=dev)
    stats = {"fold": torch.zeros(R, dtype=torch.uint8, device=dev),
             "rec_count": torch.zeros(1, dtype=torch.int32, device=dev)}

    def step(delta, k):
        sf.verify_layer(sh, parent, lws[k % n_copies], pf, None, H_in, delta, H_out, ws, stats=stats)

    # ---------------------------------------------------------------- eager reference + counts
    results = {}
    for delta in (wl.delta, 0.0):
        step(delta, 0)
        torch.cuda.synchronize()
        results[delta] = {"H_out": H_out.clone(), "fold": stats["fold"].cpu().numpy().copy(),
                          "M": int(stats["rec_count"].item())}

    if args.counters > 0:
        # fixed dispatch sequence for rocprofv3 --pmc passes: the counters are read per dispatch,
        # and the plan tells which dispatch is which
        plan = []
        for delta in (wl.delta, 0.0):
            for k in range(args.counters):
                step(delta, 1 + k % (n_copies - 1))
                torch.cuda.synchronize()
            plan.append({"delta": delta, "steps": args.counters, "launches_per_step": len(sf.stage_names()),
                         "M": results[delta]["M"]})
        flat = gate_flat_leg(torch, sf, dev, once=True)
        n = (256 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"counters_plan": plan, "stage_names": sf.stage_names(), "flat": flat,
                          "copy_bytes": 4 * n, "workload": wl.name}), flush=True)
        return

    # ---------------------------------------------------------------- graph-timed throughput
    # exactly K = --steps layer steps per graph replay; consecutive steps read consecutive weight
    # copies (cold: the copies total more than the 256 MB Infinity Cache, so every step streams
    # its weights from HBM; warm: one copy, resident in the cache)
    K = max(1, args.steps)

    def timed(delta, copies_used):
        def check():
            if not torch.equal(H_out.view(torch.int16), results[delta]["H_out"].view(torch.int16)):
                raise RuntimeError("graph replay differs from the eager call")
        fns = [lambda k=k: step(delta, k % copies_used) for k in range(K)]
        ms = time_graph(torch, fns, rounds=args.rounds, warmup_replays=-(-args.warmup // K),
                        warmup_s=args.warmup_seconds, check=check)
        med = float(np.median(ms))
        return {"steps": K, "ms_per_step": med / K, "round_ms_per_step": [round(x / K, 5) for x in ms],
                "branch_tokens_per_s": R * K / (med / 1e3)}

    cold_f, cold_d = timed(wl.delta, n_copies), timed(0.0, n_copies)
    warm_f, warm_d = timed(wl.delta, 1), timed(0.0, 1)
    folded, dense = (warm_f, warm_d) if args.regime == "warm" else (cold_f, cold_d)
    print(f"[bench] cold: folded {cold_f['ms_per_step'] * 1e3:.1f} us/step, dense {cold_d['ms_per_step'] * 1e3:.1f}; "
          f"warm: folded {warm_f['ms_per_step'] * 1e3:.1f}, dense {warm_d['ms_per_step'] * 1e3:.1f}",
          file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- per-launch durations (events)
    def stage_times(delta):
        tm = sf.StageTimer()
        acc = None
        calls = max(1, args.stage_calls)
        skip = min(3, calls - 1)                  # untimed first calls
        for k in range(calls):
            # an untraced call first (the traced call's weight copy is then not the last one
            # read), both queued behind a spin kernel
            hold_queue(torch, 2.0)
            sf.verify_layer(sh, parent, lws[(k + 1) % n_copies], pf, None, H_in, delta, H_out, ws, stats=stats)
            sf.verify_layer(sh, parent, lws[k % n_copies], pf, None, H_in, delta, H_out, ws, stats=stats,
                            trace=tm.trace)
            torch.cuda.synchronize()
            t = tm.elapsed_ms()
            if k >= skip:
                acc = t if acc is None else {n: acc[n] + t[n] for n in acc}
        tm.close()
        cnt = calls - skip
        return {n: 1e3 * v / cnt for n, v in acc.items()}     # microseconds

    st_f = stage_times(wl.delta)
    st_d = stage_times(0.0)
    print("[bench] per-launch us, folded: " + ", ".join(f"{k} {v:.2f}" for k, v in st_f.items()),
          file=sys.stderr, flush=True)

    M = results[wl.delta]["M"]
    fold = results[wl.delta]["fold"].reshape(sh.n_branch, sh.block)
    fold_frac = float(fold[1:].mean()) if sh.n_branch > 1 else 0.0

    # dominant kernel: the FFN gate/up projection (59 % of the layer's weight bytes)
    gu_bytes = 2 * (2 * F * D) + 2 * M * D + 2 * M * F
    gu_us = st_f["gate_up_swiglu_gemm"]
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    roofline = {"kernel": "gate_up_swiglu_gemm", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(), "avg_us": round(gu_us, 2), "bytes_per_launch": gu_bytes,
                "tflops": round(2 * M * 2 * F * D / (gu_us * 1e-6) / 1e12, 1)}

    def regime(f, d_):
        return {"value": round(f["branch_tokens_per_s"], 1), "ms_per_step": round(f["ms_per_step"], 5),
                "round_ms_per_step": f["round_ms_per_step"],
                "dense_value": round(d_["branch_tokens_per_s"], 1), "dense_ms_per_step": round(d_["ms_per_step"], 5),
                "dense_round_ms_per_step": d_["round_ms_per_step"],
                "speedup_vs_dense": round(d_["ms_per_step"] / f["ms_per_step"], 4),
                "layer_roofline_frac": {"folded": round(layer_roof_us(sh, M) / (f["ms_per_step"] * 1e3), 4),
                                        "dense": round(layer_roof_us(sh, R) / (d_["ms_per_step"] * 1e3), 4)}}

    out = {
        "metric": METRIC,
        "value": round(folded["branch_tokens_per_s"], 1),
        "unit": "branch-tokens/s",
        "n_gpus": 1,
        "steps": folded["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(folded["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded random weights, prefix KV and parent-linked draft hidden states)",
        "config": {"workload": wl.name, "hidden": D, "n_q_heads": sh.n_q_heads, "n_kv_heads": sh.n_kv_heads,
                   "head_dim": sh.head_dim, "ffn": F, "block": sh.block, "drafts": sh.n_branch - 1,
                   "prefix": sh.prefix_len, "delta": wl.delta, "rows": R, "regime": args.regime,
                   "weight_copies": n_copies if args.regime == "cold" else 1,
                   "timing": f"HIP graph of exactly {K} steps, median of {args.rounds} event-timed replays",
                   "parallelism": "single GPU"},
        "speedup_vs_dense": round(dense["ms_per_step"] / folded["ms_per_step"], 4),
        "dense": {"value": round(dense["branch_tokens_per_s"], 1), "ms_per_step": round(dense["ms_per_step"], 5),
                  "rec_rows": results[0.0]["M"]},
        "fold_fraction_drafts": round(fold_frac, 4),
        "rec_rows": M,
        "layer_roofline_frac": {"folded": round(layer_roof_us(sh, M) / (folded["ms_per_step"] * 1e3), 4),
                                "dense": round(layer_roof_us(sh, R) / (dense["ms_per_step"] * 1e3), 4)},
        "regimes": {"cold": regime(cold_f, cold_d), "warm": regime(warm_f, warm_d)},
        "roofline": roofline,
        "kernel_frac_of_peak": kernel_pct(sh, st_f, M),
        "kernel_frac_of_peak_dense": kernel_pct(sh, st_d, R),
        "stages_us": {"folded": {k: round(v, 2) for k, v in st_f.items()},
                      "dense": {k: round(v, 2) for k, v in st_d.items()}},
    }

    if not args.no_gate_flat:
        out["gate_flat"] = gate_flat_leg(torch, sf, dev)

    if args.correction:
        out["correction"] = correction_leg(torch, sf, sh, wl, parent, H_in, w0, pk, pv, args)

    if args.serialized:
        out["serialized"] = serialized_leg(torch, sf, sh, lws, pf, H_in, results[0.0]["H_out"], dense, args)

    if args.copy_probe_mb > 0:
        n = args.copy_probe_mb * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        out["copy_probe_bytes"] = 4 * n

    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["verified"] = cpu_baseline_leg(
            sh, wl, parent, H_host, w_host, pk_h, pv_h, results[wl.delta], args.cpu_seconds)
    if emit:
        print(json.dumps(out), flush=True)
    return out


def serialized_leg(torch, sf, sh, lws, pf, H_in, H_dense, dense, args):
    """Serialized verification [SpecFold summary, App. C]: every branch verified alone (one
    branch, parent map [-1], delta 0), as a vanilla verifier would, B+1 layer calls per step.
    Reports its throughput against the batched dense layer (delta 0, same kernels) and how its
    outputs compare with the batched layer's: the K-split decomposition is a function of the
    projection's shape only, so every row should carry the same bits either way (the parity of
    both forms with the oracle is the tests' business)."""
    N = sh.block
    sh1 = sh.with_branches(1)
    ws1 = sf.new_workspace(sh1)
    y = torch.empty_like(H_dense)
    par1 = [-1]
    n_copies = len(lws)

    def run_all(k):
        for i in range(sh.n_branch):
            sf.verify_layer(sh1, par1, lws[k], pf, None, H_in[i * N:(i + 1) * N], 0.0, y[i * N:(i + 1) * N], ws1)

    run_all(0)
    torch.cuda.synchronize()
    same = (y.view(torch.int16) == H_dense.view(torch.int16)).all(dim=1)
    diff = (y.float() - H_dense.float()).abs()
    reps = max(1, args.steps // (4 * n_copies))
    ms = graph_time(torch, [lambda k=k: run_all(k) for k in range(n_copies)], reps=reps) / n_copies
    R = sh.rows
    return {"ms_per_step": round(ms, 5), "branch_tokens_per_s": round(R / (ms * 1e-3), 1),
            "batched_dense_speedup": round(ms / dense["ms_per_step"], 4),
            "rows_bitwise_equal_to_batched": round(float(same.float().mean().item()), 4),
            "max_abs_diff_vs_batched": round(float(diff.max().item()), 6),
            "finite": bool(torch.isfinite(y.float()).all().item()),
            "note": "each of the B+1 branches alone (n_branch 1, delta 0), graph-replayed"}


def correction_leg(torch, sf, sh, wl, parent, H_in, w, pk, pv, args):
    """The pages' attention-state correction [SpecFold summary, App. B, §A.1, §A.3] against the
    library's prefix-partial + block merge, on the same folded layer's projections (the
    library's gate, compaction, source resolution and QKV).  The variant (variants/, not part
    of the library) computes fresh fp32 states for the recompute rows, corrects the folded
    rows one tree level at a time, and divides; the library computes every row's attention
    in two launches.  Both are compared with direct attention evaluated in float64 by torch
    on the device from the same bf16 projections."""
    from variants import correction as corr

    dev = H_in.device
    R, Hq, Hkv, d, N = sh.rows, sh.n_q_heads, sh.n_kv_heads, sh.head_dim, sh.block
    I32 = torch.int32
    rho = torch.empty(R, device=dev)
    fold = torch.empty(R, dtype=torch.uint8, device=dev)
    inv = torch.empty(R, device=dev)
    rec = torch.zeros(R, dtype=I32, device=dev)
    cnt = torch.zeros(4, dtype=I32, device=dev)
    off = torch.zeros(sh.n_branch + 1, dtype=I32, device=dev)
    slot = torch.zeros(R, dtype=I32, device=dev)
    src_b = torch.zeros(R, dtype=I32, device=dev)
    src = torch.zeros(R, dtype=I32, device=dev)
    q = torch.zeros((R, Hq, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((R, Hkv, d), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    ws = sf.new_workspace(sh)
    sf.gate(sh, parent, H_in, wl.delta, rho, fold, inv_rms=inv)
    sf.compact(sh, fold, rec, cnt[:1], off, slot)
    sf.resolve_sources(sh, parent, fold, slot, src_b, src)
    sf.sparse_qkv(sh, H_in, inv, rec, cnt[:1], w["ln1"], w["w_qkv"], q, k, v, ws)
    attn = torch.empty((R, Hq * d), dtype=torch.bfloat16, device=dev)
    state = torch.empty(corr.state_shape(sh), device=dev)
    out = torch.empty((R, Hq, d), device=dev)
    levels = corr.levels(sh, parent)

    def lib():
        sf.folded_attention(sh, q, k, v, rec, cnt[:1], src, pk, pv, attn, ws)

    def fresh():
        corr.fresh(sh, q, k, v, rec, cnt[:1], src, pk, pv, state)

    def variant():
        corr.attention(sh, parent, q, k, v, rec, cnt[:1], src, fold, pk, pv, state, out)

    lib()
    variant()
    torch.cuda.synchronize()
    # every phase reads only inputs it does not write, so a graph of REP back-to-back copies
    # times one copy without the graph launch in the figure
    REP = 16
    reps = max(10, args.steps // REP)

    def per_call(fn):
        return graph_time(torch, [fn] * REP, reps) / REP

    t = {"library_merge": per_call(lib), "variant_total": per_call(variant), "variant_fresh": per_call(fresh)}
    variant()                                       # the states every level reads are the final ones
    t_levels = [per_call(lambda m=m: corr.level(sh, parent, m, q, k, v, src, fold, state)) for m in levels]
    t["variant_finalize"] = per_call(lambda: corr.finalize(sh, state, out))
    variant()
    torch.cuda.synchronize()

    # direct attention in float64 from the same projections (rows gathered by source slot)
    sl = src.long()
    Q = q.double()[sl].view(sh.n_branch, N, Hq, d)
    K = k.double()[sl].view(sh.n_branch, N, Hkv, d)
    V = v.double()[sl].view(sh.n_branch, N, Hkv, d)
    G = Hq // Hkv
    ref = torch.empty((sh.n_branch, N, Hq, d), dtype=torch.float64, device=dev)
    for g in range(Hkv):
        keys = torch.cat([pk.double()[:, g].unsqueeze(0).expand(sh.n_branch, -1, -1), K[:, :, g]], dim=1)
        vals = torch.cat([pv.double()[:, g].unsqueeze(0).expand(sh.n_branch, -1, -1), V[:, :, g]], dim=1)
        for h in range(g * G, (g + 1) * G):
            s = torch.matmul(Q[:, :, h], keys.transpose(1, 2).contiguous()) / (d ** 0.5)
            ref[:, :, h] = torch.matmul(torch.softmax(s, dim=-1), vals)
    ref = ref.view(R, Hq, d)

    def err(x):
        x = x.double().view(R, Hq, d)
        return {"rel_l2": float(((x - ref).norm() / ref.norm()).item()),
                "max_abs": float((x - ref).abs().max().item())}

    M = int(cnt[0].item())
    return {"levels": len(levels), "rec_rows": M,
            "folded_rows": int(fold.sum().item()),
            "us": {k_: round(1e3 * v_, 2) for k_, v_ in t.items()},
            "variant_level_us": [round(1e3 * v_, 2) for v_ in t_levels],
            "numerics_vs_f64_direct": {"library_merge_bf16_out": err(attn.float()),
                                       "variant_fp32_out": err(out)},
            "note": "same projections for both; library output is bf16, the variant's fp32"}


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "gate_up_swiglu_gemm_layer-1.5b_traffic.md")


def measured_traffic(record=None):
    """HBM bytes per launch of the gate/up GEMM from a committed counter record (FETCH_SIZE +
    WRITE_SIZE, calibrated by a copy of known size), or None when the record is missing or was
    taken for a different version of the GEMM sources."""
    import hashlib
    try:
        text = open(record or TRAFFIC_RECORD).read()
        rec = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    h = hashlib.sha256()
    for f in ("gemm.hip", "kernels.h", "common.h"):
        with open(os.path.join(ROOT, "sparse_layer_rho_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return rec.get("traffic_bytes") if rec.get("source_sha256") == h.hexdigest() else None


_SPIN = {}


def hold_queue(torch, ms):
    """Put a spin kernel of about ``ms`` milliseconds on the current stream: the launches the
    host queues behind it meanwhile run back to back when it ends, so per-launch event timing
    measures the GPU and not the host's enqueue rate (an eager call that outruns the host would
    otherwise count the host's gaps into the next launch), and the first traced launch follows
    queued work as every launch of a stack does (not a launch onto an idle GPU)."""
    if "cycles_per_ms" not in _SPIN:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(2_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SPIN["cycles_per_ms"] = 2_000_000 / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(ms * _SPIN["cycles_per_ms"]))


def time_graph(torch, fns, rounds=5, warmup_replays=1, warmup_s=0.5, check=None, reps=1):
    """Capture fns (callables launching on the current stream) in one HIP graph, replay it untimed
    for at least `warmup_replays` replays and `warmup_s` seconds, then time `rounds` rounds of
    `reps` replays, each round between its own pair of events.  Returns ms per replay of every
    round.  check() runs after the warm-up and after the timed rounds."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for f in fns:
            f()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    t0, done = time.perf_counter(), 0
    while done < warmup_replays or time.perf_counter() - t0 < warmup_s:
        g.replay()
        done += 1
        if done % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    if check:
        check()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(rounds)]
    for e0, e1 in ev:
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
    torch.cuda.synchronize()
    if check:
        check()
    del g
    return [e0.elapsed_time(e1) / reps for e0, e1 in ev]


def graph_time(torch, fns, reps, warmup_s=0.5):
    """ms per replay of a graph of fns: the median of 5 rounds of `reps` replays."""
    import statistics
    return statistics.median(time_graph(torch, fns, rounds=5, warmup_s=warmup_s, reps=max(1, reps)))


def gate_flat_leg(torch, sf, dev, once=False):
    """Gate and compaction alone on a large flattened input, as bandwidth evidence: 9 branches of
    16384 positions at D = 1536 (453 MB of H) for the gate; 64 x 262144 rows for the compaction.
    once: one eager call of each, untimed (counter runs); returns their sizes."""
    from synth import Shape
    sh = Shape(9, 16384, 1536, 12, 2, 128, 8960, 0)
    R, D = sh.rows, sh.hidden
    parent = [-1, 0, 0, 1, 1, 2, 3, 4, 5]
    H = torch.randn((R, D), device=dev).to(torch.bfloat16)
    rho = torch.empty(R, device=dev)
    fold = torch.empty(R, dtype=torch.uint8, device=dev)
    if once:
        sf.gate(sh, parent, H, 0.1, rho, fold)
        torch.cuda.synchronize()
    # 8 back-to-back calls per graph replay, so the replay's own launch is not in the figure
    ms = 0.0 if once else graph_time(torch, [lambda: sf.gate(sh, parent, H, 0.1, rho, fold)] * 8, reps=10) / 8
    # algorithmic bytes: every row of H read once (a parent row serves all its children), rho and
    # fold written
    gbytes = R * D * 2 + R * 5
    del H
    sc = Shape(64, 262144, 64, 4, 2, 16, 128, 0)
    Rc = sc.rows
    fold_c = (torch.rand(Rc, device=dev) < 0.7).to(torch.uint8)
    rec_rows = torch.empty(Rc, dtype=torch.int32, device=dev)
    rec_count = torch.empty(1, dtype=torch.int32, device=dev)
    branch_off = torch.empty(sc.n_branch + 1, dtype=torch.int32, device=dev)
    row_slot = torch.empty(Rc, dtype=torch.int32, device=dev)
    cws = sf.compact_workspace(sc, dev)
    if once:
        sf.compact(sc, fold_c, rec_rows, rec_count, branch_off, row_slot, ws=cws)
        torch.cuda.synchronize()
        return {"gate": {"rows": R, "hidden": D, "bytes": R * D * 2 + R * 5},
                "compact": {"rows": Rc, "M": int(rec_count.item()),
                            "bytes": Rc + 4 * Rc + 4 * int(rec_count.item()) + 4 * (sc.n_branch + 1)}}
    ms_c = graph_time(torch, [lambda: sf.compact(sc, fold_c, rec_rows, rec_count, branch_off, row_slot, ws=cws)] * 8,
                      reps=10) / 8
    M = int(rec_count.item())
    # algorithmic bytes: the flags read once; the row map, list and offsets written
    cbytes = Rc + 4 * Rc + 4 * M + 4 * (sc.n_branch + 1)
    return {"gate": {"rows": R, "hidden": D, "us": round(ms * 1e3, 2), "bytes": gbytes,
                     "gbs": round(gbytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(gbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
            "compact": {"rows": Rc, "us": round(ms_c * 1e3, 2), "bytes": cbytes,
                        "gbs": round(cbytes / (ms_c * 1e-3) / 1e9, 1),
                        "hbm_frac": round(cbytes / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}


def stack_measure(torch, sf, wl, layers, steps, args, dev, with_head=False, keep=False):
    """Verification passes through an L-layer stack: per-branch residual streams carried across
    layers, every layer re-gating on its own input.  S input steps (a new draft tree and new
    hidden states each); one graph holds exactly K = --steps passes, pass k on input k % S; the
    median of --rounds timed replays is reported, after at least --warmup untimed passes.
    keep: also return the device objects (for the per-launch timing and the CPU baseline)."""
    import numpy as np

    from synth import bf16_round, device_layer, step_inputs

    sh = wl.shape
    R, D = sh.rows, sh.hidden
    L = layers if layers > 1 else wl.layers
    S = steps if steps > 0 else max(1, wl.steps)
    K = max(1, args.steps)
    t0 = time.time()
    # every layer's weights and prefix cache drawn on the device (synth.device_layer)
    layer_list = [device_layer(torch, sh, 1000 * wl.base_seed + l, dev, wl.weight_std) for l in range(L)]
    lws = [sf.layer_weights_struct(w) for w, _, _ in layer_list]
    pfs = [sf.prefix_view(pk, pv) for _, pk, pv in layer_list]
    steps_in = []
    for s in range(S):
        inp = step_inputs(sh, wl.base_seed, s, tree=wl.tree, child_law=wl.child_law)
        Hs = bf16_round(inp["H"].astype(np.float32))
        steps_in.append((inp["parent"], torch.from_numpy(Hs.reshape(R, D)).to(dev).to(torch.bfloat16)))
    torch.cuda.synchronize()
    print(f"[bench] stack ready in {time.time() - t0:.1f}s: {wl.name}, {L} layers, {S} input steps, "
          f"{L * sh.weight_bytes_bf16() / 1e9:.2f} GB of weights", file=sys.stderr, flush=True)

    ws = sf.new_workspace(sh)
    buf = [torch.empty((R, D), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    # per-layer statistics; rows padded to 16 bytes (the library takes 16-byte aligned pointers)
    Rp = (R + 15) // 16 * 16
    fold = torch.zeros((L, Rp), dtype=torch.uint8, device=dev)
    cnt = torch.zeros((L, 4), dtype=torch.int32, device=dev)

    def run_step(s, delta, stats=True, traces=None):
        parent, H0 = steps_in[s]
        x = H0
        for l in range(L):
            y = buf[l % 2]
            sf.verify_layer(sh, parent, lws[l], pfs[l], None, x, delta, y, ws,
                            stats={"fold": fold[l, :R], "rec_count": cnt[l, :1]} if stats else None,
                            trace=traces[l].trace if traces else None)
            x = y
        return x

    res = {}
    for delta in (wl.delta, 0.0):
        Ms, ff, outs = [], [], []
        for s in range(S):
            x = run_step(s, delta)
            torch.cuda.synchronize()
            outs.append(x.clone())
            Ms.append(cnt[:, 0].cpu().numpy().copy())
            ff.append(fold[:, :R].cpu().numpy().reshape(L, sh.n_branch, sh.block)[:, 1:].mean(axis=(1, 2)))
        last = outs[(K - 1) % S]

        def check(last=last, delta=delta):
            if not torch.equal(buf[(L - 1) % 2].view(torch.int16), last.view(torch.int16)):
                raise RuntimeError(f"stack graph replay differs from the eager pass (delta {delta})")
        ms = time_graph(torch, [lambda k=k, delta=delta: run_step(k % S, delta) for k in range(K)],
                        rounds=args.rounds, warmup_replays=-(-args.warmup // K), warmup_s=args.warmup_seconds,
                        check=check)
        med = float(np.median(ms))
        res[delta] = {"ms_per_step": med / K, "round_ms_per_step": [round(x / K, 5) for x in ms],
                      "M": np.mean(Ms, axis=0), "fold": np.mean(ff, axis=0),
                      "finite": all(bool(torch.isfinite(o.float()).all().item()) for o in outs)}
        print(f"[bench] stack delta {delta}: {med / K:.3f} ms per step", file=sys.stderr, flush=True)

    f, d = res[wl.delta], res[0.0]
    out = {
        "workload": wl.name, "layers": L, "steps": K, "input_steps": S,
        "value": round(R / (f["ms_per_step"] * 1e-3), 1), "unit": "branch-tokens/s",
        "ms_per_step": round(f["ms_per_step"], 5), "round_ms_per_step": f["round_ms_per_step"],
        "dense_value": round(R / (d["ms_per_step"] * 1e-3), 1), "dense_ms_per_step": round(d["ms_per_step"], 5),
        "dense_round_ms_per_step": d["round_ms_per_step"],
        "speedup_vs_dense": round(d["ms_per_step"] / f["ms_per_step"], 4),
        "us_per_layer": {"folded": round(1e3 * f["ms_per_step"] / L, 2), "dense": round(1e3 * d["ms_per_step"] / L, 2)},
        "rec_rows_mean": round(float(np.mean(f["M"])), 1),
        "rec_rows_per_layer": [round(float(v), 1) for v in f["M"]],
        "fold_fraction_drafts": round(float(np.mean(f["fold"])), 4),
        "fold_fraction_drafts_per_layer": [round(float(v), 4) for v in f["fold"]],
        "finite_output": bool(f["finite"] and d["finite"]),
        "config": {"hidden": D, "n_q_heads": sh.n_q_heads, "n_kv_heads": sh.n_kv_heads, "head_dim": sh.head_dim,
                   "ffn": sh.ffn, "block": sh.block, "drafts": sh.n_branch - 1, "prefix": sh.prefix_len,
                   "delta": wl.delta, "rows": R, "layers": L, "input_steps": S, "weight_std": list(wl.weight_std),
                   "regime": f"cold by size ({L * sh.weight_bytes_bf16() / 1e9:.2f} GB of weights per pass)",
                   "timing": f"HIP graph of exactly {K} passes through the {L} layers (input step k % {S}), "
                             f"median of {args.rounds} event-timed replays"},
    }
    if with_head:
        out["pass_with_head"] = pass_leg(torch, sf, sh, wl, args, [(p, None, H) for p, H in steps_in], lws, pfs, ws,
                                         buf, fold, cnt, L, S, dev)
    if not keep:
        return out
    ctx = {"sh": sh, "L": L, "S": S, "layer_list": layer_list, "lws": lws, "pfs": pfs, "steps_in": steps_in,
           "ws": ws, "buf": buf, "fold": fold, "cnt": cnt, "run_step": run_step, "M": {wl.delta: f["M"], 0.0: d["M"]}}
    return out, ctx


def stack_stage_times(torch, sf, ctx, delta, n_steps=0):
    """Event-timed duration of every launch of every layer over n_steps eager passes (default:
    one per input step, the mix the timed graphs run), each traced pass queued behind a spin
    kernel (hold_queue), so its launches run back to back as in the replayed graphs.  Returns
    per-layer stage dicts (microseconds, mean over the passes) and per-layer M."""
    import numpy as np

    L, S = ctx["L"], ctx["S"]
    timers = [sf.StageTimer() for _ in range(L)]
    acc = [None] * L
    Ms = []
    n = min(n_steps, S) if n_steps > 0 else S
    for s in range(n):
        hold_queue(torch, 20.0)
        ctx["run_step"](s, delta, stats=True, traces=timers)
        torch.cuda.synchronize()
        Ms.append(ctx["cnt"][:, 0].cpu().numpy().copy())
        for l in range(L):
            t = timers[l].elapsed_ms()
            acc[l] = t if acc[l] is None else {k: acc[l][k] + t[k] for k in t}
    for tm in timers:
        tm.close()
    per_layer = [{k: 1e3 * v / n for k, v in a.items()} for a in acc]
    return per_layer, np.mean(Ms, axis=0)


def stack_bench(args, wl):
    """Stack workloads (the default, stack-1.5b, and stack-7b): the line's throughput is the
    stack's; the dominant kernel's roofline and the per-launch fractions come from event timing of
    every launch of every layer; stack-1.5b also carries the single layer (layer-1.5b) as a
    sub-object, the flat gate and compaction, and the CPU oracle on sampled layers."""
    import copy

    import numpy as np
    import torch

    from sparse_layer_rho_amd import specfold as sf
    from synth import WORKLOADS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.counters > 0:
        return stack_counters(torch, sf, wl, args, dev)
    st, ctx = stack_measure(torch, sf, wl, args.layers, args.stack_steps, args, dev, with_head=args.with_head,
                            keep=True)
    sh, L = ctx["sh"], ctx["L"]
    D, F = sh.hidden, sh.ffn
    per_f, M_f = stack_stage_times(torch, sf, ctx, wl.delta)
    per_d, M_d = stack_stage_times(torch, sf, ctx, 0.0)
    mean_stage = lambda per: {k: float(np.mean([p[k] for p in per])) for k in per[0]}
    st_f, st_d = mean_stage(per_f), mean_stage(per_d)
    print("[bench] stack per-launch us (mean over layers), folded: " +
          ", ".join(f"{k} {v:.2f}" for k, v in st_f.items()), file=sys.stderr, flush=True)

    # dominant kernel: the FFN gate/up projection, every launch of the traced passes
    gu_bytes = [2 * (2 * F * D) + 2 * m * D + 2 * m * F for m in M_f]
    gu_us = [p["gate_up_swiglu_gemm"] for p in per_f]
    achieved = float(np.sum(gu_bytes)) / (float(np.sum(gu_us)) * 1e-6) / 1e9
    roofline = {"kernel": "gate_up_swiglu_gemm", "bound": "hbm", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(stack_traffic_record(wl.name)),
                "avg_us": round(float(np.mean(gu_us)), 2), "bytes_per_launch": round(float(np.mean(gu_bytes))),
                "launches": f"{L} layers x {ctx['S']} passes (one per input step), event-timed on the launch stream",
                "tflops": round(2 * float(np.mean(M_f)) * 2 * F * D / (float(np.mean(gu_us)) * 1e-6) / 1e12, 1)}
    Mm_f, Mm_d = float(np.mean(M_f)), float(np.mean(M_d))
    roof_f = sum(layer_roof_us(sh, m) for m in M_f)
    roof_d = sum(layer_roof_us(sh, m) for m in M_d)
    out = {
        "metric": METRIC, "value": st["value"], "unit": "branch-tokens/s", "n_gpus": 1, "steps": st["steps"],
        "warmup": args.warmup, "ms_per_step": st["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random weights and prefix KV per layer, parent-linked draft hidden states per step)",
        "config": {"workload": wl.name, **st["config"], "parallelism": "single GPU"},
        "speedup_vs_dense": st["speedup_vs_dense"],
        "dense": {"value": st["dense_value"], "ms_per_step": st["dense_ms_per_step"]},
        "fold_fraction_drafts": st["fold_fraction_drafts"], "rec_rows_mean": st["rec_rows_mean"],
        "layer_roofline_frac": {"folded": round(roof_f / (st["ms_per_step"] * 1e3), 4),
                                "dense": round(roof_d / (st["dense_ms_per_step"] * 1e3), 4)},
        "roofline": roofline,
        "kernel_frac_of_peak": kernel_pct(sh, st_f, Mm_f),
        "kernel_frac_of_peak_dense": kernel_pct(sh, st_d, Mm_d),
        "stages_us_mean_over_layers": {"folded": {k: round(v, 2) for k, v in st_f.items()},
                                       "dense": {k: round(v, 2) for k, v in st_d.items()}},
        "stack": st,
    }
    if wl.name == "stack-1.5b" and not args.no_layer:
        a = copy.copy(args)
        a.no_cpu_baseline, a.no_gate_flat, a.steps = True, True, 200
        out["layer"] = layer_main(a, WORKLOADS["layer-1.5b"], emit=False)
    if not args.no_gate_flat and wl.name == "stack-1.5b":
        out["gate_flat"] = gate_flat_leg(torch, sf, dev)
    if wl.name == "stack-1.5b":
        pk = measured_peaks(torch, dev)
        out["measured_peaks"] = pk
        out["roofline"]["frac_of_measured_copy_rate"] = round(roofline["achieved"] / pk["hbm_copy_gbs"], 4)
    if not args.no_cpu_baseline:
        out["cpu_baseline"], out["verified"] = stack_cpu_baseline(torch, sf, ctx, wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def measured_peaks(torch, dev):
    """Achievable rates on this machine from library kernels, as context for the vendor peaks: a
    1 GiB device copy (HBM read + write), copies within a 128 MiB working set (last-level
    cache) and a 8192^3 bf16 matrix product (hipBLASLt); each the best of 5 event-timed runs
    after a warm-up.  (torch's reductions read more slowly than the
    library's own gate kernel does, so they are no read-bandwidth reference.)"""
    def best(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)
    n = (1 << 30) // 4
    x = torch.empty(n, dtype=torch.float32, device=dev).uniform_()
    y = torch.empty_like(x)
    t_copy = best(lambda: y.copy_(x))
    del x, y
    # the same with a 128 MiB working set (two 64 MiB buffers), copied 8 times back to back:
    # after the first copy both stay in the 256 MB last-level cache (MALL)
    n2 = (64 << 20) // 4
    x2 = torch.empty(n2, dtype=torch.float32, device=dev).uniform_()
    y2 = torch.empty_like(x2)

    def copies():
        for _ in range(8):
            y2.copy_(x2)
    t_mall = best(copies) / 8
    del x2, y2
    m = 8192
    a_ = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    b_ = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    t_mm = best(lambda: torch.matmul(a_, b_))
    del a_, b_
    return {"hbm_copy_gbs": round(2 * (1 << 30) / t_copy / 1e9, 1),
            "mall_copy_gbs": round(2 * (64 << 20) / t_mall / 1e9, 1),
            "bf16_matmul_tflops": round(2 * m ** 3 / t_mm / 1e12, 1),
            "how": "best of 5 event-timed runs: torch 1 GiB device copy (bytes read + written); "
                   "the mean of 8 back-to-back 64 MiB copies between two cache-resident buffers; "
                   "torch.matmul 8192^3 bf16 (hipBLASLt)"}


def stack_traffic_record(name):
    return os.path.join(ROOT, "profiles", f"gate_up_swiglu_gemm_{name}_traffic.md")


def stack_counters(torch, sf, wl, args, dev):
    """Counter runs of a stack: N folded then N dense passes through its layers (one per input
    step), then a 256 MiB device copy for calibration; prints the dispatch plan (no timing)."""
    a = argparse.Namespace(**vars(args))
    a.steps, a.rounds, a.warmup, a.warmup_seconds = 1, 1, 0, 0.0
    n = args.counters
    # stack_measure's eager passes and one-replay timing come first; the plan starts after them
    st, ctx = stack_measure(torch, sf, wl, args.layers, n, a, dev, keep=True)
    torch.cuda.synchronize()
    plan = []
    for delta in (wl.delta, 0.0):
        for s in range(n):
            ctx["run_step"](s, delta)
            torch.cuda.synchronize()
        plan.append({"delta": delta, "passes": n, "layers": ctx["L"], "launches_per_layer": len(sf.stage_names()),
                     "M_per_layer": [round(float(v), 1) for v in ctx["M"][delta]]})
    nb = (256 << 20) // 4
    x = torch.empty(nb, dtype=torch.float32, device=dev).uniform_()
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"counters_plan": plan, "stage_names": sf.stage_names(), "copy_bytes": 4 * nb,
                      "workload": wl.name}), flush=True)


def stack_cpu_baseline(torch, sf, ctx, wl, seconds):
    """The CPU oracle on a bounded sample of the stack: the first, middle and last layers of the
    first input step, each teacher-forced on the GPU's own input of that layer and checked
    against the GPU's output (mask exact outside |rho - delta| < 1e-4, relative L2 <= 2e-2).
    The stack rate is the sampled layers' mean time times the layer count.  Timings are the
    median of up to 3 passes after one warm-up: with the BLAS threads the host gives this
    process, with one thread (first sampled layer), and the dense pass (delta 0)."""
    import contextlib
    import platform
    import statistics

    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle

    sh, L = ctx["sh"], ctx["L"]
    R, D = sh.rows, sh.hidden
    sample = sorted({0, L // 2, L - 1})
    parent, H0 = ctx["steps_in"][0]
    host = lambda t: t.float().cpu().numpy().astype(np.float64)
    # the GPU's input and output of every sampled layer (one eager folded pass)
    ins, outs, folds = {}, {}, {}
    x = H0
    for l in range(L):
        y = ctx["buf"][l % 2]
        st = {"fold": ctx["fold"][l, :R], "rec_count": ctx["cnt"][l, :1]}
        if l in sample:
            ins[l] = host(x).reshape(sh.n_branch, sh.block, D)
        sf.verify_layer(sh, parent, ctx["lws"][l], ctx["pfs"][l], None, x, wl.delta, y, ctx["ws"], stats=st)
        torch.cuda.synchronize()
        if l in sample:
            outs[l] = host(y).reshape(sh.n_branch, sh.block, D)
            folds[l] = ctx["fold"][l, :R].cpu().numpy().reshape(sh.n_branch, sh.block).astype(bool)
        x = y
    checks, ok = [], True
    wsd = {}
    for l in sample:
        w, pk, pv = ctx["layer_list"][l]
        wsd[l] = ({k: host(v) for k, v in w.items()}, host(pk), host(pv))
        wh, pkh, pvh = wsd[l]
        rho_o, fold_o = oracle.gate(ins[l], parent, wl.delta)
        band = np.abs(rho_o - wl.delta) < 1e-4
        mask_ok = bool(np.array_equal(folds[l][~band], fold_o[~band]))
        ref = oracle.verify_layer(ins[l], parent, wh, pkh, pvh, wl.delta, sh, fold=folds[l])
        err = float(np.linalg.norm(outs[l] - ref["H_out"]) / np.linalg.norm(ref["H_out"]))
        checks.append({"layer": l, "rel_l2": round(err, 6), "mask_match_outside_band": mask_ok})
        ok = ok and mask_ok and err <= 2e-2

    def timed(delta, limit, layers):
        ctx_ = threadpool_limits(limits=limit) if limit else contextlib.nullcontext()
        per = []
        with ctx_:
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
            for l in layers:
                wh, pkh, pvh = wsd[l]
                t0 = time.perf_counter()
                oracle.verify_layer(ins[l], parent, wh, pkh, pvh, delta, sh)       # warm-up
                first = time.perf_counter() - t0
                n = 3 if 3 * first * len(layers) <= seconds else 1
                ts = []
                for _ in range(n):
                    t0 = time.perf_counter()
                    oracle.verify_layer(ins[l], parent, wh, pkh, pvh, delta, sh)
                    ts.append(time.perf_counter() - t0)
                per.append(statistics.median(ts))
        return float(np.mean(per)), threads

    t_all, threads = timed(wl.delta, None, sample)
    t_one, _ = timed(wl.delta, 1, sample[:1])
    t_dense, _ = timed(0.0, None, sample)
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = sorted({f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info()
                   if p.get("user_api") == "blas"})
    cpu = {"value": round(R / (t_all * L), 1), "unit": "branch-tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"float64 oracle on layers {sample} of the first input step ({R} rows, delta {wl.delta}), "
                     f"teacher-forced on the GPU's layer inputs, {threads} BLAS threads; the stack rate is their "
                     f"mean time per layer ({t_all:.3f} s) times {L} layers",
           "seconds_per_layer": round(t_all, 4),
           "one_thread": {"value": round(R / (t_one * L), 1), "seconds_per_layer": round(t_one, 4),
                          "layers": sample[:1]},
           "dense_delta0": {"value": round(R / (t_dense * L), 1), "seconds_per_layer": round(t_dense, 4),
                            "speedup_of_folding": round(t_dense / t_all, 4)},
           "cpu_model": model, "host_cpus_available": len(os.sched_getaffinity(0)), "blas": blas}
    return cpu, {"ok": bool(ok), "layers": checks}


def pass_leg(torch, sf, sh, wl, args, steps, lws, pfs, ws, buf, fold, cnt, L, S, dev):
    """Whole verification passes from token ids [SpecFold summary, App. B]: embedding gather,
    the L-layer stack (folded at the workload's delta, or dense), final RMSNorm + LM head +
    greedy token of every row.  The drafts' tokens copy their parent's block with 1-4 newly
    unmasked positions, so the first layer's gate sees identical rows wherever a draft agrees
    with its parent.  The head's parity with the oracle is checked by the tests; here every
    greedy token must name a vocabulary entry and every best logit be finite."""
    import numpy as np

    from synth import step_tokens

    R, D, V = sh.rows, sh.hidden, args.vocab
    g = torch.Generator(device=dev)
    g.manual_seed(7919 * wl.base_seed + 17)
    E = torch.randn(V, D, device=dev, generator=g).to(torch.bfloat16)
    W_lm = (0.02 * torch.randn(V, D, device=dev, generator=g)).to(torch.bfloat16)
    ln_f = torch.ones(D, dtype=torch.bfloat16, device=dev)
    toks = [torch.from_numpy(step_tokens(sh, V, wl.base_seed, s, steps[s][0]).reshape(R)).to(dev) for s in range(S)]
    hws = sf.head_workspace(sh, V)
    H0 = torch.empty((R, D), dtype=torch.bfloat16, device=dev)
    tok_out = torch.empty(R, dtype=torch.int32, device=dev)
    logit_out = torch.empty(R, dtype=torch.float32, device=dev)

    def run_pass(s, delta, stats=False):
        sf.embed(sh, toks[s], E, H0)
        x = H0
        for l in range(L):
            y = buf[l % 2]
            sf.verify_layer(sh, steps[s][0], lws[l], pfs[l], None, x, delta, y, ws,
                            stats={"fold": fold[l, :R], "rec_count": cnt[l, :1]} if stats else None)
            x = y
        sf.lm_head(sh, x, ln_f, W_lm, tok_out, logit_out, hws)
        return x

    res = {}
    for delta in (wl.delta, 0.0):
        ff = []
        for s in range(S):
            run_pass(s, delta, stats=True)
            torch.cuda.synchronize()
            ff.append(fold[:, :R].cpu().numpy().reshape(L, sh.n_branch, sh.block)[:, 1:].mean(axis=(1, 2)))
        reps = max(1, args.steps // (S * 4))
        ms = graph_time(torch, [lambda s=s: run_pass(s, delta) for s in range(S)], reps=reps) / S
        res[delta] = (ms, np.mean(ff, axis=0))
        print(f"[bench] pass with head, delta {delta}: {ms:.3f} ms", file=sys.stderr, flush=True)
    reps = max(1, args.steps)
    embed_ms = graph_time(torch, [lambda: sf.embed(sh, toks[0], E, H0)], reps=reps)
    head_ms = graph_time(torch, [lambda: sf.lm_head(sh, buf[0], ln_f, W_lm, tok_out, logit_out, hws)], reps=reps)
    run_pass(0, wl.delta)
    torch.cuda.synchronize()
    tg = tok_out.cpu().numpy()
    ok = bool(((tg >= 0) & (tg < V)).all() and torch.isfinite(logit_out).all().item())
    (fms, ffold), (dms, _) = res[wl.delta], res[0.0]
    head_bytes = 2 * V * D + 2 * R * D
    return {"vocab": V, "ms_per_pass": round(fms, 5), "dense_ms_per_pass": round(dms, 5),
            "speedup_vs_dense": round(dms / fms, 4), "branch_tokens_per_s": round(R / (fms * 1e-3), 1),
            "embed_us": round(1e3 * embed_ms, 2), "lm_head_us": round(1e3 * head_ms, 2),
            "lm_head_hbm_frac": round(head_bytes / (head_ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
            "fold_fraction_drafts_per_layer": [round(float(v), 4) for v in ffold],
            "tokens_in_vocab_and_logits_finite": ok,
            "data": "token ids: main uniform, drafts copy the parent's block with 1-4 new tokens; "
                    "E ~ N(0,1), W_lm ~ N(0, 0.02^2), final norm weight 1 (seeded, on the device)"}


def sweep_bench(args, wl):
    """One layer swept over draft count B and delta (one tree and one set of hidden states per B,
    reused across delta, so the folded fraction is monotone in delta).  The tests check the
    layer's parity with the oracle at points of this sweep."""
    import numpy as np
    import torch

    from sparse_layer_rho_amd import specfold as sf
    from synth import bf16_round, layer_weights, prefix_kv, step_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    base = wl.shape

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(torch.bfloat16)

    t0 = time.time()
    w_host = layer_weights(base, wl.base_seed, 0)
    pk_h, pv_h = prefix_kv(base, wl.base_seed, 0)
    w0 = {k: to_dev(v) for k, v in w_host.items()}
    n_copies = max(2, int(np.ceil(600e6 / base.weight_bytes_bf16())))
    # the copies must outlive every launch that reads them: the structs hold raw pointers, and
    # graph capture empties the allocator's cache, returning freed blocks to the runtime
    copies = [w0] + [{k: v.clone() for k, v in w0.items()} for _ in range(n_copies - 1)]
    lws = [sf.layer_weights_struct(c) for c in copies]
    pk, pv = to_dev(pk_h), to_dev(pv_h)
    pf = sf.prefix_view(pk, pv)
    print(f"[bench] sweep ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    points = []
    for B in wl.branch_sweep:
        sh = base.with_branches(B + 1)
        R, D = sh.rows, sh.hidden
        inp = step_inputs(sh, wl.base_seed, 0, tree=wl.tree, child_law=wl.child_law)
        parent, H_host = inp["parent"], bf16_round(inp["H"].astype(np.float32))
        H = to_dev(H_host.reshape(R, D))
        ws = sf.new_workspace(sh)
        y = torch.empty((R, D), dtype=torch.bfloat16, device=dev)
        st = {"fold": torch.zeros(R, dtype=torch.uint8, device=dev), "rec_count": torch.zeros(1, dtype=torch.int32, device=dev)}
        per = {}
        for delta in wl.delta_sweep:
            sf.verify_layer(sh, parent, lws[0], pf, None, H, delta, y, ws, stats=st)
            torch.cuda.synchronize()
            M = int(st["rec_count"].item())
            ff = float(st["fold"].cpu().numpy().reshape(sh.n_branch, sh.block)[1:].mean())
            reps = max(1, args.steps // (4 * n_copies))
            ms = graph_time(torch, [lambda k=k, delta=delta: sf.verify_layer(sh, parent, lws[k], pf, None, H, delta, y, ws)
                                    for k in range(n_copies)], reps=reps) / n_copies
            per[delta] = (ms, M, ff)
        sf.verify_layer(sh, parent, lws[0], pf, None, H, wl.delta, y, ws, stats=st)
        torch.cuda.synchronize()
        finite = bool(torch.isfinite(y.float()).all().item())
        ms0 = per[0.0][0] if 0.0 in per else None
        for delta, (ms, M, ff) in per.items():
            points.append({"drafts": B, "delta": delta, "rec_rows": M, "fold_fraction_drafts": round(ff, 4),
                           "us": round(ms * 1e3, 2), "branch_tokens_per_s": round(R / (ms * 1e-3), 1),
                           "speedup_vs_dense": round(ms0 / ms, 4) if ms0 else None})
        points.append({"drafts": B, "delta": wl.delta, "finite_output": finite})
        print(f"[bench] B={B} done", file=sys.stderr, flush=True)
    print(json.dumps({"metric": METRIC, "unit": "branch-tokens/s", "workload": args.workload, "n_gpus": 1,
                      "dtype": "bf16", "data": "synthetic", "regime": f"cold ({n_copies} weight copies)",
                      "points": points}), flush=True)


def tree_bench(args, wl):
    """One layer at fixed B swept over the draft tree's shape (siblings of main, random trees of
    bounded depth, a chain), folded at the workload's delta against dense (delta 0).  The tests
    check the layer's parity with the oracle on each of these tree shapes."""
    import numpy as np
    import torch

    from sparse_layer_rho_amd import specfold as sf
    from synth import bf16_round, layer_weights, prefix_kv, step_inputs, tree_of

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sh = wl.shape
    R, D = sh.rows, sh.hidden

    def to_dev(x):
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev).to(torch.bfloat16)

    t0 = time.time()
    w_host = layer_weights(sh, wl.base_seed, 0)
    pk_h, pv_h = prefix_kv(sh, wl.base_seed, 0)
    w0 = {k: to_dev(v) for k, v in w_host.items()}
    n_copies = max(2, int(np.ceil(600e6 / sh.weight_bytes_bf16())))
    # the copies must outlive every launch that reads them: the structs hold raw pointers, and
    # graph capture empties the allocator's cache, returning freed blocks to the runtime
    copies = [w0] + [{k: v.clone() for k, v in w0.items()} for _ in range(n_copies - 1)]
    lws = [sf.layer_weights_struct(c) for c in copies]
    pk, pv = to_dev(pk_h), to_dev(pv_h)
    pf = sf.prefix_view(pk, pv)
    ws = sf.new_workspace(sh)
    y = torch.empty((R, D), dtype=torch.bfloat16, device=dev)
    st = {"fold": torch.zeros(R, dtype=torch.uint8, device=dev), "rec_count": torch.zeros(1, dtype=torch.int32, device=dev)}
    print(f"[bench] tree sweep ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    points = []
    n_steps = 4                                   # verification steps per tree shape (new draws each)
    for kind in wl.tree_sweep:
        parents, Hs = [], []
        for s in range(n_steps):
            parent = tree_of(kind, sh.n_branch, wl.base_seed, s)
            inp = step_inputs(sh, wl.base_seed, s, child_law=wl.child_law, parent=parent)
            parents.append(parent)
            Hs.append(to_dev(bf16_round(inp["H"].astype(np.float32)).reshape(R, D)))
        depth = np.zeros(sh.n_branch, dtype=np.int64)
        for i in range(1, sh.n_branch):
            depth[i] = depth[parents[0][i]] + 1
        res = {}
        for delta in (wl.delta, 0.0):
            Ms, ffs = [], []
            for s in range(n_steps):
                sf.verify_layer(sh, parents[s], lws[0], pf, None, Hs[s], delta, y, ws, stats=st)
                torch.cuda.synchronize()
                Ms.append(int(st["rec_count"].item()))
                ffs.append(float(st["fold"].cpu().numpy().reshape(sh.n_branch, sh.block)[1:].mean()))
            reps = max(1, args.steps // (4 * n_copies))
            ms = graph_time(torch, [lambda k=k, delta=delta: sf.verify_layer(sh, parents[k % n_steps], lws[k], pf, None,
                                                                            Hs[k % n_steps], delta, y, ws)
                                    for k in range(n_copies)], reps=reps) / n_copies
            res[delta] = (ms, float(np.mean(Ms)), float(np.mean(ffs)), ffs)
        finite = True
        for s in range(n_steps):
            sf.verify_layer(sh, parents[s], lws[0], pf, None, Hs[s], wl.delta, y, ws)
            torch.cuda.synchronize()
            finite = finite and bool(torch.isfinite(y.float()).all().item())
        (msf, M, ff, ffs), (msd, _, _, _) = res[wl.delta], res[0.0]
        points.append({"tree": kind, "parent_step0": parents[0].tolist(), "max_depth_step0": int(depth.max()),
                       "rec_rows_mean": round(M, 1), "fold_fraction_drafts": round(ff, 4),
                       "fold_fraction_per_step": [round(v, 4) for v in ffs], "us": round(msf * 1e3, 2),
                       "dense_us": round(msd * 1e3, 2), "branch_tokens_per_s": round(R / (msf * 1e-3), 1),
                       "speedup_vs_dense": round(msd / msf, 4), "finite_output": finite})
        print(f"[bench] tree {kind} done", file=sys.stderr, flush=True)
    print(json.dumps({"metric": METRIC, "unit": "branch-tokens/s", "workload": args.workload, "n_gpus": 1,
                      "dtype": "bf16", "data": "synthetic", "delta": wl.delta, "drafts": sh.n_branch - 1,
                      "regime": f"cold ({n_copies} weight copies)", "points": points}), flush=True)


def cpu_baseline_leg(sh, wl, parent, H_host, w_host, pk_h, pv_h, gpu_res, seconds):
    """Time the CPU oracle on the bench's first input and check the GPU's output of that same step
    against it (teacher-forced on the GPU's mask within 1e-4 of delta).  Timings are the median
    of 3 passes after one warm-up: with the BLAS threads the host gives this process, with one
    thread, and the dense pass (delta 0); `seconds` bounds each of the three (fewer passes are
    timed when one pass takes longer)."""
    import contextlib
    import platform
    import statistics

    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle

    H = H_host.astype(np.float64)
    fold_g = gpu_res["fold"].reshape(sh.n_branch, sh.block).astype(bool)
    rho_o, fold_o = oracle.gate(H, parent, wl.delta)
    band = np.abs(rho_o - wl.delta) < 1e-4
    ok_mask = bool(np.array_equal(fold_g[~band], fold_o[~band]))
    ref = oracle.verify_layer(H, parent, w_host, pk_h, pv_h, wl.delta, sh, fold=fold_g)
    got = gpu_res["H_out"].float().cpu().numpy().astype(np.float64).reshape(H.shape)
    err = float(np.linalg.norm(got - ref["H_out"]) / np.linalg.norm(ref["H_out"]))
    verified = ok_mask and err <= 2e-2 and gpu_res["M"] == ref["rec_rows"].size

    def timed(delta, limit):
        ctx = threadpool_limits(limits=limit) if limit else contextlib.nullcontext()
        with ctx:
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
            t0 = time.perf_counter()
            oracle.verify_layer(H, parent, w_host, pk_h, pv_h, delta, sh)       # warm-up
            first = time.perf_counter() - t0
            n = 3 if 3 * first <= seconds else 1
            ts = []
            for _ in range(n):
                t0 = time.perf_counter()
                oracle.verify_layer(H, parent, w_host, pk_h, pv_h, delta, sh)
                ts.append(time.perf_counter() - t0)
        return statistics.median(ts), n, threads

    t_all, n_all, threads = timed(wl.delta, None)
    t_one, n_one, _ = timed(wl.delta, 1)
    t_dense, n_dense, _ = timed(0.0, None)
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = sorted({f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info()
                   if p.get("user_api") == "blas"})
    cpu = {"value": round(sh.rows / t_all, 1), "unit": "branch-tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"median of {n_all} float64 oracle passes (after one warm-up) of the bench's first step "
                     f"({sh.rows} rows, delta {wl.delta}) on {threads} BLAS threads",
           "seconds_per_pass": round(t_all, 4),
           "one_thread": {"value": round(sh.rows / t_one, 1), "seconds_per_pass": round(t_one, 4), "passes": n_one},
           "dense_delta0": {"value": round(sh.rows / t_dense, 1), "seconds_per_pass": round(t_dense, 4),
                            "passes": n_dense, "speedup_of_folding": round(t_dense / t_all, 4)},
           "cpu_model": model, "host_cpus_available": len(os.sched_getaffinity(0)), "blas": blas}
    return cpu, {"ok": bool(verified), "rel_l2": round(err, 6), "mask_match_outside_band": ok_mask}


if __name__ == "__main__":
    main()
