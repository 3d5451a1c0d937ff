"""Benchmark: one global cross-frame attention layer at 1000 frames, all forms.

A step is one pass of the whole hot path over one batch of seeded synthetic
Q/K/V (1000 frames x 1374 tokens, 16 heads, d=64, bf16; inputs resident in HBM
before timing starts):
  dense global attention; frame attention (early-layer form);
  GSA: pool -> compressed attention -> top-16 selection -> fine attention -> gate;
  AVGGT subsampled attention (4x4 stride): compaction -> attention.
Every kernel of the step is launched on torch's current stream; per-call times
come from HIP events on that stream over the timed region.

After the timed steps, variants are timed outside the step: the Speed3R GSA
variants on the same inputs (the VGGT adaptation: reference frame 0 kept
whole, top-16 over the other frames; the test-time top-128; the block-level
compressed branch; pooling of the zero-padded grid), the AVGGT subsampling factor 2..9, its token-level
diagonal, and AVGGT's layer schedule (frame attention for the early layers,
subsampled after) at 100, 300 and 800 frames.

Then the GSA form at 128 frames and the subsampled form at 256 frames are each
timed against dense attention at the same size, and the fp64 CPU oracle is
timed on a seeded row sample of every form of the step.

Prints one JSON line. `value` = tokens of the batch / seconds per step. The
per-form rates and speed-ups also appear as plain numbers in `roofline` and
`cpu_baseline`, whose scalar fields the run record keeps.
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

METRIC = "global-attn layer tokens/s @1000 frames (dense vs GSA vs subsampled); % MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="scene1000")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="query rows of the CPU-oracle baseline's dense sample (0 disables the "
                         "baseline); frame and subsampled attention take 8x, GSA 2x as many rows")
    ap.add_argument("--cpu-rows-all", type=int, default=0,
                    help="if set, every form's CPU sample takes this many rows (e.g. 4096)")
    ap.add_argument("--small-configs", type=int, default=1,
                    help="also time the 128-frame GSA and 256-frame subsampled configurations "
                         "against dense at the same size (0 skips them)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--variant-steps", type=int, default=1,
                    help="timed passes of each GSA variant after one untimed pass (0 skips them)")
    ap.add_argument("--cpu-report", default="",
                    help="only run the CPU-baseline leg over every configuration (the fp64 "
                         "oracle on this host: the whole layer at 4 and 32 frames, 4096 seeded "
                         "rows at 128, 256 and 1000 frames) and write its JSON to this path")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (3 times) "
                         "so hardware byte counters can be scaled against known traffic")
    return ap.parse_args()


def copy_calibration(mib: int):
    import torch
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)


def main():
    args = parse()
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return
    if args.cpu_report:
        cpu_report(args.cpu_report, args.seed)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the sharded multi-GPU "
              "path is a design note, not part of this build.", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_global_amd as sga
    from synth import WORKLOADS, make_gate, make_qkv

    wl = WORKLOADS[args.workload]
    geom = wl.geom
    T, H, d, N = geom.n_tokens, geom.n_heads, geom.head_dim, geom.n_frames
    nb, _ = sga.pooled_shape(geom)
    sh, sw = wl.stride
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = make_qkv(geom, seed=args.seed, device=dev, distribution=wl.distribution)
    w, b = make_gate(H, d, seed=args.seed, device=dev)
    ws = torch.empty(sga.workspace_bytes(geom, sh, sw, sga.SGA_BF16), dtype=torch.uint8, device=dev)
    ws_fine = torch.empty(sga.fine_workspace_bytes(geom, sga.SGA_BF16, True), dtype=torch.uint8,
                          device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready: {args.workload} T={T} H={H} d={d}", file=sys.stderr, flush=True)

    names = ["dense", "frame", "gsa_pool", "gsa_compressed", "gsa_topk", "gsa_fine", "gsa_gate",
             "sga"]

    last = {}

    def gsa_chain(ev, i, top_k, keep_ref, ws_f, pooled_q=False, include_pad=False, prob=False):
        """The five GSA calls, an event recorded after each."""
        k_cmp, v_cmp, k32, q32 = sga.gsa_compress(q, k, v, geom, include_pad=include_pad)
        ev[i].record(); i += 1
        if pooled_q:
            o_cmp = sga.gsa_compressed_pooled(q32, k_cmp, v_cmp, geom)
        else:
            o_cmp = sga.dense_global_attn(q, k_cmp, v_cmp, geom, n_keys=N * nb)
        ev[i].record(); i += 1
        if prob:
            idx = sga.gsa_select_topk_probability(q, k32, geom, top_k, keep_ref=keep_ref)
        else:
            idx = sga.gsa_select_topk(q32, k32, geom, top_k, keep_ref=keep_ref)
        ev[i].record(); i += 1
        o_slc = sga.gsa_sparse_attn(q, k, v, idx, geom, top_k, ws=ws_f, keep_ref=keep_ref)
        ev[i].record(); i += 1
        sga.gsa_gate(q, o_cmp, o_slc, w, b, geom)
        ev[i].record(); i += 1
        return i, idx

    def step(ev):
        i = 0
        ev[i].record(); i += 1
        sga.dense_global_attn(q, k, v, geom)
        ev[i].record(); i += 1
        sga.dense_global_attn(q, k, v, geom, frame_local=True)
        ev[i].record(); i += 1
        i, last["idx"] = gsa_chain(ev, i, wl.top_k, False, ws_fine)
        sga.subsampled_global_attn(q, k, v, geom, sh, sw, ws=ws)
        ev[i].record(); i += 1

    def events():
        return [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]

    for it in range(args.warmup):
        step(events())
        torch.cuda.synchronize()
        print(f"[bench] warmup step {it + 1}/{args.warmup} done", file=sys.stderr, flush=True)

    per = {n: 0.0 for n in names}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    all_ev = []
    for it in range(args.steps):
        ev = events()
        step(ev)
        all_ev.append(ev)
        ev[-1].synchronize()  # progress line per step; costs one host wait per step
        print(f"[bench] timed step {it + 1}/{args.steps} done", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for ev in all_ev:
        for j, n in enumerate(names):
            per[n] += ev[j].elapsed_time(ev[j + 1]) / args.steps  # ms
    ms_step = wall * 1e3 / args.steps
    print(f"[bench] timed {args.steps} steps: {ms_step:.1f} ms/step", file=sys.stderr, flush=True)

    # ---- derived figures ------------------------------------------------------
    flop_dense = 4.0 * T * T * d * H
    flop_frame = 4.0 * N * geom.tokens_per_frame ** 2 * d * H
    flop_cmp = 4.0 * T * (N * nb) * d * H
    mk, has_mean = sga.compact_rows(geom, sh, sw)
    keys_sga = geom.tokens_per_frame + (N - 1) * (mk + has_mean)
    flop_sga = 4.0 * T * keys_sga * d * H
    t_gsa = sum(per[n] for n in names if n.startswith("gsa_"))
    layers = {
        "dense": {"ms": per["dense"], "tokens_per_s": T / per["dense"] * 1e3,
                  "tflops": flop_dense / per["dense"] / 1e9,
                  "mfma_frac": flop_dense / per["dense"] / 1e9 / PEAK_BF16_TFLOPS},
        "frame": {"ms": per["frame"], "tokens_per_s": T / per["frame"] * 1e3,
                  "tflops": flop_frame / per["frame"] / 1e9,
                  "mfma_frac": flop_frame / per["frame"] / 1e9 / PEAK_BF16_TFLOPS},
        "gsa": {"ms": t_gsa, "tokens_per_s": T / t_gsa * 1e3,
                "speedup_vs_dense": per["dense"] / t_gsa,
                "kernels_ms": {n[4:]: per[n] for n in names if n.startswith("gsa_")},
                "compressed_tflops": flop_cmp / per["gsa_compressed"] / 1e9,
                "compressed_mfma_frac": flop_cmp / per["gsa_compressed"] / 1e9 / PEAK_BF16_TFLOPS,
                "kernels_roofline": None},
        "subsampled": {"ms": per["sga"], "tokens_per_s": T / per["sga"] * 1e3,
                       "speedup_vs_dense": per["dense"] / per["sga"],
                       "tflops": flop_sga / per["sga"] / 1e9,
                       "mfma_frac": flop_sga / per["sga"] / 1e9 / PEAK_BF16_TFLOPS},
    }
    if args.variant_steps > 0:
        layers["gsa_variants"] = {}
        for vname, vk, vref, vpool, vpad, vprob in (
                ("vggt_reference_frame", wl.top_k, True, False, False, False),
                ("top128", 128, False, False, False, False),
                ("block_level_compressed", wl.top_k, False, True, False, False),
                ("zero_padded_pooling", wl.top_k, False, False, True, False),
                ("probability_mean_block_score", wl.top_k, False, False, False, True)):
            ws_v = torch.empty(sga.fine_workspace_bytes(geom, sga.SGA_BF16, True, vref),
                               dtype=torch.uint8, device=dev)
            gnames = [n for n in names if n.startswith("gsa_")]
            vper = {n: 0.0 for n in gnames}
            for rep in range(1 + args.variant_steps):  # the first pass is untimed
                ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(gnames) + 1)]
                ev[0].record()
                _, vidx = gsa_chain(ev, 1, vk, vref, ws_v, vpool, vpad, vprob)
                torch.cuda.synchronize()
                if rep:
                    for j, n in enumerate(gnames):
                        vper[n] += ev[j].elapsed_time(ev[j + 1]) / args.variant_steps
            t_v = sum(vper.values())
            layers["gsa_variants"][vname] = {
                "top_k": vk, "reference_frame_kept": vref, "block_level_compressed": vpool,
                "zero_padded_pooling": vpad, "probability_mean_block_score": vprob, "ms": t_v,
                "tokens_per_s": T / t_v * 1e3, "speedup_vs_dense": per["dense"] / t_v,
                "kernels_ms": {n[4:]: vper[n] for n in gnames},
                "kernels_roofline": gsa_rooflines(geom, vper, vidx, keep_ref=vref, pooled_q=vpool, prob=vprob)}
            del ws_v, vidx
            print(f"[bench] variant {vname}: {t_v:.1f} ms", file=sys.stderr, flush=True)

    fine_windows_ms = None
    if args.variant_steps > 0:
        def timed(fn, reps):
            """ms per call from HIP events on the current stream; one untimed call first."""
            fn()
            t = 0.0
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                fn()
                e1.record()
                e1.synchronize()
                t += e0.elapsed_time(e1) / reps
            return t

        # the fine branch's window kernel alone (no always-kept tokens)
        fine_windows_ms = timed(lambda: sga.gsa_sparse_attn(q, k, v, last["idx"], geom, wl.top_k,
                                                            keep_special=False), args.variant_steps)
        # the gate folded into the fine branch's epilogue (what gsa_layer runs):
        # against the separate fine and gate calls of the step
        k_cmp_g, v_cmp_g, _, _ = sga.gsa_compress(q, k, v, geom)
        o_cmp_g = sga.dense_global_attn(q, k_cmp_g, v_cmp_g, geom, n_keys=N * nb)
        del k_cmp_g, v_cmp_g
        t_fg = timed(lambda: sga.gsa_sparse_attn_gated(q, k, v, last["idx"], o_cmp_g, w, b, geom, wl.top_k,
                                                       ws=ws_fine), args.variant_steps)
        del o_cmp_g
        layers["gsa"]["gate_fused_into_fine"] = {
            "fine_gated_ms": t_fg, "fine_then_gate_ms": per["gsa_fine"] + per["gsa_gate"],
            "saved_ms": per["gsa_fine"] + per["gsa_gate"] - t_fg,
            "layer_ms": t_gsa - per["gsa_fine"] - per["gsa_gate"] + t_fg}
        # AVGGT compaction alone (HBM: read K and V, write the compacted set)
        t_cp = timed(lambda: sga.sga_compact(k, v, geom, sh, sw), args.variant_steps)
        cp_bytes = 2 * T * H * d * 2 + 2 * N * (mk + has_mean) * H * d * 2
        layers["subsampled"]["compaction"] = {
            "ms": t_cp, "bound": "hbm", "gb_per_s": cp_bytes / (t_cp * 1e-3) / 1e9,
            "frac": cp_bytes / (t_cp * 1e-3) / 1e9 / PEAK_HBM_GBS, "bytes": cp_bytes}
        # AVGGT subsampling factor sigma = 2..9 (sigma x sigma windows)
        sweep = {}
        for sig in range(2, 10):
            ws_s = torch.empty(sga.workspace_bytes(geom, sig, sig, sga.SGA_BF16), dtype=torch.uint8,
                               device=dev)
            t_s = timed(lambda: sga.subsampled_global_attn(q, k, v, geom, sig, sig, ws=ws_s),
                        args.variant_steps)
            mk_s, hm_s = sga.compact_rows(geom, sig, sig)
            fl_s = 4.0 * T * (geom.tokens_per_frame + (N - 1) * (mk_s + hm_s)) * d * H
            sweep[str(sig)] = {"ms": t_s, "speedup_vs_dense": per["dense"] / t_s,
                               "keys_per_query": geom.tokens_per_frame + (N - 1) * (mk_s + hm_s),
                               "tflops": fl_s / t_s / 1e9,
                               "mfma_frac": fl_s / t_s / 1e9 / PEAK_BF16_TFLOPS}
            del ws_s
        layers["subsampled_sigma_sweep"] = sweep
        # AVGGT's diagonal read at token level (mode 2), at the workload's stride
        ws_td = torch.empty(sga.workspace_bytes(geom, sh, sw, sga.SGA_BF16), dtype=torch.uint8,
                            device=dev)
        t_td = timed(lambda: sga.subsampled_global_attn(q, k, v, geom, sh, sw, mode=2, ws=ws_td),
                     args.variant_steps)
        fl_td = 4.0 * T * N * (mk + has_mean) * d * H
        layers["subsampled_token_diagonal"] = {
            "ms": t_td, "speedup_vs_dense": per["dense"] / t_td, "tflops": fl_td / t_td / 1e9,
            "mfma_frac": fl_td / t_td / 1e9 / PEAK_BF16_TFLOPS}
        del ws_td
        print(f"[bench] token-diagonal subsampled: {t_td:.1f} ms", file=sys.stderr, flush=True)
        print("[bench] sigma sweep: " + " ".join(f"{k_}:{v_['ms']:.0f}ms" for k_, v_ in sweep.items()),
              file=sys.stderr, flush=True)
        layers["avggt_schedule"] = avggt_schedule(sga, torch, make_qkv, geom, wl, dev, timed,
                                                  args.seed)

    layers["gsa"]["kernels_roofline"] = gsa_rooflines(geom, per, last["idx"],
                                                      fine_windows_ms=fine_windows_ms)

    achieved = flop_dense / (per["dense"] * 1e-3) / 1e12
    roofline = {"kernel": "flash_bf16_kernel<GLOBAL> (dense global attention)",
                "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "flop_per_launch": flop_dense, "traffic": None}
    traffic = measured_traffic(args.workload)
    if traffic is not None:
        roofline["traffic"] = traffic
        roofline["traffic_unit"] = "bytes per launch (HBM read + write, rocprofv3 FETCH_SIZE/WRITE_SIZE scaled)"

    small = None
    if args.small_configs:
        del q, k, v
        torch.cuda.empty_cache()
        small = small_config_speedups(sga, torch, make_qkv, make_gate, args.seed, dev)
        q, k, v = make_qkv(geom, seed=args.seed, device=dev, distribution=wl.distribution)

    cpu = None
    if args.cpu_rows > 0:
        rows_per_form = ({f: args.cpu_rows_all for f in ("dense", "frame", "gsa", "subsampled")}
                         if args.cpu_rows_all else
                         {"dense": args.cpu_rows, "frame": 8 * args.cpu_rows, "gsa": 2 * args.cpu_rows,
                          "subsampled": 8 * args.cpu_rows})
        cpu = cpu_baseline(q, k, v, w, b, geom, wl, rows_per_form, args.seed, layers)

    # the per-form figures as plain numbers in the two objects whose scalar
    # fields the run record keeps
    roofline["dense_tokens_per_s"] = layers["dense"]["tokens_per_s"]
    roofline["gsa_tokens_per_s"] = layers["gsa"]["tokens_per_s"]
    roofline["subsampled_tokens_per_s"] = layers["subsampled"]["tokens_per_s"]
    roofline["frame_tokens_per_s"] = layers["frame"]["tokens_per_s"]
    roofline["gsa_speedup_vs_dense"] = layers["gsa"]["speedup_vs_dense"]
    roofline["subsampled_speedup_vs_dense"] = layers["subsampled"]["speedup_vs_dense"]
    roofline["gsa_compressed_mfma_frac"] = layers["gsa"]["compressed_mfma_frac"]
    roofline["gsa_topk_ms"] = layers["gsa"]["kernels_ms"]["topk"]
    roofline["subsampled_mfma_frac"] = layers["subsampled"]["mfma_frac"]
    if small is not None:
        roofline["gsa128_speedup_vs_dense"] = small["gsa128"]["speedup_vs_dense"]
        roofline["sga256_speedup_vs_dense"] = small["sga256"]["speedup_vs_dense"]
        layers["small_configs"] = small

    line = {
        "metric": METRIC, "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded scene-correlated Q/K/V, no dataset or weights)",
        "config": {"workload": f"{args.workload}: {N} frames x {geom.tokens_per_frame} tokens "
                               f"(37x37 patches + camera + 4 registers), 16 heads, d=64, bf16; "
                               f"step = dense + frame + GSA(4x4 pool, top-{wl.top_k}) + "
                               f"subsampled({sh}x{sw})",
                   "frames": N, "tokens": T, "heads": H, "head_dim": d, "top_k": wl.top_k,
                   "stride": [sh, sw]},
        "layers": layers,
        "forms": {n: {"tokens_per_s": layers[n]["tokens_per_s"], "ms": layers[n]["ms"],
                      "speedup_vs_dense": per["dense"] / layers[n]["ms"]}
                  for n in ("dense", "frame", "gsa", "subsampled")},
        "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


GLOBAL_LAYERS = 24   # global-attention layers of the model (not stated by the pages; VGGT's depth)
FRAME_LAYERS = 9     # early global layers turned into frame attention (indices 0-8)


def avggt_schedule(sga, torch, make_qkv, geom1000, wl, dev, timed, seed):
    """AVGGT's two-step schedule over the model's global-attention layers at
    100, 300 and 800 frames: layers 0-8 as frame attention, the rest as
    subsampled attention (4x4), against every layer dense. One timed call of
    each form per size; the per-layer times let any layer count be recomposed."""
    out = {"global_layers": GLOBAL_LAYERS, "frame_layers": FRAME_LAYERS, "stride": list(wl.stride)}
    sh, sw = wl.stride
    for n in (100, 300, 800):
        g = geom1000.replace(n_frames=n)
        q, k, v = make_qkv(g, seed=seed, device=dev, distribution=wl.distribution)
        ws_d = torch.empty(sga.dense_workspace_bytes(g, sga.SGA_BF16), dtype=torch.uint8, device=dev)
        ws_f = torch.empty(sga.dense_workspace_bytes(g, sga.SGA_BF16, frame_local=True),
                           dtype=torch.uint8, device=dev)
        ws_s = torch.empty(sga.workspace_bytes(g, sh, sw, sga.SGA_BF16), dtype=torch.uint8, device=dev)
        t_d = timed(lambda: sga.dense_global_attn(q, k, v, g, ws=ws_d), 1)
        t_f = timed(lambda: sga.dense_global_attn(q, k, v, g, frame_local=True, ws=ws_f), 1)
        t_s = timed(lambda: sga.subsampled_global_attn(q, k, v, g, sh, sw, ws=ws_s), 1)
        dense_stack = GLOBAL_LAYERS * t_d
        avggt_stack = FRAME_LAYERS * t_f + (GLOBAL_LAYERS - FRAME_LAYERS) * t_s
        out[str(n)] = {"dense_ms": t_d, "frame_ms": t_f, "subsampled_ms": t_s,
                       "dense_stack_ms": dense_stack, "avggt_stack_ms": avggt_stack,
                       "speedup": dense_stack / avggt_stack}
        print(f"[bench] avggt schedule at {n} frames: {dense_stack:.0f} ms dense, "
              f"{avggt_stack:.0f} ms scheduled ({dense_stack / avggt_stack:.1f}x)",
              file=sys.stderr, flush=True)
        del q, k, v, ws_d, ws_f, ws_s
    return out


def gsa_rooflines(geom, per, idx, keep_ref=False, pooled_q=False, fine_windows_ms=None, prob=False):
    """Per-step roofline of the GSA kernels from their timed durations:
    algorithmic bytes (HBM-bound steps) or flop (MFMA steps) per call. With
    ``keep_ref`` frame 0 is attended whole and its blocks do not compete.
    Given the time of the fine branch's window kernel alone, the fine branch is
    split into its window gather (bytes of the selected keys and values) and
    the attention over the always-kept tokens (MFMA)."""
    import torch
    T, H, d, N, S = geom.n_tokens, geom.n_heads, geom.head_dim, geom.n_frames, geom.n_special
    nbh, nbw = -(-geom.grid_h // 4), -(-geom.grid_w // 4)
    nb = nbh * nbw
    nqb = nb + (1 if S else 0)
    # tokens per 4x4 window (edge windows are clipped to the grid)
    rows = torch.tensor([min(4, geom.grid_h - 4 * by) for by in range(nbh)])
    cols = torch.tensor([min(4, geom.grid_w - 4 * bx) for bx in range(nbw)])
    win = (rows[:, None] * cols[None, :]).reshape(-1).to(idx.device)
    qcount = torch.cat([win, torch.tensor([S], device=idx.device)])[:nqb] if S else win
    sel = win[(idx.long() % nb)].sum(dim=2)                   # [H, N*nqb] keys chosen
    per_block = qcount.repeat(N)[None, :].double()            # queries per block
    kept = (geom.tokens_per_frame + (N - 1) * S) if keep_ref else N * S
    pairs = float((per_block * (sel.double() + kept)).sum())  # (query, key) pairs, all heads
    kept_pairs = float(per_block.sum()) * H * kept
    n_cand = (N - 1) * nb if keep_ref else N * nb
    out = {}
    pool_bytes = 3 * T * H * d * 2 + N * nb * H * d * (2 + 2 + 4) + N * nqb * H * d * 4
    gate_bytes = 4 * T * H * d * 2
    # top-K: one product per block score; with probability-mean scores one per
    # token logit, twice (the log-sum-exp over all pooled keys, then the sums)
    topk_flop = (2.0 * d * T * (N * nb + n_cand) * H) if prob else 2.0 * d * (N * nqb) * n_cand * H
    flops = {"compressed": 4.0 * (N * nqb if pooled_q else T) * N * nb * d * H,
             "topk": topk_flop,
             "fine": 4.0 * d * pairs}
    for name, nbytes in (("pool", pool_bytes), ("gate", gate_bytes)):
        gbs = nbytes / (per["gsa_" + name] * 1e-3) / 1e9
        out[name] = {"bound": "hbm", "gb_per_s": gbs, "frac": gbs / PEAK_HBM_GBS, "bytes": nbytes}
    for name, fl in flops.items():
        tf = fl / (per["gsa_" + name] * 1e-3) / 1e12
        out[name] = {"bound": "mfma", "tflops": tf, "frac": tf / PEAK_BF16_TFLOPS, "flop": fl}
    # the scores run as three bf16 products (hi*hi + hi*lo + lo*hi) for fp32
    # accuracy; token logits as two (the bf16 query times hi and lo)
    mult = 2 if prob else 3
    out["topk"]["executed_flop"] = mult * flops["topk"]
    out["topk"]["executed_tflops"] = mult * out["topk"]["tflops"]
    # in-grid tokens per selected window (16 for an inner window, 4 or 1 at the edges)
    out["fine"]["selected_tokens_per_window"] = float(sel.double().sum()) / idx.numel()
    if fine_windows_ms is not None:
        gather_bytes = float(sel.double().sum()) * d * 2 * 2   # selected keys' K and V rows, bf16
        gbs = gather_bytes / (fine_windows_ms * 1e-3) / 1e9
        out["fine_windows"] = {"bound": "gather (HBM/L2)", "ms": fine_windows_ms, "gb_per_s": gbs,
                               "frac": gbs / PEAK_HBM_GBS, "bytes": gather_bytes}
        t_kept = per["gsa_fine"] - fine_windows_ms
        if t_kept > 0:
            tf = 4.0 * d * kept_pairs / (t_kept * 1e-3) / 1e12
            out["fine_kept"] = {"bound": "mfma", "ms": t_kept, "tflops": tf,
                                "frac": tf / PEAK_BF16_TFLOPS, "flop": 4.0 * d * kept_pairs}
    return out


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "flash_dense_scene1000_traffic.json")


def measured_traffic(workload):
    """HBM bytes per launch of the dense kernel from the committed counter
    record, only while the kernel sources are the ones it was taken from."""
    if workload != "scene1000" or not os.path.exists(TRAFFIC_RECORD):
        return None
    with open(TRAFFIC_RECORD) as fh:
        rec = json.load(fh)
    digest = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as fh:
            digest.update(fh.read())
    if digest.hexdigest() != rec["sources_sha256"]:
        return None
    return rec["fetch_bytes"] + rec["write_bytes"]


def cpu_baseline(q, k, v, w, b, geom, wl, rows_per_form, seed, layers):
    """Time the fp64 oracle, as it stands, on a bounded sample of each form of
    the step (a seeded row sample per form, all heads), on this host's cores."""
    import oracle
    from synth import sample_rows

    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:
        host_cores = os.cpu_count() or 1
    workers = max(1, min(16, host_cores))
    print(f"[bench] cpu baseline: copying inputs to host; {host_cores} host cores, "
          f"{workers} oracle threads", file=sys.stderr, flush=True)
    host = lambda x: x.detach().to("cpu").float().numpy()  # noqa: E731
    qh, kh, vh, wh, bh = host(q), host(k), host(v), host(w), host(b)
    sh, sw = wl.stride
    T = geom.n_tokens
    calls = {
        "dense": lambda r: oracle.dense_attention(qh, kh, vh, rows=r, workers=workers),
        "frame": lambda r: oracle.frame_attention(qh, kh, vh, geom, rows=r),
        "gsa": lambda r: oracle.gsa_layer(qh, kh, vh, geom, wh, bh, wl.top_k, rows=r, workers=workers),
        "subsampled": lambda r: oracle.subsampled_attention(qh, kh, vh, geom, sh, sw, rows=r, workers=workers),
    }
    out = {"value": None, "unit": "tokens/s", "cores": workers, "host_cores": host_cores,
           "oracle_threads": workers, "kind": "oracle"}
    total_rows, total_s = 0, 0.0
    for i, (form, fn) in enumerate(calls.items()):
        rows = sample_rows(T, rows_per_form[form], seed=seed + 100 + i).numpy()
        t0 = time.perf_counter()
        fn(rows)
        dt = time.perf_counter() - t0
        rate = len(rows) / dt
        out[f"{form}_rows"] = len(rows)
        out[f"{form}_s"] = dt
        out[f"{form}_tokens_per_s"] = rate
        out[f"{form}_extrapolated_full_layer_s"] = T / rate
        out[f"{form}_gpu_over_cpu"] = layers[form]["tokens_per_s"] / rate
        total_rows += len(rows)
        total_s += dt
        print(f"[bench] cpu baseline {form}: {len(rows)} rows in {dt:.1f} s ({rate:.1f} rows/s)",
              file=sys.stderr, flush=True)
    # the whole step (all four forms) at the sampled per-form rates
    step_s = sum(T / out[f"{f}_tokens_per_s"] for f in calls)
    out["value"] = T / step_s
    out["extrapolated_full_step_s"] = step_s
    out["sample"] = (", ".join(f"{f} {out[f + '_rows']}" for f in calls) +
                     f" seeded query rows x all {geom.n_heads} heads (GSA incl. its whole pooling, "
                     f"subsampled incl. its whole compaction), fp64 NumPy oracle, {workers} threads; "
                     f"{total_s:.1f} s")
    return out


def cpu_report(path, seed):
    """The CPU-baseline leg over every configuration: the fp64 oracle, as it
    stands, timed on this host's cores (no GPU is used). The whole layer where
    it is affordable (4 frames, fp32; 32 frames), else 4096 seeded query rows
    (all heads) with the full layer extrapolated from the measured rate."""
    import contextlib
    import io
    import numpy as np
    import oracle
    from synth import WORKLOADS, make_gate, make_qkv, sample_rows

    try:
        host_cores = len(os.sched_getaffinity(0))
    except AttributeError:
        host_cores = os.cpu_count() or 1
    workers = max(1, min(16, host_cores))
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        np.show_config()
    plan = [("tiny", ("dense", "frame", "gsa", "subsampled"), None),
            ("dense32", ("dense", "frame"), None),
            ("gsa128", ("dense", "gsa"), 4096),
            ("sga256", ("dense", "frame", "subsampled"), 4096),
            ("scene1000", ("dense", "frame", "gsa", "subsampled"), 4096)]
    out = {"command": f"python bench.py --cpu-report {path}", "kind": "oracle", "host_cores": host_cores,
           "oracle_threads": workers,
           "numpy": np.__version__, "numpy_config": buf.getvalue(), "configs": {}}
    for name, forms, n_rows in plan:
        wl = WORKLOADS[name]
        g = wl.geom
        q, k, v = make_qkv(g, seed=seed, device="cpu", distribution=wl.distribution)
        w, b = make_gate(g.n_heads, g.head_dim, seed=seed, device="cpu")
        qh, kh, vh = (x.float().numpy() for x in (q, k, v))
        wh, bh = w.numpy(), b.numpy()
        del q, k, v
        T = g.n_tokens
        rows = None if n_rows is None else sample_rows(T, n_rows, seed=seed + 7).numpy()
        sh, sw = wl.stride
        calls = {
            "dense": lambda r: oracle.dense_attention(qh, kh, vh, rows=r, workers=workers),
            "frame": lambda r: oracle.frame_attention(qh, kh, vh, g, rows=r),
            "gsa": lambda r: oracle.gsa_layer(qh, kh, vh, g, wh, bh, wl.top_k, rows=r, workers=workers),
            "subsampled": lambda r: oracle.subsampled_attention(qh, kh, vh, g, sh, sw, rows=r,
                                                                workers=workers),
        }
        res = {"frames": g.n_frames, "tokens": T, "heads": g.n_heads, "dtype": g.dtype,
               "rows": T if rows is None else len(rows)}
        all_rows = np.arange(T) if rows is None else rows
        for form in forms:
            # in parts of about 1024 rows, each reported (the GSA layer pools the
            # whole batch on every call, so it runs in one part)
            parts = [all_rows] if form == "gsa" else np.array_split(all_rows, max(1, len(all_rows) // 1024))
            dt = 0.0
            for part in parts:
                t0 = time.perf_counter()
                calls[form](None if (rows is None and len(parts) == 1) else part)
                dt += time.perf_counter() - t0
                print(f"[cpu-report] {name} {form}: part of {len(part)} rows done", file=sys.stderr,
                      flush=True)
            n = T if rows is None else len(rows)
            res[form] = {"seconds": dt, "rows_per_s": n / dt,
                         "full_layer_s": dt if rows is None else T * dt / n,
                         "full_layer": "measured" if rows is None else "extrapolated"}
            print(f"[cpu-report] {name} {form}: {n} rows in {dt:.1f} s", file=sys.stderr, flush=True)
        out["configs"][name] = res
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps({k: v for k, v in out.items() if k != "numpy_config"}), flush=True)


def small_config_speedups(sga, torch, make_qkv, make_gate, seed, dev):
    """The GSA form at 128 frames and the subsampled form at 256 frames against
    dense attention at the same size, and every form at 4 frames (fp32) and 32
    frames (one untimed call each, then the median of three timed ones)."""
    from synth import WORKLOADS

    def timed(fn):
        fn()
        ts = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        return sorted(ts)[1]

    out = {}
    for name in ("gsa128", "sga256"):
        wl = WORKLOADS[name]
        g = wl.geom
        q, k, v = make_qkv(g, seed=seed, device=dev, distribution=wl.distribution)
        ws_d = torch.empty(sga.dense_workspace_bytes(g, sga.SGA_BF16), dtype=torch.uint8, device=dev)
        t_d = timed(lambda: sga.dense_global_attn(q, k, v, g, ws=ws_d))
        if name == "gsa128":
            w, b = make_gate(g.n_heads, g.head_dim, seed=seed, device=dev)
            t_x = timed(lambda: sga.gsa_layer(q, k, v, w, b, g, wl.top_k))
        else:
            sh, sw = wl.stride
            ws_s = torch.empty(sga.workspace_bytes(g, sh, sw, sga.SGA_BF16), dtype=torch.uint8, device=dev)
            t_x = timed(lambda: sga.subsampled_global_attn(q, k, v, g, sh, sw, ws=ws_s))
        T = g.n_tokens
        out[name] = {"frames": g.n_frames, "dense_ms": t_d, "form_ms": t_x,
                     "dense_tokens_per_s": T / t_d * 1e3, "form_tokens_per_s": T / t_x * 1e3,
                     "speedup_vs_dense": t_d / t_x}
        print(f"[bench] {name}: dense {t_d:.1f} ms, {'GSA' if name == 'gsa128' else 'subsampled'} "
              f"{t_x:.1f} ms ({t_d / t_x:.1f}x)", file=sys.stderr, flush=True)
        del q, k, v
        torch.cuda.empty_cache()
    # the two configurations parity runs on whole: 4 frames in fp32 (one head,
    # every form) and 32 frames in bf16 (dense and frame attention)
    for name in ("tiny", "dense32"):
        wl = WORKLOADS[name]
        g = wl.geom
        q, k, v = make_qkv(g, seed=seed, device=dev, distribution=wl.distribution)
        sh, sw = wl.stride
        forms = {"dense": lambda: sga.dense_global_attn(q, k, v, g),
                 "frame": lambda: sga.dense_global_attn(q, k, v, g, frame_local=True)}
        if name == "tiny":
            w, b = make_gate(g.n_heads, g.head_dim, seed=seed, device=dev)
            forms["gsa"] = lambda: sga.gsa_layer(q, k, v, w, b, g, wl.top_k)
            forms["subsampled"] = lambda: sga.subsampled_global_attn(q, k, v, g, sh, sw)
        T = g.n_tokens
        res = {"frames": g.n_frames, "heads": g.n_heads, "dtype": g.dtype}
        for form, fn in forms.items():
            t = timed(fn)
            res[form] = {"ms": t, "tokens_per_s": T / t * 1e3}
        out[name] = res
        print(f"[bench] {name}: " + ", ".join(f"{f} {res[f]['ms']:.3f} ms" for f in forms),
              file=sys.stderr, flush=True)
        del q, k, v
    return out


if __name__ == "__main__":
    main()
