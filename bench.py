"""Decode-step benchmark of the lossless compressed-KV attention path on one MI355X.

Workload (default): the 64K-token Qwen3-8B-like layer -- 1 sequence, 8 KV heads, 32 query heads,
head_dim 128, 65,536 context tokens, 64-token blocks, 16-token exponent groups, synthetic BF16
K/V with per-head log-normal channel scales and 4 outlier key channels per head.

One timed step = one decode step of one layer (kv_decode_step): append the new token and attend
over every token -- the split-K attention kernel over the finished blocks, then the merge kernel,
which also attends the tail with the new token and stores the token into the tail; a step whose
token completes a block runs the append (with the block encode) and both attention kernels.  Steps rotate over --layers independent layer caches so each step reads its layer cold
from HBM (the compressed layer, ~190 MB, would otherwise sit in the 256 MB last-level cache).
Layer i starts at 65536 - 8 i tokens, so block-completing appends (block encodes) fall inside the
timed steps at their natural rate, about one step in 64.  The same steps run on an uncompressed
BF16 cache with the same table, layout and kernel structure (the speedup baseline).  Before the
W warm-up steps, read-only attention passes run over every layer cache (at least two rotations
and 20 ms of GPU work), so no layer is read for the first time, and no clock ramp falls, inside
the timed region.  `value` is the clean pass: K steps with an event at each layer rotation and
nothing else (median/p10/p90 over those windows are reported beside the mean); a second,
instrumented pass of K steps runs the step's parts as separate calls (append, split attention,
merge) with events between them and times each one on the stream it runs on.

Prints one JSON line (rank 0, N = 1).
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
# Sources the compressed attention kernel is built from: the HBM-traffic figure recorded from
# hardware counters is only reported while these are byte-identical to what was profiled.
KERNEL_SOURCES = ("decode_attention_calibrate_amd/csrc/attention_kernels.hip",
                  "decode_attention_calibrate_amd/csrc/codec_dev.h",
                  "decode_attention_calibrate_amd/csrc/kvc_internal.h")
TRAFFIC_FILE = os.path.join("profiles", "attn_comp_kernel_qwen3-8b-64k_hbm_counters.md")
METRIC = "decode-attention µs/step + effective HBM GB/s at 64K ctx; lossless ratio"
LAYER_STAGGER = 8  # layer i starts 8 i tokens short of the context


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--splits", type=int, default=256)
    ap.add_argument("--layers", type=int, default=8, help="layer caches rotated through (cold-cache protocol)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--sweep", type=str, default="4,8,16,128,512",
                    help="comma-separated split counts at which the attention kernel alone is also timed (4, 8 "
                         "and 16 splits are the literal reading of 64-256 blocks per split); '' for none")
    ap.add_argument("--probe", action="store_true", help="also time plain HBM copy / read kernels (torch)")
    ap.add_argument("--extra", type=str, default="context,fp8,g8,paged,groups,nested,rope,serving,prefill,d256",
                    help="comma list of extra workloads measured after the headline one: context (the cfg2 "
                         "layer at 32K and 128K tokens), fp8 (the 64K layer in "
                         "FP8 E5M2 and E4M3), g8 (the 64K layer with 8-token exponent groups), paged (32-sequence paged serving mix), prefill (a 4K-token prompt: encode, "
                         "decode_blocks, causal prefill attention), groups (the 64K layer's "
                         "codec with 16- and 8-token exponent groups), rope (escape bytes and raw tiles along "
                         "the 64K layer with RoPE-rotated keys, per calibration policy), serving (sequences "
                         "admitted and decode throughput under one KV byte budget), d256 (a 32K-token layer with "
                         "256-channel heads, compressed and uncompressed decode steps); '' for none")
    ap.add_argument("--extra-steps", type=int, default=48)
    ap.add_argument("--paged-splits", type=int, default=16)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import decode_attention_calibrate_amd as K
    import synth

    torch.cuda.set_device(0)
    cfg = synth.config(2)
    T, D, Hkv, Hq = cfg.T, cfg.D, cfg.Hkv, cfg.Hq
    L0 = cfg.context[0]
    S = args.splits
    n_layers = args.layers
    log(f"[bench] generating {L0} tokens x {Hkv} heads x {D}")
    g, toks = synth.sequence_tokens(cfg)
    k0, v0 = toks[0]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    kd, vd = dev(k0[None]), dev(v0[None])
    steps_total = args.warmup + 2 * args.steps  # warm-up, clean pass, instrumented pass
    per_layer = (steps_total + n_layers - 1) // n_layers + 1
    kn, vn = g.tokens(per_layer * n_layers)
    k_new = dev(kn.reshape(n_layers, per_layer, 1, 1, Hkv, D))
    v_new = dev(vn.reshape(n_layers, per_layer, 1, 1, Hkv, D))
    q = dev(synth.queries(cfg))
    max_blocks = (L0 + per_layer) // T + 2
    n_tiles = max_blocks * 2 * Hkv

    def make(compressed, li):
        c = K.KVCache(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T, max_seqs=1,
                      max_blocks_per_seq=max_blocks, num_comp_slots=n_tiles if compressed else 0,
                      num_raw_slots=256 if compressed else n_tiles, compressed=compressed, perm_seed=7)
        c.calibrate(dev(k0[:cfg.n_cal]), dev(v0[:cfg.n_cal]))
        n0 = L0 - LAYER_STAGGER * li
        c.append([0], kd[:, :n0].contiguous(), vd[:, :n0].contiguous())
        return c

    # prefill: the bulk encode of the whole 64K-token layer (every block encoded in one launch)
    def bulk_encode_us(compressed):
        ts = []
        for _ in range(3):
            c = K.KVCache(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T, max_seqs=1,
                          max_blocks_per_seq=max_blocks, num_comp_slots=n_tiles if compressed else 0,
                          num_raw_slots=256 if compressed else n_tiles, compressed=compressed, perm_seed=7)
            c.calibrate(dev(k0[:cfg.n_cal]), dev(v0[:cfg.n_cal]))
            torch.cuda.synchronize()
            a_ = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            c.append([0], kd, vd)
            b_.record(stream)
            torch.cuda.synchronize()
            ts.append(a_.elapsed_time(b_) * 1e3)
            del c
        return float(np.median(ts))
    stream = torch.cuda.current_stream()
    bulk_c, bulk_r = bulk_encode_us(True), bulk_encode_us(False)
    log(f"[bench] bulk encode of {L0} tokens: compressed {bulk_c:.1f} us, uncompressed {bulk_r:.1f} us")

    log(f"[bench] building {n_layers} compressed + {n_layers} uncompressed layer caches")
    comp = [make(True, li) for li in range(n_layers)]
    raw = [make(False, li) for li in range(n_layers)]
    torch.cuda.synchronize()
    flags, st = comp[0].status()
    if flags:
        raise RuntimeError(f"cache status flags {flags}")

    # ---- byte accounting (algorithmic bytes one attention launch must read) ----
    TD = T * D
    n_grp = TD // 16
    payload_per_comp_tile = (2 * n_grp + 3 * TD + 8 * TD) // 8          # TAG + CODE + SM, without escapes
    comp_kv_bytes = st["comp_tiles"] * payload_per_comp_tile + st["esc_bytes"] + st["raw_tiles"] * TD * 2
    raw_kv_bytes = (st["comp_tiles"] + st["raw_tiles"]) * TD * 2
    codec_ratio = raw_kv_bytes / comp_kv_bytes
    resident = st["comp_tiles"] * comp[0].slot_stride + st["raw_tiles"] * TD * 2 + 4 * (st["comp_tiles"] + st["raw_tiles"])
    resident_ratio = raw_kv_bytes / resident
    q_bytes = Hq * D * 2
    table_bytes = 4 * (st["comp_tiles"] + st["raw_tiles"])
    log(f"[bench] codec ratio {codec_ratio:.4f}, resident ratio {resident_ratio:.4f}, tiles {st}")
    # exponent concentration (GAAC page §3.1): share of each head-channel's 65,536 exponents
    # inside its best window of w consecutive values (kv_window_coverage), mean over channels
    coverage = {"what": "mean over (kv-head, channel) of the share of the layer's exponents inside the "
                        "channel's best window of w consecutive exponent values (kv_window_coverage)"}
    for nm, x in (("k", kd[0]), ("v", vd[0])):
        for w in (4, 6, 8, 16):
            coverage[f"{nm}_w{w}"] = round(float(comp[0].window_coverage(x, w).double().mean()) / L0, 4)
    log(f"[bench] exponent coverage {coverage}")

    wsc = comp[0].workspace(1, S)
    out = torch.empty((1, Hq, D), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()

    def run(caches, n_steps, record, splits=S, ws=wsc, start=0):
        """n_steps decode steps starting at global step `start` (layer = step % n_layers).
        Unrecorded steps are kv_decode_step calls (the product's decode step); recorded steps
        run its three parts as separate calls (append, split attention, merge) with events
        between them, for the per-kernel breakdown."""
        ev = []
        for i in range(n_steps):
            step = start + i
            li = step % n_layers
            c = caches[li]
            pos = step // n_layers
            if not record:
                c.decode_step([0], k_new[li, pos], v_new[li, pos], q, cfg.scale, splits, ws, out)
                continue
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
            c.append([0], k_new[li, pos], v_new[li, pos])
            e[1].record(stream)
            c.attention_partials([0], q, cfg.scale, splits, ws)
            e[2].record(stream)
            c.attention_combine([0], q, cfg.scale, splits, ws, out)
            e[3].record(stream)
            ev.append(e)
        return ev

    def prime(caches, min_ms=20.0):
        """Read-only attention passes (split kernel + merge, no append, so no cache state changes)
        over every layer cache until at least two full rotations and min_ms of GPU work have run:
        every layer has been read before the timed region, and the GPU has left its idle clocks,
        whatever --warmup says.  Returns (passes, ms)."""
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        n = 0
        while n < 2 * len(caches) or (time.perf_counter() - h0) * 1e3 < min_ms:
            for c in caches:
                c.attention_partials([0], q, cfg.scale, S, wsc)
                c.attention_combine([0], q, cfg.scale, S, wsc, out)
                n += 1
            torch.cuda.synchronize()
        return n, (time.perf_counter() - h0) * 1e3

    def timed(caches, start):
        prime_n, prime_ms = prime(caches)
        run(caches, args.warmup, False, start=start)
        torch.cuda.synchronize()
        # the clean pass: K decode steps with one event per full layer rotation (window) and
        # nothing else between them; value = the whole pass over K
        n_win = max(1, args.steps // n_layers)
        bounds = [round(i * args.steps / n_win) for i in range(n_win + 1)]
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_win + 1)]
        h0 = time.perf_counter()
        evs[0].record(stream)
        for w in range(n_win):
            run(caches, bounds[w + 1] - bounds[w], False, start=start + args.warmup + bounds[w])
            evs[w + 1].record(stream)
        host_us = (time.perf_counter() - h0) * 1e6 / args.steps  # enqueue time per step
        torch.cuda.synchronize()
        wall_us = (time.perf_counter() - h0) * 1e6 / args.steps  # host clock, enqueue to completion
        total_ms = evs[0].elapsed_time(evs[-1])
        win_us = np.array([evs[w].elapsed_time(evs[w + 1]) * 1e3 / (bounds[w + 1] - bounds[w]) for w in range(n_win)])
        clean = {"mean": round(total_ms * 1e3 / args.steps, 3), "median": round(float(np.median(win_us)), 3),
                 "p10": round(float(np.percentile(win_us, 10)), 3), "p90": round(float(np.percentile(win_us, 90)), 3),
                 "windows": n_win, "steps_per_window": bounds[1] - bounds[0], "host_wall_mean": round(wall_us, 3),
                 "prime": {"attention_passes": prime_n, "ms": round(prime_ms, 1)}}
        ev = run(caches, args.steps, True, start=start + args.warmup + args.steps)
        torch.cuda.synchronize()
        step_us = np.array([a.elapsed_time(d) * 1e3 for a, b, c, d in ev])
        attn_us = np.array([b.elapsed_time(c) * 1e3 for a, b, c, d in ev])
        app_us = np.array([a.elapsed_time(b) * 1e3 for a, b, c, d in ev])
        comb_us = np.array([c.elapsed_time(d) * 1e3 for a, b, c, d in ev])
        return total_ms, step_us, attn_us, app_us, comb_us, host_us, clean

    def b2b(caches, reps=96):
        """The attention kernel alone, launched back to back over the rotated layers with an event
        at each end of the loop only (per-kernel events add a few µs of their own)."""
        for i in range(n_layers):
            caches[i].attention_partials([0], q, cfg.scale, S, wsc)
        torch.cuda.synchronize()
        a_ = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        for i in range(reps):
            caches[i % n_layers].attention_partials([0], q, cfg.scale, S, wsc)
        b_.record(stream)
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) * 1e3 / reps

    log(f"[bench] timing {args.steps} compressed steps (S={S})")
    c_total, c_step, c_attn, c_app, c_comb, c_host, c_clean = timed(comp, 0)
    log(f"[bench] timing {args.steps} uncompressed steps")
    r_total, r_step, r_attn, r_app, r_comb, r_host, r_clean = timed(raw, 0)
    c_b2b, r_b2b = b2b(comp), b2b(raw)
    log(f"[bench] attention back to back: compressed {c_b2b:.2f} us, uncompressed {r_b2b:.2f} us")

    sweep = {}
    for s_ in [int(x) for x in args.sweep.split(",") if x]:
        ws_ = comp[0].workspace(1, s_)
        for name, caches in (("comp", comp), ("raw", raw)):
            times = []
            for i in range(40):
                a_ = torch.cuda.Event(enable_timing=True)
                b_ = torch.cuda.Event(enable_timing=True)
                a_.record(stream)
                caches[i % n_layers].attention_partials([0], q, cfg.scale, s_, ws_)
                b_.record(stream)
                times.append((a_, b_))
            torch.cuda.synchronize()
            sweep.setdefault(str(s_), {})[name] = float(np.median([a_.elapsed_time(b_) * 1e3 for a_, b_ in times[8:]]))
        log(f"[bench] sweep S={s_}: {sweep[str(s_)]}")

    # block-completing append (encode of 2*Hkv tiles), measured on its own
    enc_us = None
    try:
        c = comp[0]
        n_now = c.seq_length(0)
        fill = (-n_now) % T
        if fill == 0:
            fill = T
        kf, vf = g.tokens(fill)
        kfd, vfd = dev(kf[None]), dev(vf[None])
        if fill > 1:
            c.append([0], kfd[:, :fill - 1].contiguous(), vfd[:, :fill - 1].contiguous())
        a_ = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a_.record(stream)
        c.append([0], kfd[:, fill - 1:].contiguous(), vfd[:, fill - 1:].contiguous())
        b_.record(stream)
        torch.cuda.synchronize()
        enc_us = a_.elapsed_time(b_) * 1e3
    except Exception as ex:  # measurement only
        log(f"[bench] encode timing skipped: {ex}")

    probe = hbm_probe(torch, stream) if args.probe else None

    attn_c = c_b2b
    attn_r = r_b2b
    bytes_c = comp_kv_bytes + q_bytes + table_bytes
    bytes_r = raw_kv_bytes + q_bytes + table_bytes
    achieved = bytes_c / (attn_c * 1e-6) / 1e9
    attain = attainable_read(torch, K, stream, bytes_c)
    attain_r = attainable_read(torch, K, stream, bytes_r)
    bound_r = bytes_r / (attain_r["GBps"] * 1e9) * 1e6
    digest = kernel_source_digest()
    traffic = counter_traffic(digest, S, n_layers)
    value_us = c_total * 1e3 / args.steps
    result = {
        "metric": METRIC,
        "value": round(value_us, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(c_total / args.steps, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded log-normal channel scales, 4 outlier key channels/head; no model weights)",
        "config": {"workload": "qwen3-8b-like-64k-decode", "n_seqs": 1, "kv_heads": Hkv, "q_heads": Hq,
                   "head_dim": D, "context": L0, "block_tokens": T, "group_tokens": 16, "n_splits": S,
                   "layers_rotated": n_layers, "layer_start_tokens": [L0 - LAYER_STAGGER * i for i in range(n_layers)]},
        "clean_step_us": {"compressed": c_clean, "uncompressed": r_clean,
                          "note": "value = mean of the clean pass; median/p10/p90 over its windows of one layer "
                                  "rotation each; host_wall_mean = host clock from the first enqueue to the end; "
                                  "prime = read-only attention passes over every layer cache before the warm-up"},
        "instrumented_step_us": {"median": float(np.median(c_step)), "p10": float(np.percentile(c_step, 10)),
                                 "p90": float(np.percentile(c_step, 90)),
                                 "note": "append, split attention and merge as separate calls, events between"},
        "attention_us": {"compressed": round(attn_c, 3), "uncompressed": round(attn_r, 3),
                         "method": "back-to-back launches over the rotated layers, events at the loop ends",
                         "in_step_compressed_median": float(np.median(c_attn)),
                         "in_step_uncompressed_median": float(np.median(r_attn))},
        "append_us": {"compressed_median": float(np.median(c_app)), "uncompressed_median": float(np.median(r_app)),
                      "block_encode_append": enc_us},
        "prefill_encode": {"tokens": L0, "compressed_us": round(bulk_c, 1), "uncompressed_us": round(bulk_r, 1),
                           "input_GBps": round(L0 * Hkv * D * 2 * 2 / (bulk_c * 1e-6) / 1e9, 1),
                           "note": "one kv_encode_append of the whole layer into an empty cache"},
        "combine_us": float(np.median(c_comb)),
        "host_enqueue_us_per_step": {"compressed": round(c_host, 2), "uncompressed": round(r_host, 2)},
        "uncompressed_step_us": round(r_total * 1e3 / args.steps, 3),
        "speedup_step": round(r_total / c_total, 4),
        "speedup_attention": round(attn_r / attn_c, 4),
        "effective_GBps": round(achieved, 1),
        "logical_GBps": round(bytes_r / (attn_c * 1e-6) / 1e9, 1),
        "uncompressed_GBps": round(bytes_r / (attn_r * 1e-6) / 1e9, 1),
        "uncompressed_streaming_bound": {
            "us": round(bound_r, 3), "GBps": attain_r["GBps"], "speedup_attention": round(bound_r / attn_c, 4),
            "note": "the uncompressed bytes read at the streaming probe's rate at the same launch shape and bytes "
                    "per wave: the time no uncompressed kernel of this launch shape beats, and the compressed "
                    "kernel's speedup against it"},
        "codec_ratio": round(codec_ratio, 4),
        "resident_ratio": round(resident_ratio, 4),
        "exponent_coverage": coverage,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": "attn_comp_kernel<4,64>", "bytes_per_launch": bytes_c,
                     "source_digest": digest, "attainable_GBps": attain["GBps"],
                     "frac_of_attainable": round(achieved / attain["GBps"], 4)},
        "attainable_read": attain,
        "sweep_attention_us": dict(sweep, note="the split kernel alone at other split counts (median of 32 "
                                   "cold launches, an event pair around each); 4, 8 and 16 splits = 256, 128 and "
                                   "64 blocks per split, the literal reading of 64-256 blocks per split") if sweep else None,
        "hbm_probe": probe,
    }
    extras = [x for x in args.extra.split(",") if x]
    if extras:
        del comp, raw
        torch.cuda.empty_cache()
    if "context" in extras:
        import dataclasses
        result["context_sweep"] = {
            f"{L // 1024}k": extra_steps(torch, K, synth, dataclasses.replace(cfg, context=(L,), name=f"qwen3-8b-like-{L // 1024}k"),
                                         args, splits=S)
            for L in (32768, 131072)}
    if "fp8" in extras:
        result["fp8_64k"] = {name: extra_steps(torch, K, synth, synth.config(4, fmt), args, splits=S)
                             for name, fmt in (("e5m2", synth.E5M2), ("e4m3", synth.E4M3))}
    if "g8" in extras:
        import dataclasses
        result["g8_64k"] = extra_steps(torch, K, synth, dataclasses.replace(cfg, G=8, name="qwen3-8b-like-64k-g8"),
                                       args, splits=S)
    if "paged" in extras:
        result["paged_mix"] = extra_steps(torch, K, synth, synth.config(3), args, splits=args.paged_splits, layers=2)
    if "groups" in extras:
        result["codec_groups_64k"] = codec_groups(torch, K, cfg, kd, vd, k0, v0, dev, stream, q, args.splits)
    if "nested" in extras:
        result["nested_modes_64k"] = nested_modes(torch, K, cfg, kd, vd, k0, v0, dev, stream, q, args.splits)
    if "rope" in extras:
        result["rope_drift_64k"] = rope_drift(torch, K, synth, cfg, k0, v0, dev)
    if "prefill" in extras:
        result["prefill_4k"] = prefill(torch, K, synth, cfg, k0, v0, dev, stream)
    if "d256" in extras:
        import dataclasses
        c256 = dataclasses.replace(cfg, name="qwen3-8b-like-32k-head-dim-256", D=256, context=(32768,))
        # 64 splits: the 256-channel kernel's per-workgroup set-up (both half-heads, LDS zeroing,
        # the query) favours longer splits than the register-rebuild kernel's 256
        result["head_dim_256_32k"] = extra_steps(torch, K, synth, c256, args, splits=64)
    if "serving" in extras:
        result["equal_memory_serving"] = equal_memory_serving(torch, K, synth, splits=args.paged_splits)
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(cfg, k0, v0)
    print(json.dumps(result), flush=True)


def codec_groups(torch, K, cfg, kd, vd, k0, v0, dev, stream, q, n_splits, reps=5):
    """The 64K layer's codec with 16- and 8-token exponent groups (GAAC page §3.1 groups eight
    values): codec ratio, mode shares and escape bytes per tile; one bulk append encoding all
    blocks; decoding every block back to BF16 (kv_decode_blocks) and a single block; decode
    attention over the layer (kv_attention_partials, back to back on the one layer, so its
    bytes sit in the last-level cache: "hot").  Encoders: 16-token groups the register-packing
    kernel, 8-token groups the bit-assembling one; decoders: the four-token SWAR decoders;
    attention: the register-rebuild split kernels (one for each group size)."""
    T, D, Hkv, Hq = cfg.T, cfg.D, cfg.Hkv, cfg.Hq
    L0 = kd.shape[1]
    nb = L0 // T
    TD = T * D

    def ev_us(fn):
        a_ = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        fn()
        b_.record(stream)
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) * 1e3

    res = {"workload": "qwen3-8b-like-64k", "tokens": L0, "block_tokens": T}
    for Gt in (16, 8):
        enc, dec_all, dec_one = [], [], []
        for _ in range(reps):
            c = K.KVCache(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T, max_seqs=1,
                          max_blocks_per_seq=nb + 1, num_comp_slots=(nb + 1) * 2 * Hkv, num_raw_slots=256,
                          compressed=True, group_tokens=Gt, perm_seed=7)
            c.calibrate(dev(k0[:cfg.n_cal]), dev(v0[:cfg.n_cal]))
            torch.cuda.synchronize()
            enc.append(ev_us(lambda: c.append([0], kd, vd)))
            kout = torch.empty((nb * T, Hkv, D), dtype=torch.int16, device="cuda")
            vout = torch.empty_like(kout)
            dec_all.append(ev_us(lambda: c.decode_blocks(0, 0, nb, (kout, vout))))
            k1 = torch.empty((T, Hkv, D), dtype=torch.int16, device="cuda")
            v1 = torch.empty_like(k1)
            dec_one.append(ev_us(lambda: c.decode_blocks(0, nb // 2, 1, (k1, v1))))
        if not (torch.equal(kout, kd[0, :nb * T]) and torch.equal(vout, vd[0, :nb * T])):
            raise RuntimeError(f"decode_blocks with {Gt}-token groups did not rebuild the layer bit for bit")
        ws = c.workspace(1, n_splits)
        for _ in range(3):
            c.attention_partials([0], q, cfg.scale, n_splits, ws)
        attn = ev_us(lambda: [c.attention_partials([0], q, cfg.scale, n_splits, ws) for _ in range(20)]) / 20
        flags, st = c.status()
        if flags:
            raise RuntimeError(f"cache status flags {flags}")
        payload = (2 * TD // Gt + 3 * TD + 8 * TD) // 8  # TAG + CODE + SM of a compressed tile
        stored = st["comp_tiles"] * payload + st["esc_bytes"] + st["raw_tiles"] * TD * 2
        tiles = st["comp_tiles"] + st["raw_tiles"]
        groups = st["groups"][:3]  # FORMAT v1: narrow, wide, raw
        res[f"g{Gt}"] = {
            "codec_ratio": round(tiles * TD * 2 / stored, 4),
            "resident_ratio": round(tiles * TD * 2 / (st["comp_tiles"] * c.slot_stride + st["raw_tiles"] * TD * 2 + 4 * tiles), 4),
            "mode_share": [round(x / max(sum(groups), 1), 5) for x in groups],
            "raw_tiles": st["raw_tiles"],
            "esc_bytes_per_tile": round(st["esc_bytes"] / max(st["comp_tiles"], 1), 1),
            "slot_stride": c.slot_stride,
            "bulk_encode_us": round(float(np.median(enc)), 1),
            "decode_all_blocks_us": round(float(np.median(dec_all)), 1),
            "decode_one_block_us": round(float(np.median(dec_one)), 1),
            "decode_GBps_out": round(tiles * TD * 2 / (float(np.median(dec_all)) * 1e-6) / 1e9, 1),
            "attention_hot_us": round(attn, 1),
        }
        del c
    log(f"[bench] codec groups: {res}")
    return res


def nested_modes(torch, K, cfg, kd, vd, k0, v0, dev, stream, q, n_splits, reps=3):
    """The nested precision modes of GAAC page §4.7.2 / Table 4 on the 64K layer: FORMAT v1
    (3-bit, 4-bit and raw modes; the tuned path) against FORMAT v2 with a 2-bit mode added, with
    the 3-bit mode removed, and with the v1 modes in the v2 layout (each group's offsets at its
    own width in one stream), for 16- and 8-token groups: codec and resident ratio, mode shares,
    one bulk encode of the layer, kv_decode_blocks of every block (the decode latency the page
    compares) and decode attention over the layer (hot, back to back)."""
    T, D, Hkv, Hq = cfg.T, cfg.D, cfg.Hkv, cfg.Hq
    L0 = kd.shape[1]
    nb = L0 // T
    TD = T * D

    def ev_us(fn):
        a_ = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        fn()
        b_.record(stream)
        torch.cuda.synchronize()
        return a_.elapsed_time(b_) * 1e3

    variants = [("v1_3_4_raw", 0), ("v2_2_3_4_raw", 1), ("v2_4_raw", 2), ("v2_3_4_raw", 3)]
    res = {"workload": "qwen3-8b-like-64k", "tokens": L0, "block_tokens": T}
    for Gt in (8, 16):
        row = {}
        for name, ms in variants:
            enc, dec = [], []
            for _ in range(reps):
                c = K.KVCache(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T, max_seqs=1,
                              max_blocks_per_seq=nb + 1, num_comp_slots=(nb + 1) * 2 * Hkv, num_raw_slots=(nb + 1) * 2 * Hkv,
                              compressed=True, group_tokens=Gt, perm_seed=7, mode_set=ms)
                c.calibrate(dev(k0[:cfg.n_cal]), dev(v0[:cfg.n_cal]))
                torch.cuda.synchronize()
                enc.append(ev_us(lambda: c.append([0], kd, vd)))
                kout = torch.empty((nb * T, Hkv, D), dtype=torch.int16, device="cuda")
                vout = torch.empty_like(kout)
                dec.append(ev_us(lambda: c.decode_blocks(0, 0, nb, (kout, vout))))
            if not (torch.equal(kout, kd[0, :nb * T]) and torch.equal(vout, vd[0, :nb * T])):
                raise RuntimeError(f"{name}, {Gt}-token groups: decode_blocks did not rebuild the layer bit for bit")
            ws = c.workspace(1, n_splits)
            for _ in range(2):
                c.attention_partials([0], q, cfg.scale, n_splits, ws)
            attn = ev_us(lambda: [c.attention_partials([0], q, cfg.scale, n_splits, ws) for _ in range(10)]) / 10
            flags, st = c.status()
            if flags:
                raise RuntimeError(f"cache status flags {flags}")
            n_tiles = st["comp_tiles"] + st["raw_tiles"]
            ng = TD // Gt
            if ms == 0:
                payload = (2 * ng + 3 * TD + 8 * TD) // 8
                stored = st["comp_tiles"] * payload + st["esc_bytes"] + st["raw_tiles"] * TD * 2
            else:  # TAG + SM + used code bytes
                stored = st["comp_tiles"] * ((2 * ng) // 8 + TD) + st["esc_bytes"] + st["raw_tiles"] * TD * 2
            groups = st["groups"]
            row[name] = {
                "codec_ratio": round(n_tiles * TD * 2 / stored, 4),
                "resident_ratio": round(n_tiles * TD * 2 / (st["comp_tiles"] * c.slot_stride + st["raw_tiles"] * TD * 2
                                                             + 4 * n_tiles), 4),
                "mode_share": [round(x / max(sum(groups), 1), 5) for x in groups],
                "raw_tiles": st["raw_tiles"], "slot_stride": c.slot_stride,
                "bulk_encode_us": round(float(np.median(enc)), 1),
                "decode_all_blocks_us": round(float(np.median(dec)), 1),
                "attention_hot_us": round(attn, 1),
            }
            del c
            torch.cuda.empty_cache()
        base, same_layout = row["v1_3_4_raw"], row["v2_3_4_raw"]
        for name in ("v2_2_3_4_raw", "v2_4_raw"):
            r = row[name]
            r["ratio_change_vs_v1_pct"] = round(100 * (r["codec_ratio"] / base["codec_ratio"] - 1), 2)
            r["decode_latency_vs_v1"] = round(r["decode_all_blocks_us"] / base["decode_all_blocks_us"], 2)
            r["decode_latency_vs_v2_3_4_raw"] = round(r["decode_all_blocks_us"] / same_layout["decode_all_blocks_us"], 2)
        res[f"g{Gt}"] = row
    log(f"[bench] nested modes: {res}")
    return res


def prefill(torch, K, synth, cfg, k0, v0, dev, stream, n=4096, reps=5):
    """Prefill of an n-token prompt over its decoded blocks (GAAC page §3.3): the bulk append
    that encodes every block, kv_decode_blocks rebuilding them, and causal prefill attention of
    all n queries over them (the 64K layer's geometry; queries from the same seeded generator
    as the decode steps)."""
    import dataclasses
    T, D, Hkv, Hq = cfg.T, cfg.D, cfg.Hkv, cfg.Hq
    nb = n // T
    c = K.KVCache(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T, max_seqs=1, max_blocks_per_seq=nb + 1,
                  num_comp_slots=(nb + 1) * 2 * Hkv, num_raw_slots=64, compressed=True, perm_seed=7)
    c.calibrate(dev(k0[:cfg.n_cal]), dev(v0[:cfg.n_cal]))
    kd, vd = dev(k0[None, :n]), dev(v0[None, :n])
    q = dev(synth.queries(dataclasses.replace(cfg, n_seqs=n)))
    kout = torch.empty((n, Hkv, D), dtype=torch.int16, device="cuda")
    vout = torch.empty_like(kout)
    out = torch.empty((n, Hq, D), dtype=torch.int16, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)
    enc, dec, att = [], [], []
    for r in range(reps):
        c.release(0) if r else None
        e0, e1, e2, e3 = ev(), ev(), ev(), ev()
        e0.record(stream)
        c.append([0], kd, vd)
        e1.record(stream)
        c.decode_blocks(0, 0, nb, (kout, vout))
        e2.record(stream)
        c.prefill_attention(kout, vout, q, cfg.scale, out)
        e3.record(stream)
        torch.cuda.synchronize()
        enc.append(e0.elapsed_time(e1) * 1e3)
        dec.append(e1.elapsed_time(e2) * 1e3)
        att.append(e2.elapsed_time(e3) * 1e3)
    if not (torch.equal(kout, kd[0]) and torch.equal(vout, vd[0])):
        raise RuntimeError("decode_blocks did not rebuild the prompt bit for bit")
    flops = 4.0 * Hq * D * (n * (n + 1) / 2)  # QK and PV over the causal pairs
    a_us = float(np.median(att))
    res = {"workload": f"qwen3-8b-like-prefill-{n}", "tokens": n, "encode_us": round(float(np.median(enc)), 1),
           "decode_blocks_us": round(float(np.median(dec)), 1), "prefill_attention_us": round(a_us, 1),
           "prefill_attention_TFLOPs": round(flops / (a_us * 1e-6) / 1e12, 2)}
    log(f"[bench] prefill: {res}")
    return res


def rope_drift(torch, K, synth, cfg, k0, v0, dev, seg=8192):
    """RoPE positional drift (GAAC page App. C): the 64K layer with keys rotated by rotary
    position embedding (theta = 1e6), encoded once per calibration policy; per 8K-token segment,
    the mean escape bytes of the compressed K and V tiles (from their stored tag planes) and the
    share of tiles stored raw.  Policies: unrotated keys, first 256 tokens; rotated keys
    calibrated on the first 256, 8K or 32K tokens, or on 256 tokens spread evenly over the
    context (same calibration budget as the first, spread over the positions); and a live cache
    recalibrated (kv_recalibrate) before each 16K-token chunk on the 256 tokens just before it.
    The per-tile figures come from kv_tile_stats (read on the device from the stored tag planes
    and table entries)."""
    T, D, Hkv, Hq = cfg.T, cfg.D, cfg.Hkv, cfg.Hq
    L0 = k0.shape[0]
    nb = L0 // T
    kr = synth.rope_keys(k0)
    policies = [("unrotated_first256", k0, np.arange(256)), ("first256", kr, np.arange(256)),
                ("first8k", kr, np.arange(8192)), ("first32k", kr, np.arange(32768)),
                ("spread256", kr, np.arange(0, L0, L0 // 256))]
    res = {"workload": "qwen3-8b-like-64k, RoPE theta 1e6 on K", "segment_tokens": seg, "block_tokens": T}
    def summary(c):
        stats = c.tile_stats(0, 0, nb)            # kv_tile_stats: [nb][2][Hkv][7] {state, escape bytes, modes, version}
        raw = stats[..., 0] == 1
        esc = stats[..., 1].double()
        segs = []
        for s0 in range(0, nb, seg // T):
            row = {}
            for kv, nm in ((0, "k"), (1, "v")):
                r = raw[s0:s0 + seg // T, kv]
                n_comp = int((~r).sum())
                row[f"{nm}_esc_bytes_per_tile"] = round(float(esc[s0:s0 + seg // T, kv].sum()) / max(n_comp, 1), 1)
                row[f"{nm}_raw_tile_share"] = round(float(r.double().mean()), 4)
            row["base_versions"] = sorted({int(x) for x in stats[s0:s0 + seg // T, ..., 6].flatten().tolist() if x >= 0})
            segs.append(row)
        flags, st = c.status()
        return {"segments": segs, "raw_tiles": st["raw_tiles"], "status_flags": flags}

    def new_cache(versions=1):
        return K.KVCache(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T, max_seqs=1,
                         max_blocks_per_seq=nb + 1, num_comp_slots=(nb + 1) * 2 * Hkv,
                         num_raw_slots=(nb + 1) * 2 * Hkv, compressed=True, perm_seed=7, base_versions=versions)

    for name, ks, cal in policies:
        c = new_cache()
        c.calibrate(dev(ks[cal]), dev(v0[cal]))
        c.append([0], dev(ks[None]), dev(v0[None]))
        res[name] = summary(c)
        del c
    # live recalibration (kv_recalibrate): calibrated on the first 256 tokens; before each further
    # 16K-token chunk is appended, a new base version from the 256 tokens just before it (four
    # versions in all); stored blocks keep the version they were encoded with
    chunk = 16384
    c = new_cache(versions=4)
    c.calibrate(dev(kr[:256]), dev(v0[:256]))
    for s0 in range(0, L0, chunk):
        if s0 > 0:
            c.recalibrate(dev(kr[s0 - 256:s0]), dev(v0[s0 - 256:s0]))
        c.append([0], dev(kr[None, s0:s0 + chunk]), dev(v0[None, s0:s0 + chunk]))
    res["live_recalibration_every_16k"] = summary(c)
    del c
    log(f"[bench] rope drift: {res}")
    return res


def equal_memory_serving(torch, K, synth, splits, budget_mb=1536, n_requests=96, layers=4, steps=24):
    """Equal-memory serving (GAAC page §4.5): one KV byte budget per layer for both caches,
    planned and admitted by kv_admit_fcfs (the compressed cache spends 1/64 of it on raw-fallback
    slots and the rest on compressed slots, the uncompressed one all of it on raw tiles; requests
    with paged-mix lengths, T = 16, U[4096, 32768] tokens, seeded, are admitted first come, first
    served while their finished blocks plus one spare block fit in the free slots); then the
    admitted batch decodes (kv_decode_step over every admitted sequence) on `layers` rotated layer
    caches.  Sequences take their tokens from one shared token stream at staggered offsets.  No
    model weights exist here: a step is the attention layer alone, so the throughput is
    attention-only."""
    import dataclasses
    cfg = synth.config(3)
    T, D, Hkv, Hq = cfg.T, cfg.D, cfg.Hkv, cfg.Hq
    lens = np.random.default_rng([3, 4242]).integers(4096, 32768, size=n_requests, endpoint=True).tolist()
    budget = budget_mb << 20
    g = synth.LayerGen(cfg)
    pk_h, pv_h = g.tokens(max(lens) + 4096)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    pk, pv = dev(pk_h), dev(pv_h)
    stream = torch.cuda.current_stream()
    res = {"workload": "paged-mix requests, T = 16, 8/32 heads, D = 128", "budget_bytes_per_layer": budget,
           "requests": n_requests, "n_splits": splits, "layers_rotated": layers, "steps": steps,
           "admission": "kv_admit_fcfs"}

    for name, compressed in (("uncompressed", False), ("compressed", True)):
        n, n_comp, n_raw = K.admit_fcfs(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T,
                                        budget_bytes=budget, lengths=lens, compressed=compressed, raw_share=1.0 / 64)
        admitted = lens[:n]
        n = len(admitted)
        ids = list(range(n))
        max_blocks = max(admitted) // T + 2
        caches = []
        for li in range(layers):
            c = K.KVCache(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T, max_seqs=n,
                          max_blocks_per_seq=max_blocks, num_comp_slots=n_comp, num_raw_slots=n_raw,
                          compressed=compressed, perm_seed=13 + li)
            c.calibrate(pk[:256], pv[:256])
            for sid, L in enumerate(admitted):
                off = (997 * (sid + 7 * li)) % 4096
                c.append([sid], pk[None, off:off + L], pv[None, off:off + L])
            caches.append(c)
        torch.cuda.synchronize()
        flags, st = caches[0].status()
        if flags:
            raise RuntimeError(f"equal-memory serving ({name}): cache status flags {flags}")
        q = dev(synth.queries(dataclasses.replace(cfg, n_seqs=n)))
        out = torch.empty((n, Hq, D), dtype=torch.int16, device="cuda")
        ws = caches[0].workspace(n, splits)
        for i in range(4):  # warm-up
            caches[i % layers].decode_step(ids, pk[i * n:(i + 1) * n], pv[i * n:(i + 1) * n], q, cfg.scale, splits, ws, out)
        torch.cuda.synchronize()
        a_ = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        a_.record(stream)
        for i in range(4, 4 + steps):
            caches[i % layers].decode_step(ids, pk[i * n:(i + 1) * n], pv[i * n:(i + 1) * n], q, cfg.scale, splits, ws, out)
        b_.record(stream)
        torch.cuda.synchronize()
        step_us = a_.elapsed_time(b_) * 1e3 / steps
        flags, st = caches[0].status()
        if flags:
            raise RuntimeError(f"equal-memory serving ({name}): cache status flags {flags} after the steps")
        res[name] = {"admitted": n, "context_tokens": sum(admitted), "comp_slots": n_comp, "raw_slots": n_raw,
                     "raw_fallback_tiles": st["raw_tiles"] if compressed else None,
                     "step_us_per_layer": round(step_us, 1),
                     "decode_tokens_per_s_per_layer": round(n / (step_us * 1e-6), 1)}
        del caches, ws, out, q
        torch.cuda.empty_cache()
    res["admitted_ratio"] = round(res["compressed"]["admitted"] / res["uncompressed"]["admitted"], 4)
    res["context_tokens_ratio"] = round(res["compressed"]["context_tokens"] / res["uncompressed"]["context_tokens"], 4)
    res["throughput_ratio"] = round(res["compressed"]["decode_tokens_per_s_per_layer"] /
                                    res["uncompressed"]["decode_tokens_per_s_per_layer"], 4)
    log(f"[bench] equal-memory serving: {res}")
    return res


def extra_steps(torch, K, synth, cfg, args, splits, layers=4):
    """Decode steps of another workload: every step appends one token to each sequence and runs
    split attention plus the merge over all sequences, on `layers` rotated layer caches;
    compressed and uncompressed caches timed the same way.  Returns per-kernel and per-step
    medians, the codec ratio and the attention speedup.  Sequences of the paged mix take their
    tokens from one 32K-token stream (prefixes of it), which keeps input generation short."""
    T, D, Hkv, Hq, B = cfg.T, cfg.D, cfg.Hkv, cfg.Hq, cfg.n_seqs
    fmt = cfg.fmt
    lens = list(cfg.context)
    g = synth.LayerGen(cfg)
    pool_k, pool_v = g.tokens(max(lens))
    if fmt == synth.BF16:
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    else:
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.uint8)).cuda()
    steps = args.extra_steps
    warm = 4
    per_layer = (2 * steps + warm + layers - 1) // layers + 1
    kn, vn = g.tokens(per_layer * layers * B)
    k_new = dev(kn.reshape(layers, per_layer, B, 1, Hkv, D))
    v_new = dev(vn.reshape(layers, per_layer, B, 1, Hkv, D))
    q = dev(synth.queries(cfg)) if fmt == synth.BF16 else \
        torch.from_numpy(np.ascontiguousarray(synth.queries(cfg)).view(np.int16)).cuda()
    max_blocks = (max(lens) + per_layer) // T + 2
    n_tiles = B * max_blocks * 2 * Hkv * (2 if D == 256 else 1)  # 256-channel heads: two half-head tiles
    ids = list(range(B))
    log(f"[bench] {cfg.name}: building {layers} compressed + {layers} uncompressed layers ({sum(lens)} tokens each)")

    def make(compressed):
        c = K.KVCache(num_kv_heads=Hkv, num_q_heads=Hq, head_dim=D, block_tokens=T, max_seqs=B,
                      max_blocks_per_seq=max_blocks, num_comp_slots=n_tiles if compressed else 0,
                      num_raw_slots=1024 if compressed else n_tiles, compressed=compressed, perm_seed=11, dtype=fmt,
                      group_tokens=cfg.G)
        c.calibrate(dev(pool_k[:cfg.n_cal]), dev(pool_v[:cfg.n_cal]))
        for sid, L in enumerate(lens):
            c.append([sid], dev(pool_k[None, :L]), dev(pool_v[None, :L]))
        return c

    out = torch.empty((B, Hq, D), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    res = {"workload": cfg.name, "n_seqs": B, "tokens": sum(lens), "block_tokens": T, "n_splits": splits,
           "layers_rotated": layers, "steps": steps}
    for name, compressed in (("compressed", True), ("uncompressed", False)):
        caches = [make(compressed) for _ in range(layers)]
        ws = caches[0].workspace(B, splits)
        torch.cuda.synchronize()
        if compressed:
            flags, st = caches[0].status()
            Dt = min(D, 128)  # channels of a stored tile (a 256-channel head is two half-head tiles)
            n_grp = T * Dt // cfg.G
            mb = {synth.BF16: 7, synth.E5M2: 2, synth.E4M3: 3}[fmt]
            eb = 2 if fmt == synth.BF16 else 1
            payload = (2 * n_grp + 3 * T * Dt + (1 + mb) * T * Dt) // 8
            comp_bytes = st["comp_tiles"] * payload + st["esc_bytes"] + st["raw_tiles"] * T * Dt * eb
            res["codec_ratio"] = round((st["comp_tiles"] + st["raw_tiles"]) * T * Dt * eb / comp_bytes, 4)
            res["compressed_kv_bytes"] = comp_bytes
        ev = []
        for i in range(warm + steps):
            li, pos = i % layers, i // layers
            c = caches[li]
            e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            e[0].record(stream)
            c.append(ids, k_new[li, pos], v_new[li, pos])
            e[1].record(stream)
            c.attention_partials(ids, q, cfg.scale, splits, ws)
            e[2].record(stream)
            c.attention_combine(ids, q, cfg.scale, splits, ws, out)
            e[3].record(stream)
            if i >= warm:
                ev.append(e)
        torch.cuda.synchronize()
        # the product's decode step (kv_decode_step), back to back, events at the loop ends
        a_ = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        base = warm + steps
        a_.record(stream)
        for i in range(steps):
            li, pos = (base + i) % layers, (base + i) // layers
            caches[li].decode_step(ids, k_new[li, pos], v_new[li, pos], q, cfg.scale, splits, ws, out)
        b_.record(stream)
        torch.cuda.synchronize()
        step_clean = a_.elapsed_time(b_) * 1e3 / steps
        med = lambda a, b: float(np.median([x[a].elapsed_time(x[b]) * 1e3 for x in ev]))
        # the attention kernel alone, back to back over the rotated layers (events at the ends)
        a_ = torch.cuda.Event(enable_timing=True)
        b_ = torch.cuda.Event(enable_timing=True)
        reps = 8 * layers
        a_.record(stream)
        for i in range(reps):
            caches[i % layers].attention_partials(ids, q, cfg.scale, splits, ws)
        b_.record(stream)
        torch.cuda.synchronize()
        res[name] = {"attention_us": round(a_.elapsed_time(b_) * 1e3 / reps, 2), "step_us": round(step_clean, 2),
                     "in_step_attention_us": round(med(1, 2), 2), "append_us": round(med(0, 1), 2),
                     "combine_us": round(med(2, 3), 2), "unfused_step_us": round(med(0, 3), 2)}
        del caches, ws
        torch.cuda.empty_cache()
    res["speedup_attention"] = round(res["uncompressed"]["attention_us"] / res["compressed"]["attention_us"], 4)
    res["speedup_step"] = round(res["uncompressed"]["step_us"] / res["compressed"]["step_us"], 4)
    res["effective_GBps"] = round(res["compressed_kv_bytes"] / (res["compressed"]["attention_us"] * 1e-6) / 1e9, 1)
    log(f"[bench] {cfg.name}: {res}")
    return res


def kernel_source_digest():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(digest, splits, layers):
    """HBM bytes per launch of the compressed attention kernel as the FETCH_SIZE + WRITE_SIZE
    counters read them (scaled by the same counters' reading for a copy kernel of known size),
    from the committed counter summary -- or None when that summary was taken on other kernel
    sources or another launch shape."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        m = re.match(r"^\s*[-*]?\s*`?(\w+)`?\s*:\s*`?([\w.]+)`?", line)
        if m:
            kv[m.group(1)] = m.group(2)
    try:
        if kv.get("source_digest") != digest or int(kv["n_splits"]) != splits or int(kv["layers_rotated"]) != layers:
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attainable_read(torch, K, stream, nbytes, waves=2048, n_buf=8, reps=48):
    """The library's streaming-read kernel (kv_read_probe) at the split attention kernel's launch
    shape -- `waves` workgroups of one wave, here one per wave slot of the chip -- reading about
    nbytes per launch, rotated over n_buf buffers so every launch reads from HBM: the read rate
    this launch shape attains on the GPU at hand, beside the 8 TB/s peak.  Each wave reads an odd
    number of 8 KiB pieces, so the waves' start addresses do not all share one power-of-two
    alignment (and with it one memory channel)."""
    k = max(1, int(round(nbytes / waves / 8192)))
    per = 8192 * (k + 1 - k % 2)
    bufs = [torch.zeros(waves * per // 4, dtype=torch.int32, device="cuda") for _ in range(n_buf)]
    sink = torch.empty((waves, 64), dtype=torch.int32, device="cuda")
    for i in range(2 * n_buf):
        K.read_probe(bufs[i % n_buf], per, waves, sink)
    torch.cuda.synchronize()
    a_ = torch.cuda.Event(enable_timing=True)
    b_ = torch.cuda.Event(enable_timing=True)
    a_.record(stream)
    for i in range(reps):
        K.read_probe(bufs[i % n_buf], per, waves, sink)
    b_.record(stream)
    torch.cuda.synchronize()
    us = a_.elapsed_time(b_) * 1e3 / reps
    out = {"GBps": round(waves * per / (us * 1e-6) / 1e9, 1), "us": round(us, 3), "bytes_per_launch": waves * per,
           "waves": waves, "bytes_per_wave": per, "buffers_rotated": n_buf,
           "method": "kv_read_probe launched back to back, events at the loop ends"}
    log(f"[bench] attainable read: {out}")
    del bufs, sink
    torch.cuda.empty_cache()
    return out


def hbm_probe(torch, stream, nbytes=2 << 30, reps=10):
    """Plain streaming kernels of known size on the same GPU: a device copy (reads and writes
    nbytes) and a read-only reduction over nbytes.  Their rates bound what any HBM-bound kernel
    can reach here, and the copy is the reference for scaling FETCH_SIZE/WRITE_SIZE counters."""
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    out = {}
    for name, fn, moved in (("copy", lambda: dst.copy_(src), 2 * nbytes),
                            ("read", lambda: src.sum(dtype=torch.float32), nbytes)):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a_ = torch.cuda.Event(enable_timing=True)
            b_ = torch.cuda.Event(enable_timing=True)
            a_.record(stream)
            fn()
            b_.record(stream)
            ts.append((a_, b_))
        torch.cuda.synchronize()
        us = float(np.median([a_.elapsed_time(b_) * 1e3 for a_, b_ in ts]))
        out[name] = {"us": us, "bytes": moved, "GBps": round(moved / (us * 1e-6) / 1e9, 1)}
    log(f"[bench] hbm probe: {out}")
    del src, dst
    return out


def cpu_baseline(cfg, k0, v0, min_seconds=10.0):
    """The oracle as it stands, on the host.  value: one full decode step -- rebuild every tile of
    the layer from its stored form and evaluate exact fp64 attention for all 32 query heads --
    repeated for about min_seconds on all threads.  Also: the same step on one thread, the encode
    of the whole layer cache on all threads and on one, the tiny layer end to end, and one step
    each of the FP8 layer and of the paged serving mix."""
    import oracle
    import synth
    p = oracle.Params(oracle.BF16, cfg.T, cfg.D, cfg.G)
    threads = oracle._threads(None)
    log(f"[bench] cpu baseline: oracle encode, decode and fp64 attention on {threads} threads and on one")
    bases = oracle.calibrate_layer(p, k0[:cfg.n_cal], v0[:cfg.n_cal])
    enc_s = {}
    for nt in (threads, 1):  # encode of the whole layer cache (16,384 tiles), all threads then one
        s = oracle.Sequence(p, cfg.Hkv, bases)
        t0 = time.perf_counter()
        s.append(k0, v0, nthreads=nt)
        enc_s[nt] = time.perf_counter() - t0
    q = synth.queries(cfg)[0]
    # Repeat whole steps until about min_seconds of wall time have passed (at least 2 steps), so
    # that the figure does not hinge on one short run; report the mean per step.
    reps, t_dec, t_att = 0, 0.0, 0.0
    while reps < 2 or t_dec + t_att < min_seconds:
        t0 = time.perf_counter()
        kd, vd = s.decoded()
        t1 = time.perf_counter()
        oracle.attention(oracle.BF16, q, kd, vd, cfg.scale)
        t2 = time.perf_counter()
        t_dec += t1 - t0
        t_att += t2 - t1
        reps += 1
        del kd, vd
    # the same step once on a single thread
    t0 = time.perf_counter()
    kd, vd = s.decoded(nthreads=1)
    t1 = time.perf_counter()
    oracle.attention(oracle.BF16, q, kd, vd, cfg.scale, nthreads=1)
    t2 = time.perf_counter()
    del kd, vd
    single = {"us_per_step": round((t2 - t0) * 1e6, 1), "decode_s": round(t1 - t0, 3), "attention_s": round(t2 - t1, 3)}
    # the tiny two-head, 1,024-token layer end to end: calibrate, encode, rebuild, fp64 attention
    c0 = synth.config(0)
    _, toks0 = synth.sequence_tokens(c0)
    tk, tv = toks0[0]
    p0 = oracle.Params(oracle.BF16, c0.T, c0.D, c0.G)
    t0 = time.perf_counter()
    s0 = oracle.Sequence(p0, c0.Hkv, oracle.calibrate_layer(p0, tk[:c0.n_cal], tv[:c0.n_cal]))
    s0.append(tk, tv)
    k_, v_ = s0.decoded()
    oracle.attention(oracle.BF16, synth.queries(c0)[0], k_, v_, c0.scale)
    tiny_us = (time.perf_counter() - t0) * 1e6
    # one step of the FP8 E5M2 64K layer and one of the 32-sequence paged mix, all threads
    # (encode untimed: the cache is built first, as on the GPU)
    other = {}
    c4 = synth.config(4, synth.E5M2)
    _, toks4 = synth.sequence_tokens(c4)
    k4, v4 = toks4[0]
    p4 = oracle.Params(c4.fmt, c4.T, c4.D, c4.G)
    s4 = oracle.Sequence(p4, c4.Hkv, oracle.calibrate_layer(p4, k4[:c4.n_cal], v4[:c4.n_cal]))
    s4.append(k4, v4)
    t0 = time.perf_counter()
    k_, v_ = s4.decoded()
    oracle.attention(c4.fmt, synth.queries(c4)[0], k_, v_, c4.scale)
    other[c4.name + "-e5m2"] = {"us_per_step": round((time.perf_counter() - t0) * 1e6, 1),
                                "what": "rebuild all 16384 FP8 tiles + fp64 attention, 32 query heads"}
    del s4, k_, v_, toks4, k4, v4
    c3 = synth.config(3)
    _, toks3 = synth.sequence_tokens(c3)
    p3 = oracle.Params(oracle.BF16, c3.T, c3.D, c3.G)
    b3_ = oracle.calibrate_layer(p3, toks3[0][0][:c3.n_cal], toks3[0][1][:c3.n_cal])
    seqs3 = []
    for kk, vv in toks3:
        sq = oracle.Sequence(p3, c3.Hkv, b3_)
        sq.append(kk, vv)
        seqs3.append(sq)
    q3 = synth.queries(c3)
    t0 = time.perf_counter()
    for si, sq in enumerate(seqs3):
        k_, v_ = sq.decoded()
        oracle.attention(oracle.BF16, q3[si], k_, v_, c3.scale)
    other[c3.name] = {"us_per_step": round((time.perf_counter() - t0) * 1e6, 1),
                      "what": f"32 sequences, {sum(len(t[0]) for t in toks3)} tokens: rebuild every tile + fp64 attention"}
    del seqs3, toks3
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": round((t_dec + t_att) / reps * 1e6, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full decode steps of the 64K layer, each: rebuild all {len(s.tiles) * 2 * cfg.Hkv} "
                      f"tiles from their stored bytes ({t_dec / reps:.3f} s) + exact fp64 attention for all "
                      f"{cfg.Hq} query heads ({t_att / reps:.3f} s); {t_dec + t_att:.1f} s in total",
            "cpu_model": cpu_model, "nproc": os.cpu_count(), "single_thread": single,
            "encode_layer_s": {"threads": threads, "all_threads": round(enc_s[threads], 3), "one_thread": round(enc_s[1], 3),
                               "tiles": len(s.tiles) * 2 * cfg.Hkv},
            "tiny_layer_end_to_end_us": {"value": round(tiny_us, 1),
                                         "what": f"{c0.name}: calibrate, encode, rebuild and fp64 attention, {threads} threads"},
            "other_steps": other}


if __name__ == "__main__":
    main()
