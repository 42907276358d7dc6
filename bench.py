"""Decompression throughput of the 8B-shaped BF16 weight set on one MI355X.

One step = one batched decode (a single kernel launch) of all 226 compressed
tensors of the set (32 Llama-3-8B-shaped layers + embedding + LM head,
8,029,995,008 values, 16.06 GB of BF16 out), with the compressed streams
already resident in HBM: every weight is streamed once per step, as in
single-stream inference. The streams are made once, before timing, by the
GPU encoder (encode throughput is reported too), and the decoded outputs are
checked bit-exactly against the inputs after the timed region.

Printed as ONE JSON line: metric/value (BF16-out GB/s), roofline of the
decode kernel (algorithmic HBM bytes per launch / launch time vs 8 TB/s),
compression ratio, the measured device copy ceiling, the fused
decompress-GEMM against the same GEMM on uncompressed weights, and the CPU
oracle timed on a bounded sample on this host.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_DENSE_PEAK_TFLOPS = 2500.0
METRIC = "decompress GB/s (BF16 out) + % of HBM roofline; compression ratio"
CSRC = os.path.join(ROOT, "lossless_weight_compression_amd", "csrc")
DECODE_SRCS = [os.path.join(CSRC, f) for f in ("decode.hip", "group_math.h", "enc_common.h")]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "decode_batch_set8b_pmc.json")
# rotating weight copies in the GEMM timing: 8 x 88.5 MB compressed (8 x 117 MB
# dense) is well past the 256 MB last-level cache, so every call reads HBM
GEMM_COPIES = 8


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--block-size", type=int, default=512)
    p.add_argument("--layers", type=int, default=32,
                   help="decoder layers in the set (32 = the full 8B shape)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--gemm-only", action="store_true",
                   help="only the fused-GEMM measurement (for profiling runs): both layouts, "
                        "then a 1 GiB device copy of known size for counter calibration")
    p.add_argument("--gemm-m", default="1,2,4,8,16,32,64,128,256",
                   help="comma-separated M values of the [K, N] GEMM sweep")
    p.add_argument("--gemm-nt-m", default="1,16,128",
                   help="comma-separated M values of the [N, K] (linear-layer) GEMM")
    p.add_argument("--gemm-b", type=int, default=512,
                   help="block size of the compressed W in both GEMM measurements")
    p.add_argument("--no-gemm", action="store_true")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the other configurations (tiny, layer sweep, stress)")
    p.add_argument("--no-wide", action="store_true",
                   help="skip the FP16 / FP32 measurement")
    p.add_argument("--wide-layers", type=int, default=4,
                   help="layers of the set measured as FP16 and FP32")
    p.add_argument("--no-pow2", action="store_true",
                   help="skip the power-of-two-width variant of the decode step")
    p.add_argument("--cpu-layers", type=int, default=4,
                   help="layers of the set the CPU oracle encodes and decodes on all host "
                        "threads (bounded sample)")
    p.add_argument("--cpu-layers-1t", type=int, default=1,
                   help="layers of the set the CPU oracle encodes and decodes on one thread")
    return p.parse_args()


def source_hash(paths):
    """Hash of the code in the given C++ sources: line comments, trailing
    blanks and empty lines are left out, so a change to a comment does not
    retire a profile taken on the same code (the sources hold no '//' inside
    string literals and no block comments)."""
    h = hashlib.sha256()
    for p in paths:
        for line in open(p, encoding="utf-8").read().splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def traffic_from_profile(n_launch_bytes):
    """HBM bytes per decode launch from the committed rocprofv3 PMC summary,
    if it was taken on the current decode kernel source; else None."""
    try:
        d = json.load(open(PMC_SUMMARY))
    except (OSError, ValueError):
        return None
    if d.get("decode_source_sha256_16") != source_hash(DECODE_SRCS):
        return None
    return d.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the decode shards by tensor or by segment with no communication)",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from lossless_weight_compression_amd import enc, synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream()
    B = args.block_size

    if args.gemm_only:
        g = bench_gemm(enc, synth, torch, np, dev, stream, args.gemm_m, args.gemm_b)
        gnt = bench_gemm_nt(enc, synth, torch, np, dev, args.gemm_nt_m, args.gemm_b)
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)                       # calibration: 1 GiB read, 1 GiB written
        torch.cuda.synchronize()
        print(json.dumps({"metric": "fused decompress-GEMM us per call", "fused_gemm": g,
                          "fused_gemm_nt": gnt, "gemm_roofline": gemm_roofline(g, gnt, args.gemm_b)}),
              flush=True)
        return

    shapes = synth.set8b_shapes()
    if args.layers != 32:
        keep = ["L%d." % l for l in range(args.layers)]
        idx = [i for i, (nm, _, _) in enumerate(shapes)
               if any(nm.startswith(k) for k in keep) or nm in ("embed", "lm_head")]
    else:
        idx = list(range(len(shapes)))

    # ---- compress once (GPU encoder), timing each call ----------------------
    # The inputs stay resident (16 GB for the full set) for the batched
    # encoder, the power-of-two variant and the final bit-exact check.
    xs = [synth.set8b_tensor_gpu(i, device=dev) for i in idx]
    streams, enc_ms, n_total, comp_total = [], 0.0, 0, 0
    algo_read = 0
    ws_cache = {}
    warmed = set()
    for k, i in enumerate(idx):
        x = xs[k]
        n = x.numel()
        out = torch.empty(enc.enc_compress_bound(n), dtype=torch.uint8, device=dev)
        wsb = enc.enc_compress_workspace_bytes(n, B)
        ws = ws_cache.get(wsb)
        if ws is None:
            ws = ws_cache[wsb] = torch.empty(wsb, dtype=torch.uint8, device=dev)
        if n not in warmed:   # first call of each shape untimed (code loading, allocations)
            enc.enc_compress(x, B, out=out, ws=ws)
            warmed.add(n)
        # A fresh allocation's memory is cleared by the driver before its
        # first use; fill it here so that the clear is not charged to the call.
        out.fill_(0)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        comp, info = enc.enc_compress(x, B, out=out, ws=ws)   # synchronises once inside
        torch.cuda.synchronize()
        enc_ms += (time.perf_counter() - t0) * 1e3
        streams.append((comp.clone(), info))
        n_total += n
        comp_total += info.total_bytes
        if info.flags == 1:
            algo_read += 2 * n
        else:
            algo_read += n + 2 * info.n_blocks + 8 * info.n_segments + info.payload_bytes
        del x, out, comp
    ws_cache.clear()
    torch.cuda.empty_cache()
    ratio = 2 * n_total / comp_total
    log("compressed %d tensors, %d values, ratio %.4f, encode %.1f ms"
        % (len(idx), n_total, ratio, enc_ms))

    # ---- the whole set through one batched encoder call ----------------------
    b_outs = [torch.empty(enc.enc_compress_bound(x.numel()), dtype=torch.uint8, device=dev)
              for x in xs]
    b_ws = torch.empty(enc.enc_compress_batch_workspace_bytes(xs, B), dtype=torch.uint8,
                       device=dev)
    enc.enc_compress_batch(xs, B, outs=b_outs, ws=b_ws)        # warm-up
    b_ms = []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        b_res = enc.enc_compress_batch(xs, B, outs=b_outs, ws=b_ws)   # synchronises inside
        torch.cuda.synchronize()
        b_ms.append((time.perf_counter() - t0) * 1e3)
    enc_batch_ms = float(np.median(b_ms))
    for (c, inf), (bc, binf) in zip(streams, b_res):
        if bytes(inf) != bytes(binf) or not torch.equal(c, bc):
            log("MISMATCH between batched and per-tensor encoder streams")
            sys.exit(1)
    log("batched encode: %.2f ms for the set (streams identical to per-tensor calls)"
        % enc_batch_ms)
    del b_outs, b_ws, b_res
    torch.cuda.empty_cache()

    # ---- batched decode: one launch per step ---------------------------------
    outs = [torch.empty(streams[k][1].n_elems, dtype=torch.int16, device=dev)
            for k in range(len(idx))]
    table = enc.enc_batch_prepare([(c, inf, o) for (c, inf), o in zip(streams, outs)])
    count = len(idx)
    for _ in range(args.warmup):
        enc.enc_decompress_batch(table, count)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        starts[k].record(stream)
        enc.enc_decompress_batch(table, count)
        ends[k].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_launch_ms = float(np.mean(launch_ms))
    step_ms = max(wall_ms, avg_launch_ms)
    out_bytes = 2 * n_total
    launch_bytes = algo_read + out_bytes
    value = out_bytes / (step_ms * 1e-3) / 1e9
    achieved = launch_bytes / (avg_launch_ms * 1e-3) / 1e9
    log("decode: %.3f ms/step (launch avg %.3f, min %.3f), %.1f GB/s out, %.1f GB/s HBM"
        % (step_ms, avg_launch_ms, min(launch_ms), value, achieved))

    # ---- correctness of what was timed, before anything else writes `outs` --
    def check_outs(what):
        for k, i in enumerate(idx):
            if not torch.equal(outs[k], xs[k].reshape(-1)):
                log("MISMATCH in tensor %s (%s)" % (shapes[i][0], what))
                sys.exit(1)

    def poison_outs():
        for o in outs:
            o.fill_(0x5A5A)

    check_outs("timed batched decode")
    log("timed batched decode: all %d outputs bit-exact" % len(outs))

    # ---- the same step as one launch per tensor (context, not the headline) ----
    poison_outs()
    pt_ms = []
    for _ in range(max(args.steps // 4, 2)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for (c, inf), o in zip(streams, outs):
            enc.enc_decompress(c, inf, out=o)
        e1.record(stream)
        torch.cuda.synchronize()
        pt_ms.append(e0.elapsed_time(e1))
    per_tensor_ms = float(np.median(pt_ms))
    check_outs("per-tensor decode")
    log("per-tensor launches: %.3f ms/step, bit-exact" % per_tensor_ms)

    # ---- variant: power-of-two widths (stream flag 2), same tensors ---------
    pow2 = None
    if not args.no_pow2:
        p2_streams, p2_total = [], 0
        for x in xs:
            c, inf = enc.enc_compress(x, B, pow2_widths=True)
            p2_streams.append((c.clone(), inf))
            p2_total += inf.total_bytes
            del c
        p2_read = sum((2 * inf.n_elems if inf.flags == 1 else
                       inf.n_elems + 2 * inf.n_blocks + 8 * inf.n_segments + inf.payload_bytes)
                      for _, inf in p2_streams)
        p2_table = enc.enc_batch_prepare([(c, inf, o) for (c, inf), o in zip(p2_streams, outs)])
        poison_outs()
        for _ in range(args.warmup):
            enc.enc_decompress_batch(p2_table, count)
        ms = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            enc.enc_decompress_batch(p2_table, count)
            e1.record(stream)
            ms.append((e0, e1))
        torch.cuda.synchronize()
        p2_ms = float(np.mean([a.elapsed_time(b) for a, b in ms]))
        check_outs("power-of-two-width decode")
        pow2 = {
            "compression_ratio": round(2 * n_total / p2_total, 5),
            "decode_ms_per_step": round(p2_ms, 4),
            "bf16_out_gbs": round(out_bytes / (p2_ms * 1e-3) / 1e9, 1),
            "hbm_gbs": round((p2_read + out_bytes) / (p2_ms * 1e-3) / 1e9, 1),
        }
        log("power-of-two widths: ratio %.4f, decode %.3f ms/step"
            % (pow2["compression_ratio"], p2_ms))
        del p2_streams, p2_table
        torch.cuda.empty_cache()

    del outs, xs
    torch.cuda.empty_cache()

    # ---- HBM ceiling for the decoder's access shape ---------------------------
    ceiling = stream_ceiling(enc, torch, np, dev, stream, algo_read, out_bytes)
    copy_gbs = ceiling["copy_ceiling_gbs"]

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {
            "workload": ("set8b: %d x Llama-3-8B layer (q,o 4096x4096; k,v 4096x1024; gate,up "
                         "4096x14336; down 14336x4096) + 128256x4096 embedding + LM head; BF16 "
                         "N(0, sigma ~ U(0.01,0.05)) with 0.1%% of entries x20; decode all per step"
                         % args.layers),
            "tensors": len(idx),
            "elements": n_total,
            "block_size": B,
        },
        "compression_ratio": round(ratio, 5),
        "hbm_gbs": round(achieved, 1),
        "hbm_frac_of_8tbs": round(achieved / HBM_PEAK_GBS, 4),
        "copy_ceiling_gbs": round(copy_gbs, 1),
        "hbm_frac_of_copy": round(achieved / copy_gbs, 4),
        "copy_ceiling": ceiling,
        "encode_gbs": round((2 * n_total + comp_total) / (enc_ms * 1e-3) / 1e9, 1),
        "encode_ms_per_tensor_calls": round(enc_ms, 2),
        "encode_batch_ms": round(enc_batch_ms, 2),
        "encode_batch_gbs": round((2 * n_total + comp_total) / (enc_batch_ms * 1e-3) / 1e9, 1),
        "per_tensor_launch_ms_per_step": round(per_tensor_ms, 4),
        "decode_launch_ms": {"mean": round(avg_launch_ms, 4),
                             "median": round(float(np.median(launch_ms)), 4),
                             "min": round(min(launch_ms), 4), "max": round(max(launch_ms), 4)},
        "roofline": {
            "bound": "hbm",
            "kernel": "k_decode_batch",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic_from_profile(launch_bytes),
            "algorithmic_bytes_per_launch": launch_bytes,
            "avg_launch_ms": round(avg_launch_ms, 4),
        },
    }

    if pow2 is not None:
        result["pow2_widths"] = pow2

    if not args.no_wide:
        result["wide_types"] = bench_wide(enc, synth, torch, np, dev, stream, args)

    if not args.no_configs:
        result["other_configs"] = bench_configs(enc, synth, torch, np, dev, stream, args)

    if not args.no_gemm:
        result["fused_gemm"] = bench_gemm(enc, synth, torch, np, dev, stream, args.gemm_m,
                                          args.gemm_b)
        result["fused_gemm_nt"] = bench_gemm_nt(enc, synth, torch, np, dev, args.gemm_nt_m,
                                                args.gemm_b)
        result["gemm_roofline"] = gemm_roofline(result["fused_gemm"], result["fused_gemm_nt"],
                                                args.gemm_b)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth, np, torch, dev, args.cpu_layers,
                                              args.cpu_layers_1t, B)

    print(json.dumps(result), flush=True)


def bench_wide(enc, synth, torch, np, dev, stream, args):
    """The same code on FP16 and FP32 weights (header dtype 2 and 3): the
    tensors of the set's first layers generated in that type, compressed on
    the GPU, then decoded with one batched launch per step (and, for context,
    one enc_decompress launch per tensor). Bit-exactness is checked after the
    timing."""
    shapes = synth.set8b_shapes()
    keep = ["L%d." % l for l in range(args.wide_layers)]
    idx = [i for i, (nm, _, _) in enumerate(shapes) if any(nm.startswith(k) for k in keep)]
    res = {"workload": "set8b layers 0..%d (%d tensors), same value recipe"
                       % (args.wide_layers - 1, len(idx))}
    B = args.block_size
    for dt, name in ((2, "fp16"), (3, "fp32")):
        esize = 2 if dt == 2 else 4
        streams, n_total, comp_total, read, enc_ms = [], 0, 0, 0, 0.0
        S = 11 if dt == 2 else 24
        warmed = set()
        for i in idx:
            x = synth.set8b_tensor_gpu_dt(i, dt, device=dev).reshape(-1)
            out = torch.empty(enc.enc_compress_bound_dt(x.numel(), dt), dtype=torch.uint8, device=dev)
            ws = torch.empty(enc.enc_compress_workspace_bytes(x.numel(), B), dtype=torch.uint8,
                             device=dev)
            if x.numel() not in warmed:   # first call of each shape untimed
                enc.enc_compress(x, B, dtype=dt, out=out, ws=ws)
                warmed.add(x.numel())
            out.fill_(0)                  # the driver's clear of fresh memory, outside the timing
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            comp, info = enc.enc_compress(x, B, dtype=dt, out=out, ws=ws)
            torch.cuda.synchronize()
            enc_ms += (time.perf_counter() - t0) * 1e3
            streams.append((comp.clone(), info))
            n_total += info.n_elems
            comp_total += info.total_bytes
            read += (esize * info.n_elems if info.flags == 1 else
                     (S * info.n_elems + 7) // 8 + 2 * info.n_blocks + 8 * info.n_segments
                     + info.payload_bytes)
            del x, comp, out, ws
        # the same tensors in one batched single-pass launch (inputs
        # regenerated, outputs and workspace allocated once): wall clock per
        # call, host synchronisations included; every stream must equal the
        # per-tensor one
        xs = [synth.set8b_tensor_gpu_dt(i, dt, device=dev).reshape(-1) for i in idx]
        bouts = [torch.empty(enc.enc_compress_bound_dt(x.numel(), dt), dtype=torch.uint8, device=dev)
                 for x in xs]
        bws = None
        batch_ms = []
        for rep in range(4):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            bres = enc.enc_compress_batch_dt(xs, dt, B, outs=bouts, ws=bws)
            torch.cuda.synchronize()
            if rep:
                batch_ms.append((time.perf_counter() - t0) * 1e3)
            if bws is None:
                bws = torch.empty(max(int(enc.lib().enc_compress_batch_workspace_bytes(
                    enc._citems(xs, bouts), len(xs), B)), 16), dtype=torch.uint8, device=dev)
        for (bc, binf), (c, inf) in zip(bres, streams):
            if binf.total_bytes != inf.total_bytes or not torch.equal(bc, c):
                log("MISMATCH: batched %s stream differs from the per-tensor one" % name)
                sys.exit(1)
        bms = sorted(batch_ms)[len(batch_ms) // 2]
        del xs, bouts, bws, bres
        torch.cuda.empty_cache()
        outs = [torch.empty(inf.n_elems, dtype=torch.int16 if dt == 2 else torch.int32,
                            device=dev) for _, inf in streams]
        table = enc.enc_batch_prepare([(c, inf, o) for (c, inf), o in zip(streams, outs)])
        count = len(streams)

        def per_tensor():
            for (c, inf), o in zip(streams, outs):
                enc.enc_decompress(c, inf, out=o)

        def timed(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.steps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / args.steps
        pt_ms = timed(per_tensor)
        ms = timed(lambda: enc.enc_decompress_batch(table, count))
        for k, i in enumerate(idx):
            x = synth.set8b_tensor_gpu_dt(i, dt, device=dev).reshape(-1)
            if not torch.equal(outs[k], x):
                log("MISMATCH in %s tensor %s" % (name, shapes[i][0]))
                sys.exit(1)
            del x
        out_bytes = esize * n_total
        res[name] = {
            "elements": n_total,
            "compression_ratio": round(out_bytes / comp_total, 5),
            "encode_gbs": round((out_bytes + comp_total) / (enc_ms * 1e-3) / 1e9, 1),
            "encode_batch_ms": round(bms, 4),
            "encode_batch_gbs": round((out_bytes + comp_total) / (bms * 1e-3) / 1e9, 1),
            "decode_ms_per_step": round(ms, 4),
            "out_gbs": round(out_bytes / (ms * 1e-3) / 1e9, 1),
            "hbm_gbs": round((read + out_bytes) / (ms * 1e-3) / 1e9, 1),
            "per_tensor_launch_ms_per_step": round(pt_ms, 4),
        }
        log("%s: ratio %.4f, encode %.1f ms per tensor call / %.2f ms batched (%.1f GB/s), "
            "decode %.3f ms/step (%.1f GB/s HBM; per-tensor launches %.3f ms), bit-exact"
            % (name, res[name]["compression_ratio"], enc_ms, bms, res[name]["encode_batch_gbs"], ms,
               res[name]["hbm_gbs"], pt_ms))
        del streams, outs, table
        torch.cuda.empty_cache()
    return res


def bench_configs(enc, synth, torch, np, dev, stream, args):
    """Ratio and throughput of the other configurations (context for the
    headline, not the headline): the tiny matrix, one Llama-3-8B layer at
    B = 256 / 512 / 1024, and the five 2^27-value stress distributions at the
    same block sizes. Each case is compressed on the GPU (wall clock, one
    host synchronisation per tensor) and decoded with one batched launch per
    step, rotating over four copies of the streams and outputs so the
    working set exceeds the 256 MB last-level cache (the tiny case does not:
    it is launch-bound). Outputs are checked bit-exactly after the timing."""
    cases = [("tiny", [synth.tiny()], (512,))]
    layer = synth.layer()
    cases.append(("layer", [layer[k] for k in sorted(layer)], (256, 512, 1024)))
    for kind in synth.STRESS_KINDS:
        cases.append(("stress." + kind, [synth.stress(kind)], (256, 512, 1024)))
    res = {}
    for name, tensors, blocks in cases:
        xs = [torch.from_numpy(np.ascontiguousarray(t).reshape(-1).view(np.int16)).to(dev) for t in tensors]
        n = sum(x.numel() for x in xs)
        # output and workspace buffers allocated, and touched, outside the
        # timed calls (the driver clears fresh memory before its first use)
        e_outs = [torch.zeros(enc.enc_compress_bound(x.numel()), dtype=torch.uint8, device=dev)
                  for x in xs]
        e_ws = [torch.zeros(max(enc.enc_compress_workspace_bytes(x.numel(), b) for b in blocks),
                            dtype=torch.uint8, device=dev) for x in xs]
        for B in blocks:
            copies, total, enc_s = [], 0, 0.0
            for c in range(4):
                st = []
                for x, eo, ew in zip(xs, e_outs, e_ws):
                    torch.cuda.synchronize()
                    t0 = time.perf_counter()
                    comp, info = enc.enc_compress(x, B, out=eo, ws=ew)
                    torch.cuda.synchronize()
                    enc_s += time.perf_counter() - t0
                    st.append((comp.clone(), info))
                    if c == 0:
                        total += info.total_bytes
                    del comp
                outs = [torch.empty_like(x) for x in xs]
                table = enc.enc_batch_prepare([(cp, inf, o) for (cp, inf), o in zip(st, outs)])
                copies.append((st, outs, table))
            for k in range(args.warmup):
                st, outs, table = copies[k % 4]
                enc.enc_decompress_batch(table, len(outs))
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            steps = max(args.steps, 4)
            e0.record(stream)
            for k in range(steps):
                st, outs, table = copies[k % 4]
                enc.enc_decompress_batch(table, len(outs))
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            for st, outs, _ in copies:
                for x, o in zip(xs, outs):
                    if not torch.equal(o, x):
                        log("MISMATCH in config %s B=%d" % (name, B))
                        sys.exit(1)
            res["%s.B%d" % (name, B)] = {
                "elements": n,
                "compression_ratio": round(2 * n / total, 5),
                "raw_tensors": sum(1 for _, inf in copies[0][0] if inf.flags == 1),
                "decode_ms": round(ms, 4),
                "bf16_out_gbs": round(2 * n / (ms * 1e-3) / 1e9, 1),
                "hbm_gbs": round((2 * n + total) / (ms * 1e-3) / 1e9, 1),
                "encode_gbs_wall": round(4 * (2 * n + total) / enc_s / 1e9, 1),
            }
            log("config %-18s B=%4d: ratio %.4f, decode %.3f ms (%.0f GB/s HBM), bit-exact"
                % (name, B, 2 * n / total, ms, res["%s.B%d" % (name, B)]["hbm_gbs"]))
            del copies
        del xs, e_outs, e_ws
        torch.cuda.empty_cache()
    return res


def _graph_time_us(fn, torch, calls=8, replays=20):
    """GPU time per call of `fn`: `calls` calls are captured into one HIP graph
    and the graph is replayed, so no host work sits between the launches."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(replays):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (replays * calls), g


def bench_gemm(enc, synth, torch, np, dev, stream, ms, B=512):
    """Y = X W with W 4096x14336 compressed (block size B) vs the same GEMM on the
    uncompressed W, M from 1 to 256. Eight rotating weight copies keep the
    working set well above the 256 MB last-level cache; times are GPU time per
    call from HIP-graph replays, and every replayed result is checked
    bit-exactly against an eager call (the fused path is deterministic)."""
    K, N = 4096, 14336
    W = torch.from_numpy(synth.gemm_weight(K, N).view(np.int16)).to(dev)
    copies = GEMM_COPIES
    Ws = [W.clone() for _ in range(copies)]
    comps = [enc.enc_compress(w, B) for w in Ws]
    out = {"shape": "X[M,4096] x W[4096,14336], W compressed at B=%d" % B,
           "rotating_copies": copies,
           "timing": "GPU time per call, HIP-graph replay of 8 calls x 20",
           "w_bytes_compressed": comps[0][1].total_bytes, "w_bytes_dense": 2 * K * N}
    for M in [int(v) for v in ms.split(",")]:
        X = torch.from_numpy(synth.gemm_activations(M, K).view(np.int16)).to(dev)
        Xb = X.view(torch.bfloat16)
        Ys = [torch.empty((M, N), dtype=torch.float32, device=dev) for _ in range(copies)]
        ws = enc.gemm_workspace(M, K, N, B, dev)
        try:
            ref = [enc.enc_decompress_gemm(X, c, inf, N, ws=ws).clone() for c, inf in comps]
            k = [0]

            def fused():
                c, inf = comps[k[0] % copies]
                enc.enc_decompress_gemm(X, c, inf, N, y=Ys[k[0] % copies], ws=ws)
                k[0] += 1

            def dense():
                enc.enc_gemm_dense(X, Ws[k[0] % copies], y=Ys[k[0] % copies], ws=ws)
                k[0] += 1

            def blas():
                torch.matmul(Xb, Ws[k[0] % copies].view(torch.bfloat16))
                k[0] += 1

            tf, _ = _graph_time_us(fused, torch)
            for c in range(copies):
                if not torch.equal(Ys[c], ref[c]):
                    raise RuntimeError("fused GEMM graph replay differs from the eager result")
            td, _ = _graph_time_us(dense, torch)
            tb, _ = _graph_time_us(blas, torch)
            flops = 2.0 * M * K * N
            bytes_f = comps[0][1].total_bytes + 2 * M * K + 4 * M * N
            out["M%d" % M] = {
                "fused_us": round(tf, 2),
                "dense_same_kernel_us": round(td, 2),
                "hipblaslt_bf16_us": round(tb, 2),
                "fused_hbm_gbs": round(bytes_f / (tf * 1e-6) / 1e9, 1),
                "fused_tflops": round(flops / (tf * 1e-6) / 1e12, 2),
                "mfma_util_vs_2.5pf": round(flops / (tf * 1e-6) / 1e12 / BF16_DENSE_PEAK_TFLOPS, 4),
                "speedup_vs_dense_same_kernel": round(td / tf, 3),
                "speedup_vs_hipblaslt": round(tb / tf, 3),
            }
        except Exception as e:  # the GEMM kernels report through EncError
            out["M%d" % M] = {"error": str(e)}
    return out


def bench_gemm_nt(enc, synth, torch, np, dev, ms="1,16,128", B=512):
    """Y = X W^T with W in linear-layer layout [14336, 4096], compressed at
    block size B, against the same kernel on the dense W and torch's F.linear
    (hipBLASLt); eight rotating weight copies, HIP-graph replay timing."""
    import torch.nn.functional as F
    K, N = 4096, 14336
    W = torch.from_numpy(synth.gaussian_bits((N, K), 0.02, 4, 1, outliers=False).view(np.int16)).to(dev)
    copies = GEMM_COPIES
    Ws = [W.clone() for _ in range(copies)]
    comps = [enc.enc_compress(w.reshape(-1), B) for w in Ws]
    out = {"shape": "X[M,4096] x W^T, W [14336,4096] compressed at B=%d" % B,
           "rotating_copies": copies,
           "w_bytes_compressed": comps[0][1].total_bytes}
    for M in [int(v) for v in ms.split(",")]:
        X = torch.from_numpy(synth.gemm_activations(M, K).view(np.int16)).to(dev)
        Xb = X.view(torch.bfloat16)
        Y = torch.empty((M, N), dtype=torch.float32, device=dev)
        ws = enc.gemm_nt_workspace(M, K, N, B, dev)
        k = [0]

        def fused():
            c, inf = comps[k[0] % copies]
            enc.enc_decompress_gemm_nt(X, c, inf, N, y=Y, ws=ws)
            k[0] += 1

        def dense():
            enc.enc_gemm_dense_nt(X, Ws[k[0] % copies], y=Y, ws=ws)
            k[0] += 1

        def blas():
            F.linear(Xb, Ws[k[0] % copies].view(torch.bfloat16))
            k[0] += 1

        try:
            tf, _ = _graph_time_us(fused, torch)
            td, _ = _graph_time_us(dense, torch)
            tb, _ = _graph_time_us(blas, torch)
            out["M%d" % M] = {"fused_us": round(tf, 2), "dense_same_kernel_us": round(td, 2),
                              "hipblaslt_linear_us": round(tb, 2),
                              "speedup_vs_hipblaslt": round(tb / tf, 3)}
        except Exception as e:  # the GEMM kernels report through EncError
            out["M%d" % M] = {"error": str(e)}
    return out


def host_threads():
    """Threads the CPU leg uses: the CPUs this process may run on, at most 16
    (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(synth, np, torch, dev, layers_T, layers_1, B):
    """The CPU oracle as it is (plain single-threaded C), on this host: its
    encode of the set's first layers and its decode of its own streams, once
    on one thread (layers 0..layers_1-1) and once on T threads, one tensor
    per thread (layers 0..layers_T-1). The values are the same tensors the
    GPU path measures; every decode is checked against its input."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle as orc
    orc.build()
    shapes = synth.set8b_shapes()
    T = host_threads()

    def sample(layers):
        keep = ["L%d." % l for l in range(layers)]
        idx = [i for i, (nm, _, _) in enumerate(shapes) if any(nm.startswith(k) for k in keep)]
        return idx, [synth.set8b_tensor_gpu(i, device=dev).cpu().numpy().view(np.uint16).reshape(-1)
                     for i in idx]

    def run(xs, threads):
        with ThreadPoolExecutor(threads) as ex:
            t0 = time.perf_counter()
            streams = list(ex.map(lambda x: orc.encode(x, B), xs))
            enc_s = time.perf_counter() - t0
            t0 = time.perf_counter()
            ys = list(ex.map(orc.decode, streams))
            dec_s = time.perf_counter() - t0
        for x, y in zip(xs, ys):
            assert np.array_equal(x, y), "oracle round trip failed"
        return enc_s, dec_s

    idx1, xs1 = sample(layers_1)
    n1 = sum(x.size for x in xs1)
    enc1, dec1 = run(xs1, 1)
    del xs1
    idxT, xsT = sample(layers_T)
    nT = sum(x.size for x in xsT)
    encT, decT = run(xsT, T)
    del xsT
    gemm = cpu_gemm_baseline(synth, np, orc, T)
    return {
        "value": round(2 * nT / decT / 1e9, 4),
        "unit": "GB/s",
        "cores": T,
        "kind": "oracle",
        "sample": "oracle decode of its own B=%d streams of set8b layers 0-%d (%d tensors, %d "
                  "values, %.2f GB BF16 out), one tensor per thread on %d threads of a %s"
                  % (B, layers_T - 1, len(idxT), nT, 2 * nT / 1e9, T, cpu_model()),
        "cpu_model": cpu_model(),
        "threads": T,
        "decode_s": round(decT, 3),
        "encode_s": round(encT, 3),
        "encode_gbs": round(2 * nT / encT / 1e9, 4),
        "one_thread": {
            "sample": "set8b layers 0-%d (%d tensors, %d values)" % (layers_1 - 1, len(idx1), n1),
            "decode_gbs": round(2 * n1 / dec1 / 1e9, 4),
            "encode_gbs": round(2 * n1 / enc1 / 1e9, 4),
            "decode_s": round(dec1, 3),
            "encode_s": round(enc1, 3),
        },
        "gemm": gemm,
    }


GEMM_ORACLE_COLS = 112   # columns of W per thread in the oracle's GEMM timing sample


def cpu_gemm_baseline(synth, np, orc, T):
    """The oracle's fp64 GEMM (Y and its absolute bound, as the tests use it)
    on X [M, 4096] x W [4096, 14336] at M = 1, 16, 128: a bounded sample of
    GEMM_ORACLE_COLS output columns per thread, on 1 thread and on T threads
    (one contiguous column range each), scaled to the time of the whole
    product."""
    from concurrent.futures import ThreadPoolExecutor
    K, N = 4096, 14336
    W = synth.gemm_weight(K, N)
    out = {"sample": "%d output columns per thread of X[M,4096] x W[4096,14336]" % GEMM_ORACLE_COLS,
           "threads": T}
    for M in (1, 16, 128):
        X = synth.gemm_activations(M, K)
        cols1 = np.arange(GEMM_ORACLE_COLS, dtype=np.uint32)
        t0 = time.perf_counter()
        orc.gemm_f64_cols(X, W, cols1)
        t1 = time.perf_counter() - t0
        ranges = [np.arange(i * GEMM_ORACLE_COLS, (i + 1) * GEMM_ORACLE_COLS, dtype=np.uint32) % N
                  for i in range(T)]
        with ThreadPoolExecutor(T) as ex:
            t0 = time.perf_counter()
            list(ex.map(lambda c: orc.gemm_f64_cols(X, W, c), ranges))
            tT = time.perf_counter() - t0
        flops_1, flops_T = 2.0 * M * K * GEMM_ORACLE_COLS, 2.0 * M * K * GEMM_ORACLE_COLS * T
        out["M%d" % M] = {
            "one_thread_gflops": round(flops_1 / t1 / 1e9, 3),
            "threads_gflops": round(flops_T / tT / 1e9, 3),
            "threads_us_per_call": round(2.0 * M * K * N / (flops_T / tT) * 1e6, 1),
        }
    return out


def stream_ceiling(enc, torch, np, dev, stream, read_bytes, write_bytes):
    """HBM rate of the library's streaming kernel with the decoder's access
    shape (16-byte loads, non-temporal 16-byte stores, one contiguous run per
    workgroup, workgroups in order) over exactly one decode step's bytes:
    read_bytes read, write_bytes written. Workgroups of 64 or 256 threads, 1,
    2 or 4 items per thread (the decoder: 256 threads, 8 KB written per
    workgroup). The ceiling is the fastest shape. A 4 GiB torch copy_ is
    kept for context."""
    rb = (read_bytes + 15) // 16 * 16
    wb = (write_bytes + 15) // 16 * 16
    src = torch.empty(rb, dtype=torch.uint8, device=dev)
    dst = torch.empty(wb, dtype=torch.uint8, device=dev)
    src.fill_(0x3C)
    res = {"read_bytes": rb, "write_bytes": wb}
    best = 0.0
    for threads, items in ((64, 1), (64, 2), (256, 1), (256, 2), (256, 4)):
        enc.enc_stream_probe(src, dst, items, threads)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            enc.enc_stream_probe(src, dst, items, threads)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = (rb + wb) / (ms * 1e-3) / 1e9
        res["t%d_items%d" % (threads, items)] = {"ms": round(ms, 4), "gbs": round(gbs, 1),
                                                 "kb_written_per_workgroup": threads * items // 64}
        best = max(best, gbs)
        log("stream probe, %d threads x %d item(s): %.3f ms, %.1f GB/s" % (threads, items, ms, gbs))
    del src, dst
    torch.cuda.empty_cache()
    a = torch.empty(1 << 32, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    res["torch_copy_4gib_gbs"] = round(2 * a.numel() * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    res["copy_ceiling_gbs"] = round(best, 1)
    return res


GEMM_PMC = os.path.join(ROOT, "profiles", "gemm_w4096x14336_b512_pmc.json")
GEMM_SRCS = [os.path.join(CSRC, f) for f in ("gemm.hip", "group_math.h", "enc_common.h")]


def gemm_roofline(g, gnt, B=512):
    """Roofline of the fused decompress-GEMM at M = 1, 16, 128 (both
    layouts): algorithmic bytes per call (the compressed stream, X and Y) over
    the GPU time per call, against 8 TB/s, and the MFMA share of the 2.5
    PFLOP/s dense BF16 peak; the HBM traffic per call comes from the
    committed rocprofv3 PMC summary when it was taken on the current source
    (at B = 512, the block size it was taken at)."""
    pmc = None
    try:
        d = json.load(open(GEMM_PMC))
        if B == 512 and d.get("gemm_source_sha256_16") == source_hash(GEMM_SRCS):
            pmc = d
    except (OSError, ValueError):
        pass
    out = {"bound": "hbm", "peak_gbs": HBM_PEAK_GBS, "mfma_peak_tflops": BF16_DENSE_PEAK_TFLOPS}
    for name, res in (("kn", g), ("nk", gnt)):
        for M in (1, 16, 128):
            r = res.get("M%d" % M, {})
            if "fused_us" not in r:
                continue
            K, N = 4096, 14336
            alg = res["w_bytes_compressed"] + 2 * M * K + 4 * M * N
            t = r["fused_us"] * 1e-6
            ent = {
                "algorithmic_bytes": alg,
                "us_per_call": r["fused_us"],
                "achieved_gbs": round(alg / t / 1e9, 1),
                "frac": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
                "mfma_frac": round(2.0 * M * K * N / t / 1e12 / BF16_DENSE_PEAK_TFLOPS, 4),
                "traffic": None,
            }
            calls = pmc.get("per_call" if name == "kn" else "nt_per_call", {}) if pmc else {}
            if ("M%d" % M) in calls:
                tr = calls["M%d" % M]
                ent["traffic"] = tr["hbm_bytes"]
                ent["traffic_ratio"] = round(tr["hbm_bytes"] / alg, 4)
            out["%s.M%d" % (name, M)] = ent
    return out


if __name__ == "__main__":
    main()
