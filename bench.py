#!/usr/bin/env python3
"""Benchmark of the decompression hot path on one MI355X.

A step is one df_decompress of a whole Llama-3-8B-shaped transformer block
(q, k, v, o, gate, up, down: 218,103,808 BF16 weights, one codebook, one
launch) from device-resident compressed sections into a BF16 buffer.  The
compressed inputs are rotated over several device copies and the output over
two buffers, so each step reads inputs that the 256 MB Infinity Cache does
not hold.  Prints one JSON line:

  value      decompressed BF16 GB/s = 2 n K / wall time of K steps
  roofline   algorithmic HBM bytes of one launch (stream bytes + sign|mantissa
             bytes + gap bits + tile offsets read, 2 n written) / the
             launch's mean duration, against 8 TB/s.  The K launches run back
             to back between one pair of HIP events on their stream; the mean
             is that span over K.  Also: the same bytes against two plain
             device copies timed in the same run, and the HBM bytes counted
             by rocprofv3 for this kernel source (profiles/hbm_traffic.json)
  cpu_baseline  the CPU oracle's decode of the same container on the host
             cores (tile ranges on threads), a plain bit-serial reference

Other workloads (--workload) are for local measurement; the default is the
8B BF16 block.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import statistics
import sys
import time

import numpy as np

METRIC = "decompressed BF16 GB/s (+% of HBM roofline), 8B-shaped transformer block"
HBM_PEAK_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(inf) -> int:
    """Bytes one launch must move: the used stream, the gap fields, the tile
    offsets and (BF16) the sign|mantissa plane read; the output written."""
    n = int(inf["n"])
    read = (int(inf["total_bits"]) + 7) // 8 + (5 * int(inf["n_threads"]) + 7) // 8 \
        + 8 * (int(inf["n_tiles"]) + 1)
    if int(inf["kind"]) == 0:
        read += n
        write = 2 * n
    elif int(inf["kind"]) == 1:
        write = n
    else:                       # uint4, packed two per byte
        write = (n + 1) // 2
    return read + write


WORKLOADS = ("llama3_8b_block_bf16", "c1_1m_bf16", "llama3_8b_block_u8", "llama3_8b_32_blocks_bf16",
             "llama31_405b_block_t3_bf16", "llama3_8b_lm_head_bf16", "llama3_8b_block_u4")


def make_workload(name: str, seed: int):
    """Returns (kind, sources, config fields, mode).  mode "one": one
    container, one launch; "batch": several containers in one
    df_decompress_batch launch; "sequence": one launch per container, in
    order, into one reused output buffer."""
    from lossless_entropy_coded_huffman_amd import synth
    if name == "llama3_8b_block_bf16":
        src, _ = synth.bf16_block(seed)
        return 0, [src], {"matrices": "q,k,v,o,gate,up,down", "shapes": "Llama-3-8B block",
                          "dist": "N(0,s^2), s~U[0.01,0.04] per matrix"}, "one"
    if name == "c1_1m_bf16":
        return 0, [synth.c1_tensor(seed)], {"dist": "N(0,0.02^2)"}, "one"
    if name == "llama3_8b_block_u8":
        layers = synth.u8_block(seed)
        return 1, [q for _, q, _ in layers], {"matrices": "q,k,v,o,gate,up,down",
                                              "quantizers": "".join("A" if a else "U" for _, _, a in layers)}, "batch"
    if name == "llama3_8b_32_blocks_bf16":
        blocks = []
        for j in range(32):
            log("block", j)
            blocks.append(synth.bf16_block(seed, config=synth.CONFIG_8B_FULL, block=j)[0])
        return 0, blocks, {"shapes": "32 Llama-3-8B blocks, one codebook each",
                           "dist": "N(0,s^2), s~U[0.01,0.04] per matrix"}, "sequence"
    if name == "llama31_405b_block_t3_bf16":
        src, _ = synth.bf16_block(seed, config=synth.CONFIG_405B, shapes=synth.LLAMA31_405B_BLOCK,
                                  dist="t3")
        return 0, [src], {"matrices": "q,k,v,o,gate,up,down", "shapes": "Llama-3.1-405B block",
                          "dist": "Student-t(3)*0.02/sqrt(3)"}, "one"
    if name == "llama3_8b_block_u4":
        layers = synth.u4_block(seed)
        return 2, [(p, n) for _, p, n, _ in layers], {
            "matrices": "q,k,v,o,gate,up,down", "packing": "two per byte, low nibble first",
            "quantizers": "".join("A" if a else "U" for _, _, _, a in layers)}, "batch"
    if name == "llama3_8b_lm_head_bf16":
        src, _ = synth.bf16_block(seed, config=synth.CONFIG_LM_HEAD, shapes=synth.LLAMA3_8B_LM_HEAD)
        return 0, [src], {"matrices": "lm_head", "shapes": "128256x4096, one matrix, one codebook",
                          "dist": "N(0,s^2), s~U[0.01,0.04]"}, "one"
    raise SystemExit("unknown workload " + name)


def src_elems(kind, s) -> int:
    """Elements of one workload source (uint4 sources are (packed, n))."""
    return int(s[1]) if kind == 2 else int(s.size)


def src_compress(dfh, kind, s):
    return dfh.compress(kind, s[0], n=s[1]) if kind == 2 else dfh.compress(kind, s)


def src_expected(kind, s) -> np.ndarray:
    """The bytes the decoder must write for one source."""
    return s[0] if kind == 2 else s.view(np.int16) if kind == 0 else s


def out_bytes_of(kind, n) -> int:
    return 2 * n if kind == 0 else n if kind == 1 else (n + 1) // 2


def cpu_baseline(containers, srcs, kind):
    import oracle
    cores = cpu_threads()
    # a bounded sample: at most about 220M weights (one 8B block's worth)
    keep, total = 0, 0
    while keep < len(containers) and (keep == 0 or total + int(containers[keep].info()["n"]) <= 230_000_000):
        total += int(containers[keep].info()["n"])
        keep += 1
    containers, srcs = containers[:keep], srcs[:keep]
    out_bytes = sum(out_bytes_of(kind, int(c.info()["n"])) for c in containers)
    dicts = []
    for c in containers:
        inf = c.info()
        d = {k: np.asarray(c.section(k)) for k in ("bitstream", "gaps", "tile_out", "sign_mantissa")}
        d.update(kind=inf["kind"], n=inf["n"], n_tiles=inf["n_tiles"], n_threads=inf["n_threads"],
                 lengths=inf["lengths"])
        dicts.append(d)
    def decode(d, threads):   # the oracle's full output (uint4 packed by the oracle)
        o = oracle.decode_tiles(d, threads)
        return oracle.pack_u4(o) if kind == 2 else o

    def expect(s, n=None):
        e = src_expected(kind, s)
        if n is None:
            return e
        return e[: (n + 1) // 2] if kind == 2 else e[:n]

    times = []
    for _ in range(3):
        t0 = time.perf_counter()
        outs = [decode(d, cores) for d in dicts]
        times.append(time.perf_counter() - t0)
    ok = all(np.array_equal(o.view(np.uint8), expect(s).view(np.uint8)) for o, s in zip(outs, srcs))
    t_mt = statistics.median(times)
    # one thread on the first sixteenth of the tiles of the first container
    d0 = dict(dicts[0])
    nt = max(1, int(d0["n_tiles"]) // 16)
    d0["n_tiles"] = nt
    d0["n"] = int(d0["tile_out"][nt])
    d0["tile_out"] = d0["tile_out"][: nt + 1]
    t0 = time.perf_counter()
    o1 = decode(d0, 1)
    t_1 = time.perf_counter() - t0
    if kind == 2 and d0["n"] % 2:   # a cut inside a byte: compare whole bytes only
        o1 = o1[:-1]
        ok = ok and np.array_equal(o1, expect(srcs[0], d0["n"] - 1))
    else:
        ok = ok and np.array_equal(o1.view(np.uint8), expect(srcs[0], d0["n"]).view(np.uint8))
    return {
        "value": round(out_bytes / t_mt / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": "%d of the workload's containers (%d elements), oracle bit-serial decode over "
                  "contiguous tile ranges on %d threads, median of 3 runs; single-thread figure on "
                  "the first 1/16 of the first container's tiles (%d elements)"
                  % (keep, total, cores, d0["n"]),
        "value_1thread": round(out_bytes_of(kind, d0["n"]) / t_1 / 1e9, 4), "verified": bool(ok),
        "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
        "host_cpus_usable": len(os.sched_getaffinity(0)),
        "cores_note": "threads = the CPUs this process may use, at most 16 (the host CPU share "
                      "that comes with one GPU on the one-GPU hosts this runs on)",
    }


def cpu_threads() -> int:
    """Worker threads for the CPU baseline: the CPUs this process may run on,
    capped at 16, the host share that goes with one GPU here."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_model() -> str:
    """The host CPU's model name as lscpu reports it (else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for ln in out.splitlines():
            if ln.strip().startswith("Model name"):
                return ln.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--warmup-s", type=float, default=0.5,
                    help="untimed decoding for at least this many seconds before the --warmup "
                         "steps: the chip's power management slows this kernel by 10-15%% about "
                         "10-50 launches after it starts loading an idle GPU, then settles "
                         "(a plain copy kernel shows no such window)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copies", type=int, default=3, help="device copies of the compressed input")
    ap.add_argument("--workload", default="llama3_8b_block_bf16", choices=WORKLOADS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--forward", type=int, default=0, metavar="BLOCKS",
                    help="instead of the decode benchmark: a forward pass over this many "
                         "Llama-3-8B-shaped blocks, weights decoded one block ahead on a side "
                         "stream; prints the exposed decode time per block")
    ap.add_argument("--forward-caps", default="0,128,64,32",
                    help="workgroup caps of the side-stream decode measured by --forward (0: none)")
    ap.add_argument("--encode", action="store_true",
                    help="instead of the decode benchmark: encode the workload on the GPU and on "
                         "the host, check the sections are identical, print both times")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the codec, time a plain device copy of MIB MiB (the "
                         "reference kernel for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the codec needs no collectives and this build "
              "measures the single-GPU decode (a multi-GPU run would shard whole transformer "
              "blocks across GPUs with no exchange step).", file=sys.stderr)
        sys.exit(2)

    import torch
    import lossless_entropy_coded_huffman_amd as dfh
    from lossless_entropy_coded_huffman_amd import build_lib

    if not os.path.exists(build_lib.LIB):
        build_lib.build()
    if not torch.cuda.is_available():
        raise SystemExit("no GPU")
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(torch, dev, args)
        return
    if args.forward:
        forward_overlap(torch, dev, args)
        return
    if args.encode:
        encode_bench(torch, dev, args)
        return

    log("workload", args.workload, "seed", args.seed)
    kind, srcs, wconf, mode = make_workload(args.workload, args.seed)
    n = sum(src_elems(kind, s) for s in srcs)
    t0 = time.perf_counter()
    containers = [src_compress(dfh, kind, s) for s in srcs]
    log("compressed in %.2f s" % (time.perf_counter() - t0))
    infos = [c.info() for c in containers]
    # one copy when the inputs alone exceed the 256 MB Infinity Cache many times
    n_copies = 1 if mode == "sequence" else max(1, args.copies)
    copies = [[dfh.to_device(c, dev) for c in containers] for _ in range(n_copies)]
    if mode == "sequence":
        outs = [[copies[0][0].empty_output()] for _ in range(2)]  # one reused scratch
    else:
        outs = [[dc.empty_output() for dc in copies[0]] for _ in range(2)]
    stream = torch.cuda.current_stream(dev)

    def launches(k):
        """The launches of step k as callables (events go around each)."""
        dcs = copies[k % len(copies)]
        o = outs[k % 2]
        if mode == "one":
            return [lambda: dfh.df_decompress(dcs[0], o[0], stream)]
        if mode == "batch":
            return [lambda: dfh.df_decompress_batch(dcs, o, stream)]
        return [lambda dc=dc: dfh.df_decompress(dc, o[0], stream) for dc in dcs]

    # Python's cyclic collector runs once here and stays off through the
    # warm-up and the timed launches: a full collection can take tens of
    # milliseconds, several times the timed region at --steps 20, and a
    # pause of that length just before the region lets the chip's clock
    # drop again (measured: 7-11% slower timed launches).
    gc.collect()
    gc.disable()
    # Time-based warm-up first: measured per-launch times on a fresh box are
    # steady for about ten launches, 10-15% slower for the next 40 while the
    # shader clock drops under the decoder's power draw, and steady again
    # after about 100 (the clock settles near 2.35 GHz); a plain copy kernel
    # runs at its steady rate from its fifth launch.  The timed steps should
    # measure the settled chip, whatever --warmup the caller gives.
    t_w = time.perf_counter()
    n_w = 0
    while time.perf_counter() - t_w < args.warmup_s:
        for k in range(20):
            for f in launches(k):
                f()
        n_w += 20
        torch.cuda.synchronize()
    warmup_s = time.perf_counter() - t_w
    for k in range(args.warmup):
        for f in launches(k):
            f()
    torch.cuda.synchronize()
    per_step = len(launches(0))
    # The timed region holds the launches alone, back to back, between one
    # pair of events on the launch stream: events between launches cost
    # several microseconds each and would be timed as part of the decode.
    # The mean launch duration is that span over the launch count (so it
    # includes the dispatch gap between launches).
    region = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region[0].record(stream)
    for k in range(args.steps):
        for f in launches(k):
            f()
    region[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gc.enable()
    mean_ms = region[0].elapsed_time(region[1]) / (args.steps * per_step)
    # spread of single launches, each between its own events, after the
    # timed region (these figures carry the event overhead)
    n_each = min(args.steps, 50)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_each * per_step)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_each * per_step)]
    i = 0
    for k in range(n_each):
        for f in launches(k):
            starts[i].record(stream)
            f()
            ends[i].record(stream)
            i += 1
    torch.cuda.synchronize()
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]

    # bit-exact check after the timed region: every output buffer, and for a
    # sequence every container decoded again into the scratch
    verified = True
    if mode == "sequence":
        o = outs[0][0]
        for s, dc in zip(srcs, copies[0]):
            dfh.df_decompress(dc, o, stream)
            ref = torch.from_numpy(s.view(np.int16)).to(dev)
            verified = verified and bool(torch.equal(o.view(torch.int16), ref))
    else:
        for o in outs:
            for s, t in zip(srcs, o):
                ref = torch.from_numpy(src_expected(kind, s)).to(dev)
                got = t.view(torch.int16) if kind == 0 else t
                verified = verified and bool(torch.equal(got, ref))

    out_bytes = sum(out_bytes_of(kind, src_elems(kind, s)) for s in srcs)
    value = out_bytes * args.steps / wall / 1e9
    alg = sum(algorithmic_bytes(i) for i in infos) / per_step  # per launch
    achieved = alg / (mean_ms * 1e-3) / 1e9
    stored = sum(dc.compressed_bytes() for dc in copies[0])
    traffic = None
    if os.path.exists(PROFILE_COUNTERS):
        try:
            prof = json.load(open(PROFILE_COUNTERS))
            entry = prof.get(args.workload)
            if entry and entry.get("kernel_source_sha") == kernel_sha():
                traffic = entry["bytes_per_launch"]
        except (ValueError, KeyError):
            traffic = None
    line = {
        "metric": METRIC if args.workload == "llama3_8b_block_bf16" else
        ("decompressed %s GB/s (+%% of HBM roofline), %s"
         % (("BF16", "uint8", "packed uint4")[kind], args.workload)),
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_s": round(warmup_s, 3), "warmup_s_steps": n_w,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "ms_per_step_events": round(mean_ms * per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "u32",
        "data": "synthetic",
        "config": dict({"workload": args.workload, "elements": int(n), "containers": len(containers),
                        "output": ("bf16", "uint8", "uint4 packed")[kind], "seed": args.seed,
                        "stored_bytes": int(stored), "stored_over_raw": round(stored / out_bytes, 4),
                        "input_copies": len(copies), "launches_per_step": per_step}, **wconf),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": int(alg), "launch_ms_mean": round(mean_ms, 5),
                     "launch_ms_evented_median": round(statistics.median(launch_ms), 5),
                     "launch_ms_evented_min": round(min(launch_ms), 5)},
        "verified": verified,
    }
    ceil = copy_ceilings(torch, dev, stream)
    for k, v in ceil.items():
        line["roofline"][k] = round(v, 1)
    line["roofline"]["frac_of_copy_ceiling"] = round(achieved / max(ceil.values()), 4)
    line["roofline"]["traffic_gbs"] = (round(traffic / (mean_ms * 1e-3) / 1e9, 1)
                                       if traffic is not None else None)
    if not args.no_cpu_baseline:
        log("cpu baseline")
        line["cpu_baseline"] = cpu_baseline(containers, srcs, kind)
    print(json.dumps(line), flush=True)
    if not verified:
        sys.exit(1)


def forward_overlap(torch, dev, args):
    """Per-block time of a forward pass with resident BF16 weights, with
    compressed weights decoded one block ahead on a side stream, and with
    each block decoded right before it runs, at several token counts.  Each
    whole forward pass is captured once as a HIP graph and replayed, so host
    launch overhead does not hide the GPU time; every replay is checked bit
    for bit against the eager resident-weight result."""
    import lossless_entropy_coded_huffman_amd as dfh
    from lossless_entropy_coded_huffman_amd import forward as fw
    shape, nb = fw.LLAMA3_8B, args.forward
    caps = [int(c) for c in args.forward_caps.split(",")]
    log("forward: generating", nb, "blocks")
    host = fw.random_blocks(nb, shape, args.seed)
    model = fw.CompressedBlocks([dfh.compress(0, h) for h in host], shape, dev)
    resident = [fw.to_torch(h, dev) for h in host]
    del host
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator(device="cpu").manual_seed(args.seed)

    def graph_of(f):
        side = torch.cuda.Stream(device=dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            f()                                  # warm-up outside the capture
        stream.wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            out = f()
        torch.cuda.synchronize()
        return gr, out

    rows, ok = {}, True
    for tokens in (1, 16, 128, 1024, 4096):
        x = (torch.randn(tokens, shape.hidden, generator=g) * 0.5).to(torch.bfloat16).to(dev)
        ref = fw.resident_forward(x, resident, shape)
        torch.cuda.synchronize()
        graphs = {"resident": graph_of(lambda: fw.resident_forward(x, resident, shape)),
                  "serial": graph_of(lambda: model.forward(x, overlap=False))}
        for cap in caps:   # the cap is read while the graph is captured
            model.decode_workgroups = cap
            graphs["overlapped_wg%d" % cap] = graph_of(lambda: model.forward(x, overlap=True))
        times = {k: [] for k in graphs}
        same = True
        for rep in range(6):
            for name, (gr, out) in graphs.items():   # interleaved, first round untimed
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                out.zero_()
                torch.cuda.synchronize()
                a.record(stream)
                gr.replay()
                b.record(stream)
                torch.cuda.synchronize()
                same = same and bool(torch.equal(out.view(torch.int16), ref.view(torch.int16)))
                if rep:
                    times[name].append(a.elapsed_time(b) * 1e3 / nb)
        ok = ok and same
        med = {k: round(statistics.median(v), 1) for k, v in times.items()}
        best = min(caps, key=lambda c: med["overlapped_wg%d" % c])
        rows[str(tokens)] = dict(med, serial_decode_us=round(med["serial"] - med["resident"], 1),
                                 exposed_decode_us_by_cap={str(c): round(med["overlapped_wg%d" % c] - med["resident"], 1)
                                                           for c in caps},
                                 best_cap=best, bit_identical=bool(same))
        log("tokens", tokens, rows[str(tokens)])
        del graphs
    print(json.dumps({"metric": "exposed decode time per Llama-3-8B-shaped block in a forward pass",
                      "unit": "us per block", "blocks": nb, "data": "synthetic",
                      "per_block_us_by_tokens": rows, "bit_identical": bool(ok),
                      "note": "HIP graph per forward pass, median of 5 interleaved replays; "
                              "resident = BF16 weights in HBM; overlapped_wgN = next block decoded on a "
                              "side stream by at most N workgroups (0: no cap); serial = each block "
                              "decoded on the compute stream before it runs"}), flush=True)
    if not ok:
        sys.exit(1)


def encode_bench(torch, dev, args):
    """Device encoder (compress_device_batch over the workload's containers:
    device histograms, host codebooks and tables, device encodes, two reads
    back to the host in all) against the host encoder (compress, all host
    threads); sections must be identical."""
    import lossless_entropy_coded_huffman_amd as dfh
    kind, srcs, wconf, _ = make_workload(args.workload, args.seed)
    n = sum(src_elems(kind, s) for s in srcs)
    in_bytes = sum((s[0] if kind == 2 else s).nbytes for s in srcs)

    def dev_tensor(s):
        if kind == 0:
            return torch.from_numpy(s.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(s[0] if kind == 2 else s).to(dev)

    dsrc = [dev_tensor(s) for s in srcs]
    nn = [s[1] if kind == 2 else None for s in srcs]
    t0 = time.perf_counter()
    host = [src_compress(dfh, kind, s) for s in srcs]
    t_host = time.perf_counter() - t0
    ws = [torch.empty(max(dfh.df_encode_workspace_bytes(src_elems(kind, s)), 16), dtype=torch.uint8, device=dev)
          for s in srcs]
    mt = torch.zeros(1, dtype=torch.int32, device=dev)
    dcs = None
    for _ in range(3):   # warm-up
        dcs = dfh.compress_device_batch(kind, dsrc, ns=nn if kind == 2 else None)
    torch.cuda.synchronize()
    e2e, kern = [], []
    stream = torch.cuda.current_stream(dev)
    for _ in range(10):
        t0 = time.perf_counter()
        dcs = dfh.compress_device_batch(kind, dsrc, ns=nn if kind == 2 else None)
        torch.cuda.synchronize()
        e2e.append(time.perf_counter() - t0)
        # the encode kernels alone, into the same sections
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for dc, t, w in zip(dcs, dsrc, ws):
            dfh.df_encode_device(kind, t, dc.n, dc.lengths, dc.layout, dc.sections, w, mt, stream)
        b.record(stream)
        torch.cuda.synchronize()
        kern.append(a.elapsed_time(b) * 1e-3)
    same = all(np.array_equal(dc.sections[name][: h.info()["section_bytes"][name]].cpu().numpy(),
                              np.asarray(h.section(name)).view(np.uint8))
               for dc, h in zip(dcs, host) for name in dfh.SECTION_NAMES)
    med = statistics.median(e2e)
    mk = statistics.median(kern)
    print(json.dumps({
        "metric": "encode throughput, input GB/s (%s)" % args.workload, "unit": "GB/s",
        "elements": int(n), "input_bytes": int(in_bytes), "containers": len(srcs),
        "device_end_to_end_ms": round(med * 1e3, 3), "device_end_to_end_GBps": round(in_bytes / med / 1e9, 1),
        "device_encode_kernels_ms": round(mk * 1e3, 3), "device_encode_kernels_GBps": round(in_bytes / mk / 1e9, 1),
        "host_ms": round(t_host * 1e3, 1), "host_GBps": round(in_bytes / t_host / 1e9, 2),
        "host_threads": os.cpu_count(), "sections_identical": bool(same), "data": "synthetic",
        "note": "end to end = device histogram, its copy to the host, host codebook and tables, "
                "device encode; kernels = the encode launches alone; host = compress() on all "
                "host threads"}), flush=True)
    if not same:
        sys.exit(1)


def copy_ceilings(torch, dev, stream, mib=1024, reps=20):
    """Read-plus-write GB/s of two plain device copies of mib MiB, each run
    back to back between one event pair on the launch stream: the runtime's
    device-to-device copy, and an elementwise int32 negation (a stream-copy
    kernel: 4 bytes read and 4 written per element).  The faster of the two
    is the practical HBM ceiling the decoder is compared with beside the
    8 TB/s peak.  Buffers are freed on return."""
    nbytes = mib << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(7)
    dst = torch.empty_like(src)
    si, di = src.view(torch.int32), dst.view(torch.int32)
    out = {}
    with torch.cuda.stream(stream):
        for name, f in (("memcpy_d2d_gbs", lambda: dst.copy_(src)),
                        ("stream_copy_gbs", lambda: torch.neg(si, out=di))):
            for _ in range(3):
                f()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(reps):
                f()
            ev[1].record(stream)
            torch.cuda.synchronize()
            out[name] = 2 * nbytes / (ev[0].elapsed_time(ev[1]) / reps * 1e-3) / 1e9
    del src, dst, si, di
    torch.cuda.empty_cache()
    return out


def copy_calibration(torch, dev, args):
    nbytes = args.copy_calibration << 20
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes,
                      "ms_per_copy": round(dt * 1e3, 4),
                      "GBps_read_plus_write": round(2 * nbytes / dt / 1e9, 1)}), flush=True)


def kernel_sha() -> str:
    import hashlib
    p = os.path.join(ROOT, "lossless_entropy_coded_huffman_amd", "csrc", "dfh_decode.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
