#!/usr/bin/env python3
"""Throughput of df11_decode on one MI355X.

One step = one df11_decode launch over a whole transformer block's linear
weights (one code book, one stream), from DF11 arrays resident in HBM to BF16
words in HBM.  The default workload is the Llama-3.1-8B-shaped block (q/o
4096x4096, k/v 1024x4096, gate/up 14336x4096, down 4096x14336; 218,103,808
weights, N(0, sigma_m) with per-matrix sigma jitter).  R identical encoded
copies at different addresses, each with its own output buffer, are decoded
in turn (R large enough that they span three times the 256 MB Infinity
Cache) so that a launch finds none of its bytes cached by the launch before.

Prints one JSON line.  value = effective GB/s = (algorithmic bytes read +
2n bytes written) / device time of one launch, where the bytes read are the
code stream (total_bits / 8), the 5-bit gaps, the block positions, the n
sign|mantissa bytes and the lookup tables.  roofline.ceiling_gbs is the rate
of a traffic-only kernel (df11_stream_ceiling) moving the same bytes on the
same buffers, timed right after the decode.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak (vendor figure)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "df11_decode_llama8b_block_traffic.txt")


def kernel_hash(name: str = "df11_decode_kernel<32>") -> str | None:
    """Hash of a kernel's machine code in the built library (written by the
    build next to it): counters stay valid exactly as long as it is equal."""
    path = os.path.join(ROOT, "huffman_decode_amd", "libdf11.kernels.json")
    try:
        with open(path) as f:
            return json.load(f).get(name)
    except (OSError, ValueError):
        return None


def algorithmic_bytes(enc) -> tuple[int, int]:
    """(bytes read, bytes written) that DF11 itself must move for one decode."""
    s = enc.sizes
    n, nb = int(s.n), int(s.n_blocks)
    read = (int(s.total_bits) + 7) // 8            # exponent codes
    read += (5 * (64 * nb + 1) + 7) // 8           # gaps
    read += 4 * (nb + 1)                            # block output positions
    read += n                                       # sign|mantissa
    read += int(s.lut_bytes)                        # tables
    return read, 2 * n


def measured_traffic(n_launch_bytes: int):
    """HBM bytes per launch from committed rocprofv3 counters, if they were taken
    on the current kernel source and on this workload (the profile's
    algorithmic bytes per launch equal n_launch_bytes); else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_isa_sha16") != kernel_hash():
        return None
    try:
        if int(vals["algorithmic_bytes_per_launch"]) != int(n_launch_bytes):
            return None
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def host_threads() -> int:
    """Host threads for the parallel oracle leg: the CPUs this process may run
    on, at most 16 (a GPU's share of its host)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    return max(1, min(avail, 16))


def _gap_fields(gaps_packed, slices):
    """5-bit gap fields at the given slice indices (packed least significant
    bit first)."""
    import numpy as np
    bits = 5 * np.asarray(slices, dtype=np.int64)
    lo = gaps_packed[bits >> 3].astype(np.uint32)
    hi = gaps_packed[(bits >> 3) + 1].astype(np.uint32)
    return (((hi << 8) | lo) >> (bits & 7).astype(np.uint32)) & 31


def cpu_baseline(wlx, enc) -> dict:
    """The oracle's bit-by-bit decode + join of the whole block: serially on one
    core, and split at block starts over the host's cores (each chunk of blocks
    decodes from its first slice's gap offset on its own, which is the chunk
    decode property the DF11 format rests on).  Both are checked bit-exact.
    Beside them, the oracle's encoder on one core, checked against the arrays
    of the product's host encoder."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    n = int(enc.sizes.n)
    total = int(enc.sizes.total_bits)
    lengths = enc.codebook.lengths
    rd, wr = algorithmic_bytes(enc)

    t0 = time.perf_counter()
    ex, end = oracle.decode(enc.stream, total, 0, n, lengths)
    w = oracle.join_bf16(ex, enc.signmant[:n])
    dt1 = time.perf_counter() - t0
    ok1 = bool(np.array_equal(w, wlx.weights)) and end == total
    del ex, w

    threads = host_threads()
    nb = int(enc.sizes.n_blocks)
    edges = np.linspace(0, nb, min(nb, 8 * threads) + 1).astype(np.int64)
    starts = 4096 * edges[:-1] + _gap_fields(enc.gaps, 64 * edges[:-1]).astype(np.int64)
    out = np.empty(n, np.uint16)
    bp = enc.block_pos.astype(np.int64)

    def chunk(i):
        b0, b1 = int(edges[i]), int(edges[i + 1])
        p0, p1 = int(bp[b0]), int(bp[b1])
        stop = 4096 * b1 if b1 < nb else total
        e = oracle.decode_range(enc.stream, total, int(starts[i]), stop, lengths, p1 - p0)
        out[p0:p1] = oracle.join_bf16(e, enc.signmant[p0:p1])
        return e.size == p1 - p0

    # the threaded leg is short (a fraction of a second on a 218 M-weight
    # block), so it runs five times and the median is reported
    runs, okn = [], True
    with ThreadPoolExecutor(max_workers=threads) as pool:
        for _ in range(5):
            out.fill(0)
            t0 = time.perf_counter()
            sizes_ok = all(pool.map(chunk, range(len(edges) - 1)))
            runs.append(time.perf_counter() - t0)
            okn = okn and sizes_ok and bool(np.array_equal(out, wlx.weights))
    dtn = sorted(runs)[len(runs) // 2]

    # the oracle's encoder on the whole block, one core: code book, bit-by-bit
    # stream, gaps and block positions; it must give the arrays the product's
    # host encoder gave
    t0 = time.perf_counter()
    oe = oracle.encode(wlx.weights)
    dte = time.perf_counter() - t0
    nbytes = (oe.total_bits + 7) // 8
    enc_ok = (oe.total_bits == total and np.array_equal(oe.lengths, lengths)
              and np.array_equal(oe.stream[:nbytes], enc.stream[:nbytes])
              and np.array_equal(oe.block_pos, enc.block_pos[: oe.n_blocks + 1])
              and np.array_equal(oe.signmant, enc.signmant[:n]))
    del oe
    return {"value": round((rd + wr) / dtn / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "gweights_per_s": round(n / dtn / 1e9, 5),
            "seconds": round(dtn, 3), "seconds_of_5_runs": [round(t, 3) for t in runs],
            "bit_exact": okn and ok1,
            "host_cpu_count": os.cpu_count(),
            "one_core": {"value": round((rd + wr) / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                         "gweights_per_s": round(n / dt1 / 1e9, 5), "seconds": round(dt1, 3)},
            "encode_one_core": {"seconds": round(dte, 3), "gweights_per_s": round(n / dte / 1e9, 5),
                                "same_arrays_as_host_encoder": bool(enc_ok)},
            "sample": f"whole {wlx.name} ({n} weights): oracle tree-walk decode of every "
                      f"code, then BF16 join; value: {len(edges) - 1} chunks of whole blocks "
                      f"on {threads} threads, median of 5 runs; one_core: serial from bit 0"}


def run_copy(args) -> int:
    """A plain device-to-device copy of known size: the reference that the HBM
    byte counters of a profiler run are scaled by, and the practical streaming
    rate of this GPU at a given size.  Rotating source/destination pairs span
    at least 768 MB (three times the 256 MB Infinity Cache), so that a copy
    finds none of its bytes cached by the one before."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nbytes = args.copy_mib << 20
    pairs = max(1, -(-768_000_000 // (2 * nbytes)))
    srcs = [torch.empty(nbytes // 2, dtype=torch.int16, device=dev).random_(-100, 100)
            for _ in range(pairs)]
    dsts = [torch.empty_like(s) for s in srcs]
    stream = torch.cuda.current_stream(dev)
    for k in range(args.warmup):
        dsts[k % pairs].copy_(srcs[k % pairs])
    torch.cuda.synchronize()
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_begin.record(stream)
    for k in range(args.steps):
        dsts[k % pairs].copy_(srcs[k % pairs])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_begin.elapsed_time(t_end) / args.steps
    print(json.dumps({"mode": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "rotating_pairs": pairs, "kernel_ms": round(ms, 5),
                      "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
                      "ok": all(bool(torch.equal(a, b)) for a, b in zip(srcs, dsts))}), flush=True)
    return 0


def run_stream(args) -> int:
    """The GPU's own streaming rates, beside which the decode's figure is read:
    read-only, write-only and copy kernels of the library (16-byte accesses,
    four in flight per thread) over --copy-mib MiB, and torch's fill and copy,
    on rotating buffers that span at least 768 MB."""
    import torch
    import huffman_decode_amd as hd
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nbytes = args.copy_mib << 20
    k_bufs = max(3, -(-768_000_000 // nbytes))
    src = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev).random_(-1000, 1000)
           for _ in range(k_bufs)]
    dst = [torch.empty_like(t) for t in src]
    grids = (2048, 8192, 32768)  # workgroups of 256 threads; reads favour few, writes many
    slots = torch.empty(max(hd.df11_stream_read_slots(nbytes, g) for g in grids),
                        dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    legs = {
        "read_only": (nbytes, lambda k, g: hd.df11_stream_read(src[k % k_bufs], slots, nbytes, g,
                                                                 stream)),
        "write_only": (nbytes, lambda k, g: hd.df11_stream_write(dst[k % k_bufs], nbytes, k, g,
                                                                   stream)),
        "copy": (2 * nbytes, lambda k, g: hd.df11_stream_copy(src[k % k_bufs], dst[k % k_bufs],
                                                              nbytes, g, stream)),
    }
    res = {"mode": "stream", "bytes_each_way": nbytes, "rotating_buffers": k_bufs}
    for name, (moved, fn) in legs.items():
        best = None
        for g in grids:  # the best grid of the three
            ms = launch_time_ms(lambda k: fn(k, g), stream, reps=args.steps, warmup=args.warmup)
            if best is None or ms < best[0]:
                best = (ms, g)
        res[name] = {"kernel_ms": round(best[0], 5), "grid": best[1],
                     "GBps": round(moved / (best[0] * 1e-3) / 1e9, 1)}
    for name, (moved, fn) in {"torch_fill": (nbytes, lambda k: dst[k % k_bufs].fill_(k)),
                              "torch_copy": (2 * nbytes,
                                             lambda k: dst[k % k_bufs].copy_(src[k % k_bufs]))}.items():
        ms = launch_time_ms(fn, stream, reps=args.steps, warmup=args.warmup)
        res[name] = {"kernel_ms": round(ms, 5), "GBps": round(moved / (ms * 1e-3) / 1e9, 1)}
    # the kernels did what they say
    hd.df11_stream_copy(src[0], dst[0], nbytes, stream=stream)
    hd.df11_stream_read(src[0], slots, nbytes, stream=stream)
    torch.cuda.synchronize()
    import numpy as np
    want = int(np.bitwise_xor.reduce(src[0].cpu().numpy()))
    got = int(np.bitwise_xor.reduce(slots.cpu().numpy()))
    res["ok"] = bool(torch.equal(src[0], dst[0])) and got == want
    print(json.dumps(res), flush=True)
    return 0 if res["ok"] else 1


def launch_time_ms(launch, stream, reps=20, warmup=300) -> float:
    """Average duration of launch(k) over `reps` back-to-back calls between one
    pair of events on `stream`, after `warmup` untimed calls (after an idle
    stretch, such as a host-side encode, the GPU's clocks take over a hundred
    back-to-back launches of ~0.1 ms to settle: a kernel trace of the tiled
    product showed launches 20-50 at 129 us and launch 110 still falling, at
    111 us)."""
    import torch
    for k in range(warmup):
        launch(k)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for k in range(reps):
        launch(k)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def captured(fn, outputs=None, replays=3):
    """fn() captured in a HIP graph (torch.cuda.CUDAGraph), so that its many
    small launches replay with no host overhead in between.  Returns the
    graph.  The graph is used only if it gives what the eager calls give:
    the outputs (those passed, else the tensors fn returns) are overwritten
    with a byte pattern before each of a few replays, with the program's own
    work in between, and must then equal an eager run's."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        eager = fn()  # also warms the libraries outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    expect = [t.clone() for t in (outputs if outputs is not None else eager)]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = fn()
    outs = list(outputs if outputs is not None else outs)
    for _ in range(replays):
        for t in outs:
            t.view(torch.uint8).fill_(0xA5)
        graph.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, e) for a, e in zip(outs, expect)):
            raise RuntimeError("a captured graph's replay differs from the eager result")
    return graph


def gemm_ratios(wlx, out, decode_ms, stream, batches=(1, 2, 4, 16, 64), reps=20) -> dict:
    """Decode time of the block over the time of the block's bf16 GEMMs
    (y = x W^T for each of its matrices, on the decoded weights) at each batch.
    The 7 GEMMs of a batch are replayed as one HIP graph: launched one by one
    from Python they would partly measure the host (about 20 us per GEMM)."""
    import torch
    res = {}
    mats, off = [], 0
    for m in wlx.matrices:
        mats.append(out[off: off + m.rows * m.cols].view(m.rows, m.cols))
        off += m.rows * m.cols
    g = torch.Generator(device=out.device).manual_seed(7)
    for b in batches:
        xs = [torch.randn(b, w.shape[1], device=out.device, generator=g).to(torch.bfloat16)
              for w in mats]

        def block_gemms():
            return [torch.nn.functional.linear(x, w) for x, w in zip(xs, mats)]
        graph = captured(block_gemms)
        gms = launch_time_ms(lambda _k: graph.replay(), stream, reps)
        # bytes a BF16 GEMM moves: the weights, x and y (bf16)
        moved = sum(2 * w.numel() + 2 * b * (w.shape[0] + w.shape[1]) for w in mats)
        # and the time those bytes take at the HBM peak: a floor for any BF16
        # GEMM on resident weights, which this library's GEMM does not reach
        res[f"batch{b}"] = {"gemm_ms": round(gms, 5), "decode_over_gemm": round(decode_ms / gms, 4),
                            "gemm_gbs": round(moved / (gms * 1e-3) / 1e9, 1),
                            "bf16_bytes_at_peak_ms": round(moved / (HBM_PEAK_GBS * 1e9) * 1e3, 5)}
        del graph
    return res


def run_stack(args) -> int:
    """The 32-block Llama-3.1-8B-shaped stack: each block decoded into a reused
    BF16 buffer, then its 7 bf16 GEMMs, at batches 1, 4, 16 and 64.  Reports
    the time of one forward pass (all blocks) for the decodes alone, the GEMMs
    alone on resident BF16 weights, decode+GEMMs on one stream, decode of
    block i+1 overlapped with the GEMMs of block i on two streams, and the
    fused products; and their ratios.  Every schedule runs as a captured HIP
    graph."""
    import numpy as np
    import torch
    import huffman_decode_amd as hd
    from huffman_decode_amd import workloads as wl
    from huffman_decode_amd.pipeline import StackBlock, StackRunner

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    blocks, resident, exact, t_enc = [], [], True, 0.0
    for layer in range(args.layers):
        wlx = wl.llama8b_stack_block(layer)
        t0 = time.perf_counter()
        enc = hd.encode(wlx.weights)
        d = hd.to_device(enc, dev)
        shapes = [(m.rows, m.cols) for m in wlx.matrices]
        te = hd.encode_tiled(wlx.weights, shapes)
        t_enc += time.perf_counter() - t0
        blocks.append(StackBlock(d, shapes, hd.tiled_to_device(te, dev)))
        del te
        # the decoded copy doubles as the resident BF16 weights of the GEMM-only pass
        buf = torch.empty(enc.n, dtype=torch.bfloat16, device=dev)
        hd.df11_decode(d, buf)
        orig = torch.from_numpy(wlx.weights.view(np.int16)).to(dev)
        exact &= bool(torch.equal(buf.view(torch.int16), orig))
        resident.append(buf)
        del orig, wlx, enc
        print(f"[stack] layer {layer} encoded and checked", file=sys.stderr, flush=True)
    runner = StackRunner(blocks, dev)
    cs = runner.compute_stream

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cs)
        for _ in range(reps):
            fn()
        e1.record(cs)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # Every schedule is replayed as a HIP graph (hundreds of small launches
    # per forward pass would otherwise partly time the host); the overlapped
    # one forks to the decode stream and joins back inside its graph.  Each
    # graph's replays are checked against the eager outputs first.
    def graphed(fn, outputs):
        g = captured(fn, outputs)
        return lambda: g.replay(), g

    res = {}
    for batch in (1, 4, 16, 64):
        acts, outs = runner.activations(batch)
        outs_list = list(outs.values())
        run, g1 = graphed(runner.run_decodes_only, runner.buffers)
        t_dec = timed(run, args.steps)
        run, g2 = graphed(lambda: runner.run_gemms_only(acts, outs, resident), outs_list)
        t_gemm = timed(run, args.steps)
        run, g3 = graphed(lambda: runner.run_serial(acts, outs), outs_list)
        t_ser = timed(run, args.steps)
        del g1, g2, g3
        t_ovl = {}
        for cap in (0, 512, 384, 256):
            run, g6 = graphed(lambda cap=cap: runner.run_overlapped(acts, outs, cap), outs_list)
            t_ovl[cap] = timed(run, args.steps)
            del g6
        best = min(t_ovl, key=t_ovl.get)
        # the fused product in place of decode-then-GEMM (small batches only)
        t_fused = None
        if batch <= 4:
            fm, fx, fy, fws = runner.fused_inputs(batch)
            run, g4 = graphed(lambda: runner.run_fused(fm, fx, fy, fws), [fy])
            t_fused = timed(run, args.steps)
            del fx, fy, fws, g4
        tx, ty, tws = runner.tiled_inputs(batch)
        run, g5 = graphed(lambda: runner.run_fused_tiled(tx, ty, tws), [ty])
        t_tiled = timed(run, args.steps)
        del tx, ty, tws, g5
        res[f"batch{batch}"] = {
            "forward_ms": {"decode_only": round(t_dec, 4), "bf16_gemm_only": round(t_gemm, 4),
                           "df11_serial": round(t_ser, 4),
                           "df11_fused_tiled": round(t_tiled, 4),
                           "df11_overlapped_by_decode_groups": {str(g): round(t, 4)
                                                                for g, t in t_ovl.items()}},
            "df11_fused_tiled_over_bf16": round(t_tiled / t_gemm, 4),
            "decode_over_gemm": round(t_dec / t_gemm, 4),
            "df11_serial_over_bf16": round(t_ser / t_gemm, 4),
            "df11_overlapped_over_bf16": round(t_ovl[best] / t_gemm, 4),
            "overlap_decode_groups": best}
        if t_fused is not None:
            res[f"batch{batch}"]["forward_ms"]["df11_fused"] = round(t_fused, 4)
            res[f"batch{batch}"]["df11_fused_over_bf16"] = round(t_fused / t_gemm, 4)
    n = sum(b.dev.n for b in blocks)
    print(json.dumps({"mode": "stack", "workload": "llama8b_stack", "layers": args.layers,
                      "n_weights": n, "bit_exact": exact, "host_encode_s": round(t_enc, 2),
                      "reps": args.steps, **res}), flush=True)
    return 0 if exact else 1


def run_encode(args) -> int:
    """Host encoder throughput: histogram, code book, tables and encoded arrays
    of one transformer block (df11_encode and its helpers, no GPU), with all
    hardware threads and with one, next to the single-thread per-block times
    the DF11 pages report for their Python compressor (191 s for an 8B block,
    547 s for a 70B block)."""
    import numpy as np
    import huffman_decode_amd as hd
    from huffman_decode_amd import workloads as wl
    import oracle
    pages_s = {"llama8b_block": 191.0, "llama70b_block": 547.0}
    out = {"mode": "encode", "host_threads": os.cpu_count(), "blocks": {}}
    ok = True
    for name in ("llama8b_block", "llama70b_block"):
        wlx = wl.CONFIGS[name]()
        row = {"n_weights": wlx.n, "pages_single_thread_s": pages_s[name]}
        for threads in (0, 1):
            t0 = time.perf_counter()
            enc = hd.encode(wlx.weights, n_threads=threads)
            dt = time.perf_counter() - t0
            key = "all_threads" if threads == 0 else "one_thread"
            row[key] = {"seconds": round(dt, 3), "gweights_per_s": round(wlx.n / dt / 1e9, 4),
                        "speedup_vs_pages": round(pages_s[name] / dt, 1)}
        # the encoding must be the oracle's, byte for byte, on a sample of it
        row["code_plus_signmant_bits_per_weight"] = round(8 + enc.sizes.total_bits / enc.n, 4)
        k = min(enc.n, 1 << 22)
        ref = oracle.encode(wlx.weights[:k])
        same = bool(np.array_equal(hd.encode(wlx.weights[:k]).stream[:ref.stream.size], ref.stream))
        row["matches_oracle_on_first_4M"] = same
        ok &= same
        out["blocks"][name] = row
        print(f"[encode] {name} done", file=sys.stderr, flush=True)
    print(json.dumps(out), flush=True)
    return 0 if ok else 1


def fused_gemv(wlx, copies, stream, reps=20) -> dict:
    """Batch-1 y = W x straight from the DF11 stream (df11_decode_gemv, no BF16
    weights in memory), timed over back-to-back launches like the decode."""
    import numpy as np
    import torch
    import huffman_decode_amd as hd
    shapes = [(m.rows, m.cols) for m in wlx.matrices]
    mats, nx, ny = hd.gemv_matrices(shapes)
    dev0 = copies[0]
    x = torch.from_numpy(np.random.default_rng(7).standard_normal(nx).astype(np.float32)).cuda()
    x = x.to(torch.bfloat16)
    y = torch.empty(ny, dtype=torch.float32, device="cuda")
    ws = torch.empty(hd.df11_gemv_workspace_bytes(dev0), dtype=torch.uint8, device="cuda")
    ms = launch_time_ms(lambda k: hd.df11_decode_gemv(copies[k % len(copies)], mats, x, y, ws,
                                                      stream), stream, reps)
    return {"fused_ms": round(ms, 5)}


def fused_gemm(wlx, copies, stream, batch, reps=20) -> dict:
    """y_b = W x_b for `batch` vectors straight from the DF11 stream
    (df11_decode_gemm), timed over back-to-back launches like the decode."""
    import numpy as np
    import torch
    import huffman_decode_amd as hd
    shapes = [(m.rows, m.cols) for m in wlx.matrices]
    mats, nx, ny = hd.gemv_matrices(shapes)
    x = torch.from_numpy(np.random.default_rng(8).standard_normal((batch, nx)).astype(np.float32))
    x = x.cuda().to(torch.bfloat16)
    y = torch.empty(batch, ny, dtype=torch.float32, device="cuda")
    ws = torch.empty(hd.df11_gemm_workspace_bytes(copies[0], batch), dtype=torch.uint8, device="cuda")
    ms = launch_time_ms(lambda k: hd.df11_decode_gemm(copies[k % len(copies)], mats, x, y, ws,
                                                      stream), stream, reps)
    return {"fused_ms": round(ms, 5)}


def fused_tiled(wlx, stream, batches, n_copies=3, reps=20, warmup=300) -> dict:
    """y_b = W x_b for `batch` vectors on the matrix cores from the block
    encoded in operand-tile order (df11_decode_gemm_tiled), and the decode of
    that stream back to row-major BF16 (df11_decode_tiled), timed over
    back-to-back launches on rotating copies like the decode."""
    import numpy as np
    import torch
    import huffman_decode_amd as hd
    shapes = [(m.rows, m.cols) for m in wlx.matrices]
    te = hd.encode_tiled(wlx.weights, shapes)
    copies = [hd.tiled_to_device(te, "cuda") for _ in range(n_copies)]
    nx = max(m.x_offset + m.cols for m in te.mats)
    ny = sum(m.rows for m in te.mats)
    rd, wr = algorithmic_bytes(te.enc)
    res = {}
    # the decode of the same stream back to row-major BF16 (df11_decode_tiled)
    out = torch.empty(te.enc.n, dtype=torch.int16, device="cuda")
    ms = launch_time_ms(lambda k: hd.df11_decode_tiled(copies[k % n_copies], out, stream), stream,
                        reps, warmup)
    res["decode_row_major"] = {"ms": round(ms, 5), "gbs": round((rd + wr) / (ms * 1e-3) / 1e9, 1)}
    del out
    for batch in batches:
        x = torch.from_numpy(np.random.default_rng(9).standard_normal((batch, nx)).astype(np.float32))
        x = x.cuda().to(torch.bfloat16)
        y = torch.empty(batch, ny, dtype=torch.float32, device="cuda")
        need = hd.df11_tiled_workspace_bytes(te.mats, batch)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
        ms = launch_time_ms(lambda k: hd.df11_decode_gemm_tiled(copies[k % n_copies], x, y, ws,
                                                                stream), stream, reps, warmup)
        res[f"batch{batch}"] = {"fused_ms": round(ms, 5),
                                "fused_gbs": round((rd + 2 * batch * nx + 4 * batch * ny)
                                                   / (ms * 1e-3) / 1e9, 1)}
    return res


def run_tiled(args) -> int:
    """Only the tiled product (df11_decode_gemm_tiled) on the workload at each
    of --batches, with --warmup and --steps launches (a short run for counter
    collection)."""
    import torch
    from huffman_decode_amd import workloads as wl
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wlx = wl.CONFIGS[args.workload]()
    batches = [int(b) for b in args.batches.split(",")]
    stream = torch.cuda.current_stream(dev)
    res = fused_tiled(wlx, stream, batches, reps=args.steps, warmup=args.warmup)
    if args.decode_cols:
        # the row-major decode of the same words laid out as one matrix of
        # each width: at 32 columns a tile is 1 KB of contiguous output, from
        # 64 on each tile writes 64 bytes of each of its 16 rows
        import huffman_decode_amd as hd
        rd, wr = algorithmic_bytes(hd.encode(wlx.weights))
        for c in (int(v) for v in args.decode_cols.split(",")):
            if wlx.n % (16 * c):
                raise SystemExit(f"{wlx.n} weights do not make {c}-column rows in 16-row tiles")
            te = hd.encode_tiled(wlx.weights, [(wlx.n // c, c)])
            td = hd.tiled_to_device(te, "cuda")
            out = torch.empty(wlx.n, dtype=torch.int16, device="cuda")
            ms = launch_time_ms(lambda k: hd.df11_decode_tiled(td, out, stream), stream,
                                args.steps, args.warmup)
            res[f"decode_cols{c}"] = {"ms": round(ms, 5),
                                      "gbs": round((rd + wr) / (ms * 1e-3) / 1e9, 1)}
            del td, out
    print(json.dumps({"mode": "tiled", "workload": args.workload, "steps": args.steps,
                      "warmup": args.warmup, **res}), flush=True)
    return 0


def run_offload(args) -> int:
    """CPU offload over the 8B-shaped stack: compressed blocks in pinned host
    memory, each copied to the GPU and decoded in turn (copies overlapped with
    the previous block's decode).  Reports the PCIe-inclusive time per block
    next to the decode of device-resident blocks."""
    import numpy as np
    import torch
    import huffman_decode_amd as hd
    from huffman_decode_amd import workloads as wl
    from huffman_decode_amd.pipeline import OffloadRunner

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    encs, origs = [], []
    for layer in range(args.layers):
        wlx = wl.llama8b_stack_block(layer)
        encs.append(hd.encode(wlx.weights))
        origs.append(wlx.weights[:: 997].copy())  # a sample to check against
        print(f"[offload] layer {layer} encoded", file=sys.stderr, flush=True)
    sums = [e.checksum() for e in encs]
    runner = OffloadRunner(encs, sums, dev)
    exact = True

    def check(i, out):
        nonlocal exact
        got = out[:: 997].view(torch.int16).cpu().numpy().view(np.uint16)
        exact &= bool(np.array_equal(got, origs[i]))

    runner.run(check)
    torch.cuda.synchronize()
    cs = runner.compute_stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    runner.run()
    torch.cuda.synchronize()
    e0.record(cs)
    for _ in range(args.steps):
        runner.run()
    e1.record(cs)
    torch.cuda.synchronize()
    t_off = e0.elapsed_time(e1) / args.steps
    # the same blocks resident in device memory
    resident = [hd.to_device(e, dev) for e in encs]
    buf = runner.buffers[0]
    for d in resident:
        hd.df11_decode(d, buf)
    torch.cuda.synchronize()
    e0.record(cs)
    for _ in range(args.steps):
        for d in resident:
            hd.df11_decode(d, buf)
    e1.record(cs)
    torch.cuda.synchronize()
    t_res = e0.elapsed_time(e1) / args.steps
    comp = sum(e.compressed_bytes() for e in encs)
    n = sum(e.n for e in encs)
    print(json.dumps({"mode": "offload", "workload": "llama8b_stack", "layers": args.layers,
                      "n_weights": n, "compressed_bytes": comp, "bit_exact_sampled": exact,
                      "offload_ms_per_block": round(t_off / args.layers, 4),
                      "resident_ms_per_block": round(t_res / args.layers, 4),
                      "host_to_device_GBps": round(comp / (t_off * 1e-3) / 1e9, 2),
                      "offload_over_resident": round(t_off / t_res, 3)}), flush=True)
    return 0 if exact else 1


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 100 for decode and copy, else 20)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps first (default 300 for decode and copy: the GPU's "
                         "clocks take ~100 back-to-back launches to ramp up; else 3)")
    ap.add_argument("--workload", default="llama8b_block")
    ap.add_argument("--copies", type=int, default=0,
                    help="rotating encoded copies and output buffers (0: enough that they "
                         "span at least 768 MB, three times the 256 MB Infinity Cache, and "
                         "at least 3)")
    ap.add_argument("--max-groups", type=int, default=0,
                    help="cap on the decode's workgroups (0: as many as fit on the GPU)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm", action="store_true", help="skip the decode/GEMM ratios")
    ap.add_argument("--mode", choices=("decode", "copy", "stack", "encode", "offload", "ceiling",
                                       "tiled", "stream"),
                    default="decode",
                    help="ceiling: only the traffic-only kernel on the workload's bytes; "
                         "stream: the GPU's read-only, write-only and copy rates over "
                         "--copy-mib MiB; "
                         "tiled: only the tiled product at --batches; "
                         "copy: time a plain device copy of --copy-mib MiB instead; "
                         "stack: decode/GEMM schedules over the 32-block 8B-shaped stack; "
                         "encode: host encoder throughput (no GPU); "
                         "offload: blocks from pinned host memory, copied and decoded in turn")
    ap.add_argument("--layers", type=int, default=32, help="blocks in the stack mode")
    ap.add_argument("--batches", default="1,16,64", help="vectors per call in the tiled mode")
    ap.add_argument("--decode-cols", default="",
                    help="tiled mode: also time the row-major decode of the workload's words "
                         "laid out as one matrix of each of these widths (comma separated)")
    ap.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args()
    fast = args.mode in ("decode", "copy", "ceiling", "stream")
    if args.steps is None:
        args.steps = 100 if fast else 20
    if args.warmup is None:
        args.warmup = 300 if fast else 3

    if args.gpus != 1:
        print(json.dumps({"error": "df11_decode is measured on one GPU only (--gpus 1); "
                                   "across GPUs the decode shards by whole blocks with no "
                                   "communication, so no multi-GPU figure is produced"}))
        return 2

    if args.mode == "copy":
        return run_copy(args)
    if args.mode == "stack":
        return run_stack(args)
    if args.mode == "encode":
        return run_encode(args)
    if args.mode == "offload":
        return run_offload(args)
    if args.mode == "tiled":
        return run_tiled(args)
    if args.mode == "stream":
        return run_stream(args)

    import numpy as np
    import torch
    import huffman_decode_amd as hd
    from huffman_decode_amd import workloads as wl

    if not os.path.exists(hd.LIB_PATH):
        from huffman_decode_amd.build import build_library
        build_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t0 = time.perf_counter()
    wlx = wl.CONFIGS[args.workload]()
    enc = hd.encode(wlx.weights)
    t_enc = time.perf_counter() - t0
    n = enc.n
    rd, wr = algorithmic_bytes(enc)
    # rotating copies of the inputs and of the output, so that a launch finds
    # nothing of its bytes in the 256 MB Infinity Cache from the launch before
    n_copies = args.copies or max(3, -(-768_000_000 // (rd + wr)))
    copies = [hd.to_device(enc, dev) for _ in range(n_copies)]
    for c in copies:
        c.desc.max_groups = args.max_groups
    outs = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(n_copies)]
    stream = torch.cuda.current_stream(dev)

    def timed(launch, steps, warmup):
        """Average duration of `launch(k)` over `steps` back-to-back launches
        between one pair of events on the launch stream (no markers between
        launches, which would add their own gaps)."""
        for k in range(warmup):
            launch(k)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        e0.record(stream)
        for k in range(steps):
            launch(k)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps, time.perf_counter() - w0

    # the traffic-only kernel on the same bytes: sign|mantissa and the output
    # with the decode's widths, the rest of the decode's reads from a buffer
    # of exactly that size (per copy)
    n8 = n & ~7
    b_bytes = (rd - n) // 16 * 16
    extras = [torch.empty(b_bytes, dtype=torch.uint8, device=dev).fill_(k + 1)
              for k in range(n_copies)]

    def ceiling(k):
        c = k % n_copies
        hd.df11_stream_ceiling(copies[c].tensors["signmant"], extras[c], outs[c], n8, 0, stream)

    if args.mode == "ceiling":
        c_ms, _ = timed(ceiling, args.steps, args.warmup)
        cb = n8 + b_bytes + 2 * n8
        print(json.dumps({"mode": "ceiling", "workload": args.workload, "kernel_ms": round(c_ms, 5),
                          "bytes": cb, "GBps": round(cb / (c_ms * 1e-3) / 1e9, 1),
                          "copies": n_copies}), flush=True)
        return 0

    def decode(k):
        c = k % n_copies
        hd.df11_decode(copies[c], outs[c], stream)

    avg_ms, wall = timed(decode, args.steps, args.warmup)
    gbs = (rd + wr) / (avg_ms * 1e-3) / 1e9
    orig = torch.from_numpy(wlx.weights.view(np.int16)).to(dev)
    # every output buffer the launches wrote (the k-th launch writes buffer k % copies)
    written = outs[: min(n_copies, max(args.steps, args.warmup))]
    bit_exact = all(bool(torch.equal(o.view(torch.int16), orig)) for o in written)
    del orig
    traffic = measured_traffic(rd + wr)
    # single launches, each between its own pair of events (after the timed
    # region; the events add gaps between launches, so these give the spread,
    # while `value` comes from the back-to-back mean above)
    singles = []
    for k in range(20):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        decode(k)
        b.record(stream)
        singles.append((a, b))
    torch.cuda.synchronize()
    singles = sorted(a.elapsed_time(b) for a, b in singles)
    # the exponent histogram's entropy: the floor of the average code length
    hist = hd.df11_histogram(wlx.weights).astype(np.float64)
    prob = hist[hist > 0] / hist.sum()
    entropy = float(-(prob * np.log2(prob)).sum())
    # the ceiling, timed right after the decode on the same copies and buffers
    c_ms, _ = timed(ceiling, args.steps, 20)
    ceiling_gbs = (n8 + b_bytes + 2 * n8) / (c_ms * 1e-3) / 1e9
    for c in range(n_copies):  # the decoded weights again, for the GEMM ratios
        decode(c)
    torch.cuda.synchronize()
    out = outs[0]

    line = {
        "metric": "df11_decode effective HBM GB/s + Gweights/s on 1 MI355X; % of HBM roofline",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "gweights_per_s": round(n / (avg_ms * 1e-3) / 1e9, 2),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "kernel_ms": {"mean": round(avg_ms, 5),
                      "single_launches": {"count": len(singles),
                                          "median": round(singles[len(singles) // 2], 5),
                                          "min": round(singles[0], 5),
                                          "max": round(singles[-1], 5)}},
        "bit_exact": bit_exact,
        "config": {"workload": args.workload, "n_weights": n,
                   "matrices": [f"{m.name}:{m.rows}x{m.cols}" for m in wlx.matrices],
                   "bits_per_weight": round(8 * (rd - int(enc.sizes.lut_bytes)) / n, 4),
                   "total_code_bits": int(enc.sizes.total_bits),
                   "exponent_entropy_bits": round(entropy, 4),
                   "avg_code_bits": round(int(enc.sizes.total_bits) / n, 4),
                   "max_code_len": int(enc.codebook.max_len),
                   "n_tables": int(enc.codebook.n_tables),
                   "rotating_copies": n_copies, "max_groups": args.max_groups,
                   "resident_bytes_rotated": n_copies * (rd + wr),
                   "host_encode_s": round(t_enc, 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "bytes_per_launch": {"read": rd, "written": wr},
                     "ceiling_gbs": round(ceiling_gbs, 1),
                     "ceiling_ms": round(c_ms, 5),
                     "frac_of_ceiling": round(gbs / ceiling_gbs, 4)},
    }
    if not args.no_gemm:
        line["decode_vs_gemm"] = gemm_ratios(wlx, out, avg_ms, stream)
        # The fused products against the BF16 GEMMs on resident weights and
        # against decoding first and then running those GEMMs:
        #   fused: the library's product for 1-64 vectors on the matrix cores
        #     (df11_decode_gemm_tiled), from the block encoded in operand-tile
        #     order (the same code book and compressed size);
        #   fused_row_major: the product on the row-major stream itself
        #     (df11_decode_gemv at batch 1, df11_decode_gemm at 2 and 4).
        # The bytes a fused product must move: the compressed weights, x (bf16)
        # and y (fp32).
        nx = sum(m.cols for m in wlx.matrices)
        ny = sum(m.rows for m in wlx.matrices)

        def priced(f, b):
            g = line["decode_vs_gemm"][f"batch{b}"]["gemm_ms"]
            f["over_bf16_gemm"] = round(f["fused_ms"] / g, 4)
            f["over_decode_then_gemm"] = round(f["fused_ms"] / (avg_ms + g), 4)
            f["over_bf16_bytes_at_peak"] = round(
                f["fused_ms"] / line["decode_vs_gemm"][f"batch{b}"]["bf16_bytes_at_peak_ms"], 4)
            f["fused_gbs"] = round((rd + 2 * b * nx + 4 * b * ny) / (f["fused_ms"] * 1e-3) / 1e9, 1)
            f["frac_of_hbm_peak"] = round(f["fused_gbs"] / HBM_PEAK_GBS, 4)
            return f

        tiled = fused_tiled(wlx, stream, (1, 2, 4, 16, 64))
        tile_decode = tiled.pop("decode_row_major")
        fused = {"path": "df11_decode_gemm_tiled (operand-tile-order stream)"}
        for key, f in tiled.items():
            fused[key] = priced(f, int(key[len("batch"):]))
        line["decode_vs_gemm"]["fused"] = fused
        row_major = {"path": "df11_decode_gemv / df11_decode_gemm (row-major stream)"}
        for b in (1, 2, 4):
            f = fused_gemv(wlx, copies, stream) if b == 1 else fused_gemm(wlx, copies, stream, b)
            row_major[f"batch{b}"] = priced(f, b)
        line["decode_vs_gemm"]["fused_row_major"] = row_major
        # the tile-order stream decoded back to row-major BF16 (df11_decode_tiled)
        line["decode_vs_gemm"]["tile_order_decode"] = {"path": "df11_decode_tiled", **tile_decode}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wlx, enc)
    print(json.dumps(line), flush=True)
    return 0 if bit_exact else 1


if __name__ == "__main__":
    sys.exit(main())
