#!/usr/bin/env python3
"""Throughput of df11_decode on one MI355X.

One step = one df11_decode launch over a whole transformer block's linear
weights (one code book, one stream), from DF11 arrays resident in HBM to BF16
words in HBM.  The default workload is the Llama-3.1-8B-shaped block (q/o
4096x4096, k/v 1024x4096, gate/up 14336x4096, down 4096x14336; 218,103,808
weights, N(0, sigma_m) with per-matrix sigma jitter).  R identical encoded
copies at different addresses are decoded in turn so that the 256 MB
Infinity Cache cannot hold a step's inputs from the previous use.

Prints one JSON line.  value = effective GB/s = (algorithmic bytes read +
2n bytes written) / device time of one launch, where the bytes read are the
code stream (total_bits / 8), the 5-bit gaps, the block positions, the n
sign|mantissa bytes and the lookup tables.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak (vendor figure)
KERNEL_SOURCE = os.path.join(ROOT, "huffman_decode_amd", "csrc", "df11_decode.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "df11_decode_llama8b_block_traffic.txt")


def kernel_hash() -> str:
    """Hash of the kernel source's code: comments and whitespace are dropped
    first, so that only a change to the code itself retires the counters."""
    with open(KERNEL_SOURCE) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = "".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


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
    if vals.get("kernel_sha256_16") != kernel_hash():
        return None
    try:
        if int(vals["algorithmic_bytes_per_launch"]) != int(n_launch_bytes):
            return None
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(wlx, enc) -> dict:
    """The oracle's serial bit-by-bit decode + join over the whole block, one core."""
    import numpy as np
    import oracle
    n = int(enc.sizes.n)
    t0 = time.perf_counter()
    ex, end = oracle.decode(enc.stream, int(enc.sizes.total_bits), 0, n, enc.codebook.lengths)
    w = oracle.join_bf16(ex, enc.signmant[:n])
    dt = time.perf_counter() - t0
    ok = bool(np.array_equal(w, wlx.weights)) and end == int(enc.sizes.total_bits)
    rd, wr = algorithmic_bytes(enc)
    return {"value": round((rd + wr) / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle", "gweights_per_s": round(n / dt / 1e9, 5), "seconds": round(dt, 2),
            "bit_exact": ok,
            "sample": f"whole {wlx.name} ({n} weights): oracle serial tree-walk decode "
                      f"of every code from bit 0, then BF16 join, 1 thread"}


def run_copy(args) -> int:
    """A plain device-to-device copy of known size: the reference that the HBM
    byte counters of a profiler run are scaled by."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    nbytes = args.copy_mib << 20
    src = torch.empty(nbytes // 2, dtype=torch.int16, device=dev).random_(-100, 100)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_begin.record(stream)
    for k in range(args.steps):
        dst.copy_(src)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_begin.elapsed_time(t_end) / args.steps
    print(json.dumps({"mode": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                      "kernel_ms": round(ms, 5),
                      "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1),
                      "ok": bool(torch.equal(src, dst))}), flush=True)
    return 0


def gemm_ratios(wlx, out, decode_ms, stream, batches=(1, 2, 4, 64), reps=10) -> dict:
    """Decode time of the block over the time of the block's bf16 GEMMs
    (y = x W^T for each of its matrices, on the decoded weights) at each batch."""
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
        for _ in range(2):
            for x, w in zip(xs, mats):
                torch.nn.functional.linear(x, w)
        torch.cuda.synchronize()
        s0 = torch.cuda.Event(enable_timing=True)
        s1 = torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        for _ in range(reps):
            for x, w in zip(xs, mats):
                torch.nn.functional.linear(x, w)
        s1.record(stream)
        torch.cuda.synchronize()
        gms = s0.elapsed_time(s1) / reps
        res[f"batch{b}"] = {"gemm_ms": round(gms, 5), "decode_over_gemm": round(decode_ms / gms, 4)}
    return res


def run_stack(args) -> int:
    """The 32-block Llama-3.1-8B-shaped stack: each block decoded into a reused
    BF16 buffer, then its 7 bf16 GEMMs at batch 1 and 64.  Reports the time of
    one forward pass (all blocks) for the decodes alone, the GEMMs alone on
    resident BF16 weights, decode+GEMMs on one stream, and decode of block i+1
    overlapped with the GEMMs of block i on two streams; and their ratios."""
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
        t_enc += time.perf_counter() - t0
        d = hd.to_device(enc, dev)
        shapes = [(m.rows, m.cols) for m in wlx.matrices]
        blocks.append(StackBlock(d, shapes))
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

    res = {}
    for batch in (1, 4, 64):
        acts, outs = runner.activations(batch)
        t_dec = timed(runner.run_decodes_only, args.steps)
        t_gemm = timed(lambda: runner.run_gemms_only(acts, outs, resident), args.steps)
        t_ser = timed(lambda: runner.run_serial(acts, outs), args.steps)
        t_ovl = {g: timed(lambda: runner.run_overlapped(acts, outs, g), args.steps)
                 for g in (0, 512, 384, 256)}
        best = min(t_ovl, key=t_ovl.get)
        # the fused product in place of decode-then-GEMM (small batches only)
        t_fused = None
        if batch <= 4:
            fm, fx, fy, fws = runner.fused_inputs(batch)
            t_fused = timed(lambda: runner.run_fused(fm, fx, fy, fws), args.steps)
            del fx, fy, fws
        res[f"batch{batch}"] = {
            "forward_ms": {"decode_only": round(t_dec, 4), "bf16_gemm_only": round(t_gemm, 4),
                           "df11_serial": round(t_ser, 4),
                           "df11_overlapped_by_decode_groups": {str(g): round(t, 4)
                                                                for g, t in t_ovl.items()}},
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
    for k in range(3):
        hd.df11_decode_gemv(copies[k % len(copies)], mats, x, y, ws, stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for k in range(reps):
        hd.df11_decode_gemv(copies[k % len(copies)], mats, x, y, ws, stream)
    b.record(stream)
    torch.cuda.synchronize()
    return {"fused_ms": round(a.elapsed_time(b) / reps, 5)}


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
    for k in range(3):
        hd.df11_decode_gemm(copies[k % len(copies)], mats, x, y, ws, stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for k in range(reps):
        hd.df11_decode_gemm(copies[k % len(copies)], mats, x, y, ws, stream)
    b.record(stream)
    torch.cuda.synchronize()
    return {"fused_ms": round(a.elapsed_time(b) / reps, 5)}


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
    ap.add_argument("--copies", type=int, default=3,
                    help="rotating encoded copies (defeats the Infinity Cache)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm", action="store_true", help="skip the decode/GEMM ratios")
    ap.add_argument("--mode", choices=("decode", "copy", "stack", "encode", "offload"),
                    default="decode",
                    help="copy: time a plain device copy of --copy-mib MiB instead; "
                         "stack: decode/GEMM schedules over the 32-block 8B-shaped stack; "
                         "encode: host encoder throughput (no GPU); "
                         "offload: blocks from pinned host memory, copied and decoded in turn")
    ap.add_argument("--layers", type=int, default=32, help="blocks in the stack mode")
    ap.add_argument("--copy-mib", type=int, default=1024)
    args = ap.parse_args()
    fast = args.mode in ("decode", "copy")
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
    copies = [hd.to_device(enc, dev) for _ in range(max(1, args.copies))]
    out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)

    for k in range(args.warmup):
        hd.df11_decode(copies[k % len(copies)], out, stream)
    torch.cuda.synchronize()

    # Timed region: K launches back to back between one pair of events on the
    # launch stream (no markers between launches, which would add their own
    # gaps); the average launch duration is the region's time over K.
    t_begin, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record(stream)
    for k in range(args.steps):
        hd.df11_decode(copies[k % len(copies)], out, stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    avg_ms = t_begin.elapsed_time(t_end) / args.steps
    rd, wr = algorithmic_bytes(enc)
    gbs = (rd + wr) / (avg_ms * 1e-3) / 1e9
    orig = torch.from_numpy(wlx.weights.view(np.int16)).to(dev)
    bit_exact = bool(torch.equal(out.view(torch.int16), orig))
    traffic = measured_traffic(rd + wr)

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
        "kernel_ms": {"mean": round(avg_ms, 5)},
        "bit_exact": bit_exact,
        "config": {"workload": args.workload, "n_weights": n,
                   "matrices": [f"{m.name}:{m.rows}x{m.cols}" for m in wlx.matrices],
                   "bits_per_weight": round(8 * (rd - int(enc.sizes.lut_bytes)) / n, 4),
                   "total_code_bits": int(enc.sizes.total_bits),
                   "max_code_len": int(enc.codebook.max_len),
                   "n_tables": int(enc.codebook.n_tables),
                   "rotating_copies": len(copies), "host_encode_s": round(t_enc, 2)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "bytes_per_launch": {"read": rd, "written": wr}},
    }
    if not args.no_gemm:
        line["decode_vs_gemm"] = gemm_ratios(wlx, out, avg_ms, stream)
        # the fused product (df11_decode_gemv at batch 1, df11_decode_gemm at
        # 2 and 4) against the BF16 GEMMs on resident weights and against
        # decoding first and then running those GEMMs
        fused = {}
        for b in (1, 2, 4):
            f = fused_gemv(wlx, copies, stream) if b == 1 else fused_gemm(wlx, copies, stream, b)
            g = line["decode_vs_gemm"][f"batch{b}"]["gemm_ms"]
            f["over_bf16_gemm"] = round(f["fused_ms"] / g, 4)
            f["over_decode_then_gemm"] = round(f["fused_ms"] / (avg_ms + g), 4)
            fused[f"batch{b}"] = f
        line["decode_vs_gemm"]["fused"] = fused
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wlx, enc)
    print(json.dumps(line), flush=True)
    return 0 if bit_exact else 1


if __name__ == "__main__":
    sys.exit(main())
