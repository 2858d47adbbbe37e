"""Benchmark of the fused exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic inputs:
  1. causal MHA prefill, bf16, B=4 A=A_kv=32 S_q=S_k=2048 d=128 (the headline
     workload: `value` is its causal-adjusted TFLOP/s),
  2. paged single-query decode, bf16, 64 sequences with lengths ~U{512..32768},
     page 16, A=32 A_kv=8 d=128 (split + LSE merge; KV GB/s),
  3. packed varlen causal prefill, bf16, 16 log-normal sequences, A=16 d=64,
     5% of query rows fully masked (causal-adjusted TFLOP/s),
  4. long GQA causal prefill, bf16, B=1 A=32 A_kv=8 S_q=S_k=16384 d=128, V~U(-1,1)
     (causal-adjusted TFLOP/s, with its own roofline object under "gqa_long").
Inputs are resident in HBM before the timed region.  Each launch is bracketed
by HIP events recorded on the stream the library launches on.

After the timed steps, the next-step variants are timed on their own, each
under its own key (none is part of a step): "backward" (dQ, dK, dV of
workload 1 recomputed from the forward's LSE), "window" (GQA causal S=16384
with a 4096-key sliding window), "paged_prefill" (256-token chunks over the
decode workload's paged cache), "block_sparse" (workload 1 with a 50% block
mask), "dense_mask" (workload 1 with a general dense additive mask: packed
documents with their derived block mask, and a per-head distance penalty),
"key_range" (workload 1 with per-row key ranges: the same documents, forward
and backward, and prefix-LM), "alibi" (workload 1 with ALiBi computed in the
kernels, forward and backward) and
"decode_fp8" (workload 2 over E4M3 caches with per-(page, head) scales).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints one JSON line.

HBM traffic of each kernel comes from hardware-counter runs over a fixed
workload, scaled by what the same counters read for a plain device-to-device
copy of known size.  Reads are the L2-to-fabric read requests priced by their
size (TCC_EA0_RDREQ_32B/_64B/_128B: on gfx950 the FETCH_SIZE expression counts
128-byte requests as 64 bytes); writes are WRITE_SIZE; FETCH_SIZE itself is
reported beside them:

    rocprofv3 --pmc TCC_EA0_RDREQ_32B TCC_EA0_RDREQ_64B TCC_EA0_RDREQ_128B -f csv -d <dir_r> -o p -- python3 bench.py --traffic-workload
    rocprofv3 --pmc WRITE_SIZE -f csv -d <dir_w> -o p -- python3 bench.py --traffic-workload
    rocprofv3 --pmc FETCH_SIZE -f csv -d <dir_f> -o p -- python3 bench.py --traffic-workload
    python3 bench.py --traffic-summary <dir_r> <dir_w> <dir_f> > profiles/traffic_<...>.md

The summary records a hash of the code of each kernel's sources (comments and
layout excluded); a later bench run reports `traffic` only while that code is
unchanged (null otherwise).

Per-workload kernel times from one kernel trace of this same command (the
dense prefill kernel serves three workloads; they are told apart by grid size):

    rocprofv3 --kernel-trace --stats -f csv -d <dir_t> -o bench -- python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline
    python3 bench.py --trace-summary <dir_t> > profiles/kernel_trace_<...>.md

Matrix-core utilisation of the prefill kernels, from one counter run:

    rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_ANY -f csv -d <dir_m> -o p -- python3 bench.py --traffic-workload
    python3 bench.py --counter-summary <dir_m> > profiles/mfma_<...>.md
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (causal-adjusted) + paged-decode KV GB/s, % roofline"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
CSRC = os.path.join(ROOT, "exact_attention_108_amd", "csrc")
# sources that determine each timed kernel's memory traffic
KERNEL_SOURCES = {
    "prefill": ["attn_prefill_bf16.hip", "attn_device.h", "attn_kernels.h", "attn_rowblock.h"],
    "decode": ["attn_decode_bf16.hip", "attn_device.h", "attn_kernels.h"],
    "backward": ["attn_bwd_bf16.hip", "attn_bwd.h", "attn_device.h"],
}
COPY_BYTES = 1 << 30  # the reference copy kernel moves this many bytes each way


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def to_dev(x, kind):
    import torch
    if kind == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def code_text(src: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed, so that
    an edit of comments or layout leaves the hash of the code unchanged."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":  # string or character literal, copied whole
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_hash(part: str) -> str:
    """Hash of the code (comments and layout excluded) of the sources that
    determine `part`'s kernels."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[part]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def committed_traffic(part: str, sources: str = None):
    """HBM bytes per launch of `part`'s kernel from the newest traffic summary
    under profiles/ whose recorded source hash matches the current sources
    (those of `sources`, by default of `part`)."""
    want = source_hash(sources or part)
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md")), reverse=True):
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    rec = json.loads(line[len("traffic-json: "):])
                    ent = rec.get(part)
                    if ent and ent.get("source_hash") == want:
                        return ent["bytes_per_launch"], os.path.basename(path)
    return None, None


def load_inputs(log_fn=lambda *a: None):
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    t0 = time.time()
    p2 = gen.make_config(2)
    q2, k2, v2 = to_dev(p2.q, "bf16"), to_dev(p2.k, "bf16"), to_dev(p2.v, "bf16")
    o2 = torch.empty_like(q2)
    l2 = torch.empty((p2.B, p2.A, p2.S_q), dtype=torch.float32, device="cuda")
    log_fn(f"prefill inputs ready ({time.time() - t0:.1f}s)")

    t0 = time.time()
    p4 = gen.make_config(4)
    q4 = to_dev(p4.q, "bf16")
    kc4, vc4 = to_dev(p4.k_cache, "bf16"), to_dev(p4.v_cache, "bf16")
    bt4, sl4 = to_dev(p4.block_table, "i32"), to_dev(p4.seq_lens, "i32")
    o4 = torch.empty_like(q4)
    l4 = torch.empty((p4.B, p4.A), dtype=torch.float32, device="cuda")
    ws_bytes = ea.attn_decode_paged_workspace_bytes(p4.B, p4.A, p4.A_kv, p4.d, p4.page_size, p4.seq_lens)
    ws4 = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    kv_bytes = p4.kv_bytes()
    log_fn(f"decode inputs ready ({time.time() - t0:.1f}s): {kv_bytes / 1e9:.2f} GB of KV, "
           f"workspace {ws_bytes / 1e6:.1f} MB")

    t0 = time.time()
    p5 = gen.make_config(5)
    q5, k5, v5 = to_dev(p5.q, "bf16"), to_dev(p5.k, "bf16"), to_dev(p5.v, "bf16")
    o5 = torch.empty_like(q5)
    l5 = torch.empty((p5.A, p5.T), dtype=torch.float32, device="cuda")
    cu5 = to_dev(p5.cu_seqlens, "i32")
    qk5 = to_dev(p5.q_keep, "u8")
    log_fn(f"varlen inputs ready ({time.time() - t0:.1f}s): T={p5.T}")

    t0 = time.time()
    p3 = gen.make_config(3)
    q3, k3, v3 = to_dev(p3.q, "bf16"), to_dev(p3.k, "bf16"), to_dev(p3.v, "bf16")
    o3 = torch.empty_like(q3)
    l3 = torch.empty((p3.B, p3.A, p3.S_q), dtype=torch.float32, device="cuda")
    log_fn(f"long GQA prefill inputs ready ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def prefill():
        ea.attn_fwd(q2, k2, v2, o2, l2, scale=p2.scale, causal=True, stream=stream)

    def decode():
        ea.attn_decode_paged(q4, kc4, vc4, bt4, sl4, p4.seq_lens, o4, l4, ws4, scale=p4.scale, stream=stream)

    def varlen():
        ea.attn_fwd_varlen(q5, k5, v5, o5, l5, cu5, p5.cu_seqlens, scale=p5.scale, causal=True, q_keep=qk5,
                           stream=stream)

    def gqa_long():
        ea.attn_fwd(q3, k3, v3, o3, l3, scale=p3.scale, causal=True, stream=stream)

    return dict(p2=p2, p3=p3, p4=p4, p5=p5, kv_bytes=kv_bytes, ws_bytes=ws_bytes, stream=stream,
                dev2=(q2, k2, v2, o2, l2), dev4=(kc4, vc4, bt4, sl4),
                parts=[("prefill", prefill), ("decode", decode), ("varlen", varlen), ("gqa_long", gqa_long)])


def traffic_workload():
    """Each timed kernel three times, then a plain copy of COPY_BYTES three
    times (the counter scale reference); nothing is timed."""
    import torch
    torch.cuda.set_device(0)
    w = load_inputs()
    for name, fn in w["parts"]:
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
    bwd = backward_setup(w)
    for _ in range(3):
        bwd()
    torch.cuda.synchronize()
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("traffic workload done", flush=True)


def traffic_summary(dir_read: str, dir_write: str, dir_fetch: str):
    """Markdown summary of three counter runs of --traffic-workload."""
    import csv

    def per_kernel(d, value_of):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        assert files, f"no counter_collection.csv under {d}"
        by = {}
        for path in files:
            with open(path) as fh:
                for r in csv.DictReader(fh):
                    w = value_of(r["Counter_Name"])
                    if w is None:
                        continue
                    key = (r["Kernel_Name"], grid_of(r), r["Dispatch_Id"])
                    by[key] = by.get(key, 0.0) + w * float(r["Counter_Value"])
        out = {}
        for (kname, grid, _), v in by.items():
            out.setdefault((kname, grid), []).append(v)
        return out

    def mean(tab):
        return {k: sum(v) / len(v) for k, v in tab.items()}

    sizes = {"TCC_EA0_RDREQ_32B": 32.0, "TCC_EA0_RDREQ_64B": 64.0, "TCC_EA0_RDREQ_128B": 128.0}
    read_d = per_kernel(dir_read, lambda c: sizes.get(c))                          # bytes
    write_d = per_kernel(dir_write, lambda c: 1024.0 if c == "WRITE_SIZE" else None)  # KiB -> bytes
    fetch_d = per_kernel(dir_fetch, lambda c: 1024.0 if c == "FETCH_SIZE" else None)

    def pick(tab, pred):
        ks = [k for k in tab if pred(k)]
        assert len(ks) == 1, ks
        return ks[0]

    # the reference copy: the largest dispatches of the runtime's copy kernel
    # (the small ones are the input uploads), whatever their grid
    def merge_grids(d):
        out = {}
        for (kname, grid), v in d.items():
            key = ("copy", 0) if "copybuffer" in kname.lower() else (kname, grid)
            out.setdefault(key, []).extend(v)
        return out
    read_d, write_d, fetch_d = merge_grids(read_d), merge_grids(write_d), merge_grids(fetch_d)
    read, write, fetch = mean(read_d), mean(write_d), mean(fetch_d)
    nr = {k: len(v) for k, v in read_d.items()}
    cr = cw = cf = ("copy", 0)
    read[cr], write[cw], fetch[cf] = max(read_d[cr]), max(write_d[cw]), max(fetch_d[cf])
    r_scale, w_scale, f_scale = COPY_BYTES / read[cr], COPY_BYTES / write[cw], COPY_BYTES / fetch[cf]
    kernels = {part: (lambda k, pat=pat, wgs=wgs: k[0] != "copy" and grid_matches(k[0], k[1], pat, wgs))
               for part, (pat, wgs) in TRAFFIC_PARTS.items()}
    rows, rec = [], {}
    for part, pred in kernels.items():
        kr, kw, kf = pick(read, pred), pick(write, pred), pick(fetch, pred)
        rb, wb, fb = read[kr] * r_scale, write[kw] * w_scale, fetch[kf] * f_scale
        rows.append((part, kr, nr[kr], read[kr], write[kw], fetch[kf], rb, wb, fb))
        rec[part] = (rb, wb)
    out = {"copy_read_scale": r_scale, "copy_write_scale": w_scale, "copy_fetch_size_scale": f_scale,
           "prefill": {"bytes_per_launch": sum(rec["prefill"]), "read_bytes": rec["prefill"][0],
                       "write_bytes": rec["prefill"][1], "source_hash": source_hash("prefill")},
           "gqa_long": {"bytes_per_launch": sum(rec["gqa_long"]), "read_bytes": rec["gqa_long"][0],
                        "write_bytes": rec["gqa_long"][1], "source_hash": source_hash("prefill")},
           "decode": {"bytes_per_launch": sum(rec["decode_split"]) + sum(rec["decode_merge"]),
                      "source_hash": source_hash("decode")},
           "backward": {"bytes_per_launch": sum(rec["bwd_dq"]) + sum(rec["bwd_dkdv"]),
                        "dq_bytes": sum(rec["bwd_dq"]), "dkdv_bytes": sum(rec["bwd_dkdv"]),
                        "source_hash": source_hash("backward")}}
    print("# HBM traffic per launch (L2-to-fabric read requests by size, WRITE_SIZE)\n")
    print("Commands (repository root, one MI355X):\n")
    print("    rocprofv3 --pmc TCC_EA0_RDREQ_32B TCC_EA0_RDREQ_64B TCC_EA0_RDREQ_128B -f csv -d <dir_r> -o p "
          "-- python3 bench.py --traffic-workload")
    print("    rocprofv3 --pmc WRITE_SIZE -f csv -d <dir_w> -o p -- python3 bench.py --traffic-workload")
    print("    rocprofv3 --pmc FETCH_SIZE -f csv -d <dir_f> -o p -- python3 bench.py --traffic-workload")
    print("    python3 bench.py --traffic-summary <dir_r> <dir_w> <dir_f>\n")
    print(f"Scale reference: a {COPY_BYTES >> 20} MiB device copy (the runtime's copy kernel) reads "
          f"{read[cr] / 2**20:.1f} MiB by request size ({r_scale:.4f}x to the true {COPY_BYTES >> 20} MiB), "
          f"writes {write[cw] / 2**20:.1f} MiB by WRITE_SIZE ({w_scale:.4f}x) and shows "
          f"{fetch[cf] / 2**20:.1f} MiB by FETCH_SIZE ({f_scale:.4f}x).\n")
    print("| part | kernel | launches | read req. MiB | WRITE_SIZE MiB | FETCH_SIZE MiB | read MB (scaled) "
          "| write MB (scaled) | FETCH_SIZE MB (scaled) |")
    print("|---|---|---|---|---|---|---|---|---|")
    for part, k, n, r, w, f, rb, wb, fb in rows:
        print(f"| {part} | `{k[0][:60]}` (grid {k[1]}) | {n} | {r / 2**20:.1f} | {w / 2**20:.1f} | {f / 2**20:.1f} "
              f"| {rb / 1e6:.1f} | {wb / 1e6:.1f} | {fb / 1e6:.1f} |")
    print()
    print("Each `source_hash` is the hash of the code of the kernel's sources (comments and layout removed); "
          "`bench.py` reports a traffic figure only while it matches the current sources.\n")
    print("traffic-json: " + json.dumps(out))


def grid_of(row) -> int:
    """Grid size of a dispatch in a rocprofv3 CSV row (work-items)."""
    for key in ("Grid_Size", "Grid_Size_X"):
        if row.get(key) not in (None, ""):
            return int(float(row[key]))
    return 0


def grid_matches(kname: str, grid: int, pattern: str, wgs) -> bool:
    """Whether a dispatch is `pattern`'s kernel with `wgs` workgroups of 256
    work-items (None: any grid)."""
    return pattern in kname and (wgs is None or grid in (wgs, wgs * 256))


# Kernel and workgroup count of each workload's launch; the dense prefill
# kernel serves the MHA workload (16 query tiles x 32 heads x 4 batch rows), the
# long GQA workload (128 x 32) and the sliding-window leg (256 x 32), so the
# grid tells them apart.
DENSE = "prefill_bf16_kernel<128, false, false, false, false, false, false, false, false>"
FP8_DENSE = "prefill_bf16_kernel<128, false, false, false, false, true, false, false, false>"
TRAFFIC_PARTS = {
    "prefill": (DENSE, 2048),
    "gqa_long": (DENSE, 4096),
    "varlen": ("prefill_bf16_kernel<64, true, false, false, false, false, false, false, false>", None),
    "decode_split": ("decode_split_kernel<128, 1, false, 1, 4>", None),
    "decode_merge": ("decode_merge_kernel", None),
    "bwd_dq": ("bwd_dq_kernel<128, false, false, false, false>", None),
    "bwd_dkdv": ("bwd_dkdv_kernel<128, true, false, false, false, false>", None),
}


def _trace_work():
    """Algorithmic work per launch of each trace row that has a fixed one:
    (amount, unit, peak), from the workloads' seeded lengths alone."""
    from synth import gen
    mha = 4.0 * 4 * 32 * 2048 * 2048 * 128 / 2
    gqa = 4.0 * 1 * 32 * 16384 * 16384 * 128 / 2
    lv = gen.lognormal_lengths(16, 1024.0, 1.0, 64, 8192, gen.CONFIG_SEEDS[5]).astype(np.float64)
    varlen = float(np.sum(4.0 * 16 * lv ** 2 * 64)) / 2
    ld = gen.config_lengths_decode().astype(np.int64)
    tokens, pages = int(ld.sum()), int(np.sum((ld + 15) // 16))
    kv16 = 2.0 * 8 * 128 * 2 * tokens
    kv8 = 2.0 * 8 * 128 * tokens + 2.0 * 4 * 8 * pages
    win = 4.0 * 128 * 32 * window_pairs(32768, 4095)
    q = PAGED_CHUNK
    paged = 4.0 * 128 * 32 * float(np.sum(q * (ld - q) + q * (q + 1) // 2))
    tf, gb = "TFLOP/s", "GB/s"
    return {"mha": (mha, tf, PEAK_BF16_TFLOPS), "gqa": (gqa, tf, PEAK_BF16_TFLOPS),
            "window": (win, tf, PEAK_BF16_TFLOPS), "varlen": (varlen, tf, PEAK_BF16_TFLOPS),
            "decode": (kv16, gb, PEAK_HBM_GBPS), "decode_fp8": (kv8, gb, PEAK_HBM_GBPS),
            "lowkv1": (2.0 * 1 * 128 * 2 * tokens, gb, PEAK_HBM_GBPS),
            "lowkv2": (2.0 * 2 * 128 * 2 * tokens, gb, PEAK_HBM_GBPS),
            "decode_window": (2.0 * 8 * 128 * 2 * int(np.minimum(ld, DECODE_WINDOW).sum()), gb, PEAK_HBM_GBPS),
            "bwd": (2.5 * mha, tf, PEAK_BF16_TFLOPS),
            "paged": (paged, tf, PEAK_BF16_TFLOPS),
            "fp8_mha": (mha, tf, PEAK_FP8_TFLOPS), "fp8_gqa": (gqa, tf, PEAK_FP8_TFLOPS)}


# (label, kernel pattern, workgroups or None, key of _trace_work() or None).  A
# pattern (name, part) names a kernel and grid that several legs share (as many
# as TRACE_PARTS gives, else two): their dispatches split at the largest gaps
# in dispatch order (the legs run one after the other), part 0 the earliest.
TRACE_PARTS = {"decode_split_kernel<128, 1, false, 1, 4>": 3}
TRACE_ROWS = [
    ("MHA causal prefill B=4 A=32 S=2048 d=128 (headline)", DENSE, 2048, "mha"),
    ("GQA causal prefill B=1 A=32 A_kv=8 S=16384 d=128", DENSE, 4096, "gqa"),
    ("sliding-window GQA causal prefill S=32768, 4096-key window (kept pairs)", DENSE, 8192, "window"),
    ("varlen causal prefill, 16 seqs A=16 d=64", "prefill_bf16_kernel<64, true, false, false, false, false, false, false, false>",
     None, "varlen"),
    ("paged decode split, bf16 cache (KV bytes / split time)", ("decode_split_kernel<128, 1, false, 1, 4>", 0), None,
     "decode"),
    ("paged decode split with ALiBi (KV bytes / split time)", ("decode_split_kernel<128, 1, false, 1, 4>", 1), None,
     "decode"),
    ("paged decode split, 4096-token window (visible KV bytes / split time)",
     ("decode_split_kernel<128, 1, false, 1, 4>", 2), None, "decode_window"),
    ("paged decode LSE merge (all decode legs)", "decode_merge_kernel<128>", None, None),
    ("paged decode split, FP8 cache (KV bytes / split time)", "decode_split_kernel<128, 2, true, 1, 4>", None,
     "decode_fp8"),
    ("paged decode split, A=32 on A_kv=1 (two column groups)", "decode_split_kernel<128, 1, false, 2, 1>", None,
     "lowkv1"),
    ("paged decode split, A=32 on A_kv=2 (one-wave workgroups)", "decode_split_kernel<128, 1, false, 1, 1>", None,
     "lowkv2"),
    ("backward dQ pass", "bwd_dq_kernel<128, false, false, false, false>", None, None),
    ("backward dK/dV pass", "bwd_dkdv_kernel<128, true, false, false, false, false>", None, None),
    ("paged chunked prefill, 256-token chunks (causal pairs)",
     "prefill_bf16_kernel<128, true, true, false, false, false, false, false, false>", None, "paged"),
    ("block-sparse causal prefill", "prefill_bf16_kernel<128, false, false, true, false, false, false, false, false>", None, None),
    ("dense additive mask: documents + block mask", "prefill_bf16_kernel<128, false, false, true, true, false, false, false, false>",
     None, None),
    ("dense additive mask: per-head penalty", "prefill_bf16_kernel<128, false, false, false, true, false, false, false, false>", None,
     None),
    ("block mask of an additive term", "block_keep_kernel", None, None),
    ("key ranges: packed documents, causal prefill",
     ("prefill_bf16_kernel<128, false, false, false, false, false, false, true, false>", 0), None, None),
    ("key ranges: prefix-LM prefill (512-token prefix)",
     ("prefill_bf16_kernel<128, false, false, false, false, false, false, true, false>", 1), None, None),
    ("key ranges: backward dQ pass (documents)", "bwd_dq_kernel<128, false, false, true, false>", None, None),
    ("key ranges: backward dK/dV pass (documents)", "bwd_dkdv_kernel<128, true, false, false, true, false>", None, None),
    ("key ranges: the documents as packed sequences (varlen d=128)",
     "prefill_bf16_kernel<128, true, false, false, false, false, false, false, false>", None, None),
    ("ALiBi causal prefill", "prefill_bf16_kernel<128, false, false, false, false, false, false, false, true>",
     None, "mha"),
    ("ALiBi backward dQ pass", "bwd_dq_kernel<128, false, false, false, true>", None, None),
    ("ALiBi backward dK/dV pass", "bwd_dkdv_kernel<128, true, false, false, false, true>", None, None),
    ("FP8-QK causal prefill, MHA shape", FP8_DENSE, 2048, "fp8_mha"),
    ("FP8-QK causal prefill, long GQA shape", FP8_DENSE, 4096, "fp8_gqa"),
    ("paged chunked prefill over the E4M3 cache (causal pairs)",
     "prefill_bf16_kernel<128, true, true, false, false, false, true, false, false>", None, "paged"),
]


def trace_summary(d: str):
    """Markdown table of one kernel trace of the bench: the library's kernels,
    one row per (kernel, workload), so that no row mixes two workloads."""
    import csv
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    assert files, f"no kernel_trace.csv under {d}"
    disp = []
    for path in files:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                disp.append((r["Kernel_Name"], grid_of(r), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
                             int(r["Dispatch_Id"])))
    print("# Kernel trace of the bench, per kernel and workload\n")
    print("Commands (repository root, one MI355X):\n")
    print("    rocprofv3 --kernel-trace --stats -f csv -d <dir_t> -o bench -- python3 bench.py --steps 20 --warmup 5 "
          "--no-cpu-baseline")
    print("    python3 bench.py --trace-summary <dir_t>\n")
    print("Each row: the dispatches of one kernel at one workload's grid (warm-up and timed launches).  "
          "Rate = algorithmic work per launch / average duration.\n")
    print("| workload | kernel | grid (work-items) | calls | avg us | median us | min us | rate at avg |")
    print("|---|---|---|---|---|---|---|---|")
    works = _trace_work()
    for label, pat, wgs, wkey in TRACE_ROWS:
        part, nparts = None, 2
        if isinstance(pat, tuple):
            pat, part = pat[0], pat[1]
        if isinstance(TRACE_PARTS.get(pat), int):
            nparts = TRACE_PARTS[pat]
        sel = sorted((i, g, t) for k, g, t, i in disp if grid_matches(k, g, pat, wgs))
        if part is not None and len(sel) > 1:
            # the legs run one after the other: cut at the nparts - 1 largest
            # gaps in dispatch order
            gaps = sorted(range(len(sel) - 1), key=lambda j: sel[j + 1][0] - sel[j][0], reverse=True)
            cuts = sorted(j + 1 for j in gaps[:nparts - 1])
            bounds = [0] + cuts + [len(sel)]
            sel = sel[bounds[part]:bounds[part + 1]] if part + 1 < len(bounds) else []
        ts = sorted(t for _, _, t in sel)
        if not ts:
            continue
        grids = sorted({g for _, g, _ in sel})
        avg = sum(ts) / len(ts)
        rate = ""
        if wkey:
            amount, unit, peak = works[wkey]
            r = amount / (avg * 1e-9) / (1e12 if unit == "TFLOP/s" else 1e9)
            rate = f"{r:.1f} {unit} ({100 * r / peak:.1f}% of {peak:.0f})"
        print(f"| {label} | `{pat}` | {','.join(map(str, grids))} | {len(ts)} | {avg / 1e3:.1f} | "
              f"{ts[len(ts) // 2] / 1e3:.1f} | {ts[0] / 1e3:.1f} | {rate} |")
    print("\nThe backward's two passes together do 2.5x the forward's FLOPs of the MHA workload; the bench reports "
          "their combined rate.")
    # registers, LDS and the occupancy they allow, per library kernel
    res = {}
    for path in files:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if "attn::" not in r["Kernel_Name"]:
                    continue
                name = r["Kernel_Name"].replace("void ", "").replace("attn::(anonymous namespace)::", "").split("(")[0]
                res[name] = (int(r["VGPR_Count"]), int(r["Accum_VGPR_Count"]), int(r["SGPR_Count"]),
                             int(r["LDS_Block_Size"]), int(r["Scratch_Size"]), int(r["Workgroup_Size_X"]))
    if res:
        print("\nResources per kernel, as the trace records them: `VGPR_Count`, `Accum_VGPR_Count` and `SGPR_Count` "
              "(on gfx950 the VGPR field reads half the registers the kernel allocates: 237 allocated read as 120), "
              "LDS bytes per workgroup (static plus dynamic), scratch bytes per lane, and the waves per SIMD the LDS "
              "allows (160 KiB / LDS x waves per workgroup / 4); the register budget each kernel is built for is "
              "its `amdgpu_waves_per_eu` attribute.\n")
        print("| kernel | VGPR field | AGPR | SGPR | LDS bytes | scratch | waves / WG | waves per SIMD (LDS) |")
        print("|---|---|---|---|---|---|---|---|")
        for name in sorted(res):
            v, a, sg, lds, scr, wg = res[name]
            wpw = max(1, wg // 64)
            by_lds = (163840 // lds) * wpw / 4 if lds else 8
            print(f"| `{name}` | {v} | {a} | {sg} | {lds} | {scr} | {wpw} | {min(by_lds, 8):g} |")
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if stats:
        print("\n`--stats` output of the same run (per kernel name, all grids together; the library's kernels, then "
              "the five longest others: the measured ceilings, uploads and fills):\n")
        print("| kernel | calls | avg us | min us | max us | share |")
        print("|---|---|---|---|---|---|")
        with open(stats[0]) as fh:
            rows = list(csv.DictReader(fh))
        ours = [r for r in rows if "attn::" in r["Name"]]
        others = [r for r in rows if "attn::" not in r["Name"]][:5]
        for r in ours + others:
            name = r["Name"].replace("void ", "").replace("attn::(anonymous namespace)::", "")
            name = name.split("(")[0] if "attn::" in r["Name"] else name[:70]
            print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                  f"{float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")


N_XCD, N_SIMD = 8, 1024  # MI355X: 8 XCDs, 256 CUs x 4 SIMDs


def counter_summary(d: str):
    """Markdown summary of one SQ counter run of --traffic-workload."""
    import csv
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    assert files, f"no counter_collection.csv under {d}"
    by, span = {}, {}
    for path in files:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                key = (r["Kernel_Name"], grid_of(r), r["Dispatch_Id"])
                by.setdefault(key, {})
                by[key][r["Counter_Name"]] = by[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                span[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    kernels = {part: TRAFFIC_PARTS[part] for part in ("prefill", "gqa_long", "varlen", "decode_split", "bwd_dq",
                                                      "bwd_dkdv")}
    print("# Matrix-core utilisation per launch (SQ / GRBM counters)\n")
    print("Commands (repository root, one MI355X):\n")
    print("    rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA SQ_INSTS_VALU "
          "SQ_INSTS_VALU_TRANS_F32 SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_WAIT_ANY -f csv -d <dir_m> -o p "
          "-- python3 bench.py --traffic-workload")
    print("    python3 bench.py --counter-summary <dir_m>\n")
    print("Definitions: kernel cycles = GRBM_GUI_ACTIVE / 8 (one value per XCD); MFMA busy = "
          "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x kernel cycles); clock = kernel cycles / dispatch duration; "
          "waiting = SQ_WAIT_ANY / SQ_WAVE_CYCLES (both in quad-cycles).\n")
    print("| part | launches | duration us | kernel cycles | clock GHz | MFMA instr | MFMA busy | VALU instr / MFMA "
          "| exp / MFMA | wave time waiting |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    for part, (pat, wgs) in kernels.items():
        rows = [(v, span[k]) for k, v in by.items() if grid_matches(k[0], k[1], pat, wgs)]
        if not rows:
            continue
        n = len(rows)
        avg = lambda c: sum(v.get(c, 0.0) for v, _ in rows) / n
        dur = sum(t for _, t in rows) / n
        cyc = avg("GRBM_GUI_ACTIVE") / N_XCD
        busy = avg("SQ_VALU_MFMA_BUSY_CYCLES") / (N_SIMD * cyc) if cyc else 0.0
        mf = avg("SQ_INSTS_MFMA")
        print(f"| {part} | {n} | {dur / 1e3:.1f} | {cyc:.0f} | {cyc / dur:.2f} | {mf:.3g} | {100 * busy:.1f}% "
              f"| {(avg('SQ_INSTS_VALU') - mf) / max(mf, 1):.2f} | {avg('SQ_INSTS_VALU_TRANS_F32') / max(mf, 1):.2f} "
              f"| {100 * avg('SQ_WAIT_ANY') / max(avg('SQ_WAVE_CYCLES'), 1):.1f}% |")
    print("\n(SQ_INSTS_VALU counts the MFMA instructions too; they are subtracted above.)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--traffic-workload", action="store_true", help="run the counter workload and exit")
    ap.add_argument("--traffic-summary", nargs=3, metavar=("READ_DIR", "WRITE_DIR", "FETCH_DIR"),
                    help="summarise three counter runs of --traffic-workload and exit")
    ap.add_argument("--counter-summary", metavar="DIR", help="summarise one SQ counter run and exit")
    ap.add_argument("--trace-summary", metavar="DIR", help="summarise one kernel trace of the bench and exit")
    ap.add_argument("--decode-sweep", action="store_true",
                    help="time the paged decode at other page sizes, batch sizes and length mixes and exit")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.traffic_workload:
        traffic_workload()
        return
    if args.decode_sweep:
        decode_sweep(args.steps, args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the kernels run on a single device "
              "and no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    # ---------------- inputs (host -> HBM, outside the timed region)
    w = load_inputs(log)
    p2, p4, p5, kv_bytes, ws_bytes, stream = w["p2"], w["p4"], w["p5"], w["kv_bytes"], w["ws_bytes"], w["stream"]
    parts = w["parts"]

    for _ in range(args.warmup):
        for _, fn in parts:
            fn()
    torch.cuda.synchronize()
    log("warmup done")

    events = {name: [] for name, _ in parts}
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        for name, fn in parts:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            events[name].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {wall:.3f}s")

    ms = {name: np.array([a.elapsed_time(b) for a, b in evs]) for name, evs in events.items()}
    avg = {k: float(v.mean()) for k, v in ms.items()}
    med = {k: float(np.median(v)) for k, v in ms.items()}
    mn = {k: float(v.min()) for k, v in ms.items()}
    ceil = measured_ceilings(w["stream"])

    f2 = p2.flops()
    f3 = w["p3"].flops()
    f5 = p5.flops()
    tf2 = f2 / (avg["prefill"] * 1e-3) / 1e12
    tf3 = f3 / (avg["gqa_long"] * 1e-3) / 1e12
    tf5 = f5 / (avg["varlen"] * 1e-3) / 1e12
    gbs4 = kv_bytes / (avg["decode"] * 1e-3) / 1e9
    traffic_prefill, traffic_src = committed_traffic("prefill")
    traffic_gqa, traffic_gqa_src = committed_traffic("gqa_long", "prefill")
    traffic_decode, _ = committed_traffic("decode")
    p3 = w["p3"]

    out = {
        "metric": METRIC,
        "value": round(tf2, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs rounded to bf16; page permutation and lengths seeded)",
        "config": {
            "workload": "causal MHA prefill B=4 A=A_kv=32 S_q=S_k=2048 d=128 bf16 + paged decode 64 seqs "
                        "A=32 A_kv=8 d=128 page 16 lens~U{512..32768} + varlen causal 16 seqs A=16 d=64 + GQA "
                        "causal prefill B=1 A=32 A_kv=8 S_q=S_k=16384 d=128",
            "prefill": {"B": p2.B, "A": p2.A, "A_kv": p2.A_kv, "S_q": p2.S_q, "S_k": p2.S_k, "d": p2.d,
                        "causal": True, "flops_causal_adjusted": f2},
        },
        "roofline": {"bound": "mfma", "achieved": round(tf2, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf2 / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if traffic_prefill is None else round(traffic_prefill),
                     "traffic_unit": "bytes per launch (HBM, counter-scaled)", "traffic_source": traffic_src,
                     "algorithmic_bytes": p2.io_bytes() if hasattr(p2, "io_bytes") else None,
                     "kernel": "prefill_bf16_kernel<128, false, false, false, false, false, false, false, false>", "avg_launch_ms": round(avg["prefill"], 5),
                     "median_launch_ms": round(med["prefill"], 5), "min_launch_ms": round(mn["prefill"], 5),
                     "measured_ceiling": {"what": "torch.matmul bf16 8192^3 on the same GPU",
                                          "TFLOP/s": ceil["gemm_tflops"],
                                          "frac": round(tf2 / ceil["gemm_tflops"], 4)}},
        "decode": {"metric": "paged-decode KV GB/s", "value": round(gbs4, 1), "unit": "GB/s",
                   "roofline": {"bound": "hbm", "achieved": round(gbs4, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                "frac": round(gbs4 / PEAK_HBM_GBPS, 4),
                                "traffic": None if traffic_decode is None else round(traffic_decode),
                                "traffic_unit": "bytes per launch (split + merge, HBM, counter-scaled)"},
                   "measured_ceiling": {"what": "torch row sums over 4 GiB of fp32, rows of 4096 (read-only stream) on the same GPU",
                                        "GB/s": ceil["read_gbps"], "frac": round(gbs4 / ceil["read_gbps"], 4),
                                        "copy_GB/s": ceil["copy_gbps"]},
                   "avg_ms": round(avg["decode"], 5), "median_ms": round(med["decode"], 5),
                   "min_ms": round(mn["decode"], 5),
                   "kv_bytes": kv_bytes, "total_tokens": int(np.sum(p4.seq_lens, dtype=np.int64)),
                   "workspace_bytes": ws_bytes},
        "gqa_long": {"metric": "GQA causal prefill TFLOP/s (causal-adjusted)", "value": round(tf3, 2),
                     "unit": "TFLOP/s",
                     "roofline": {"bound": "mfma", "achieved": round(tf3, 2), "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf3 / PEAK_BF16_TFLOPS, 4),
                                  "traffic": None if traffic_gqa is None else round(traffic_gqa),
                                  "traffic_unit": "bytes per launch (HBM, counter-scaled)",
                                  "traffic_source": traffic_gqa_src, "algorithmic_bytes": p3.io_bytes(),
                                  "kernel": DENSE + " (grid 4096 workgroups)",
                                  "avg_launch_ms": round(avg["gqa_long"], 5),
                                  "median_launch_ms": round(med["gqa_long"], 5),
                                  "min_launch_ms": round(mn["gqa_long"], 5)},
                     "config": {"B": p3.B, "A": p3.A, "A_kv": p3.A_kv, "S_q": p3.S_q, "S_k": p3.S_k, "d": p3.d,
                                "causal": True, "flops_causal_adjusted": f3}},
        "varlen": {"metric": "varlen causal prefill TFLOP/s", "value": round(tf5, 2), "unit": "TFLOP/s",
                   "frac_of_bf16_peak": round(tf5 / PEAK_BF16_TFLOPS, 4), "avg_ms": round(avg["varlen"], 5),
                   "median_ms": round(med["varlen"], 5), "min_ms": round(mn["varlen"], 5),
                   "T": p5.T, "flops_causal_adjusted": f5, "masked_rows": int((p5.q_keep == 0).sum())},
    }

    out["backward"] = bench_backward(w, args.steps, args.warmup)
    out["window"] = bench_window(args.steps, args.warmup, stream)
    out["paged_prefill"] = bench_paged_prefill(w, args.steps, args.warmup)
    out["paged_prefill_fp8"] = bench_paged_prefill_fp8(w, args.steps, args.warmup)
    out["block_sparse"] = bench_block_sparse(w, args.steps, args.warmup)
    out["dense_mask"] = bench_dense_mask(w, args.steps, args.warmup)
    out["key_range"] = bench_key_range(w, args.steps, args.warmup, out["dense_mask"]["avg_ms"])
    out["alibi"] = bench_alibi(w, args.steps, args.warmup, out["dense_mask"]["per_head_penalty"]["avg_ms"],
                               out["backward"]["avg_ms"])
    out["decode_fp8"] = bench_decode_fp8(w, args.steps, args.warmup, avg["decode"])
    out["fp8_prefill"] = bench_fp8_prefill(args.steps, args.warmup, stream)
    out["decode_low_kv"] = bench_decode_low_kv(w, args.steps, args.warmup)
    out["decode_window"] = bench_decode_window(w, args.steps, args.warmup)

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(p2, args.cpu_seconds)
        out["decode"]["cpu_baseline"] = cpu_baseline_decode(p4, kv_bytes, args.cpu_seconds / 3)
        out["varlen"]["cpu_baseline"] = cpu_baseline_varlen(p5, args.cpu_seconds / 3)
        out["gqa_long"]["cpu_baseline"] = cpu_baseline_gqa(p3, args.cpu_seconds / 3)
    print(json.dumps(out), flush=True)


def backward_setup(w):
    """The backward call over the prefill workload: O and LSE are whatever the
    forward last wrote into the workload's buffers, dO is seeded N(0, 1)."""
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    p2, stream = w["p2"], w["stream"]
    q, k, v, o, lse = w["dev2"]
    ea.attn_fwd(q, k, v, o, lse, scale=p2.scale, causal=True, stream=stream)
    do = to_dev(gen.make_dout(p2, 2002), "bf16")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(p2.B, p2.A, p2.S_q), dtype=torch.uint8, device="cuda")

    def bwd():
        ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale=p2.scale, causal=True, stream=stream)
    return bwd


def bench_backward(w, steps: int, warmup: int) -> dict:
    """Backward of the causal prefill workload (dQ, dK, dV recomputed from the
    forward's LSE), timed on its own after the forward steps.

    FLOPs follow the usual convention for an attention backward: five
    S x S x d products (S, dP, dV, dQ, dK) against the forward's two, i.e. 2.5x
    the forward's causal-adjusted count.  The kernels execute seven (the dQ
    pass recomputes S and dP), reported as `executed_tflops`.  Algorithmic
    bytes: Q, K, V, O, dO and LSE read once, dQ, dK, dV written once."""
    import torch
    p2, stream = w["p2"], w["stream"]
    bwd = backward_setup(w)
    for _ in range(warmup):
        bwd()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        bwd()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    flops = 2.5 * p2.flops()
    tf = flops / (ms.mean() * 1e-3) / 1e12
    traffic, src = committed_traffic("backward")
    elem = p2.B * p2.A * p2.S_q * p2.d * 2
    alg_bytes = 8 * elem + p2.B * p2.A * p2.S_q * 4
    return {"metric": "attention bwd TFLOP/s (causal-adjusted, 2.5x forward FLOPs)", "value": round(tf, 2),
            "unit": "TFLOP/s",
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": None if traffic is None else round(traffic),
                         "traffic_unit": "bytes per call (dQ + dK/dV launches, HBM, counter-scaled)",
                         "traffic_source": src, "algorithmic_bytes": alg_bytes},
            "executed_tflops": round(tf * 7 / 5, 2), "avg_ms": round(float(ms.mean()), 5),
            "median_ms": round(float(np.median(ms)), 5), "min_ms": round(float(ms.min()), 5),
            "flops": flops,
            "workload": "causal MHA B=4 A=32 S=2048 d=128 bf16 (the prefill workload)",
            "kernels": "bwd_dq_kernel<128, false, false, false, false> then bwd_dkdv_kernel<128, true, false, false, false, false> (K rows in LDS; one call)"}


def window_pairs(S: int, left: int) -> int:
    """(row, key) pairs a causal sliding window of `left` keys before the
    diagonal keeps in one S x S head: sum_i min(i + 1, left + 1)."""
    w = left + 1
    if S <= w:
        return S * (S + 1) // 2
    return w * (w + 1) // 2 + (S - w) * w


def bench_window(steps: int, warmup: int, stream) -> dict:
    """Causal sliding-window prefill, GQA B=1 A=32 A_kv=8 S=32768 d=128, each
    query sees its own key and the 4095 before it: key tiles outside every
    row's window are skipped whole.  FLOPs = 4 d A x (kept pairs per head),
    the window analogue of the causal-adjusted count.  (S = 32768 also gives
    this leg a grid of its own in kernel traces: 8192 workgroups.)"""
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    B, A, A_kv, S, d, left = 1, 32, 8, 32768, 128, 4095
    p = gen.make_dense(B, A, A_kv, S, S, d, dtype="bf16", causal=True, seed=1006)
    q, k, v = to_dev(p.q, "bf16"), to_dev(p.k, "bf16"), to_dev(p.v, "bf16")
    o = torch.empty_like(q)
    lse = torch.empty((B, A, S), dtype=torch.float32, device="cuda")

    def run():
        ea.attn_fwd(q, k, v, o, lse, scale=p.scale, causal=True, window=(left, -1), stream=stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    flops = 4.0 * d * A * B * window_pairs(S, left)
    tf = flops / (ms.mean() * 1e-3) / 1e12
    return {"metric": "sliding-window causal prefill TFLOP/s (kept pairs)", "value": round(tf, 2),
            "unit": "TFLOP/s", "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "avg_ms": round(float(ms.mean()), 5), "median_ms": round(float(np.median(ms)), 5),
            "min_ms": round(float(ms.min()), 5), "flops": flops,
            "workload": f"GQA causal B={B} A={A} A_kv={A_kv} S={S} d={d} bf16, window: {left} keys before the "
                        "diagonal"}


def bench_decode_fp8(w, steps: int, warmup: int, bf16_ms: float) -> dict:
    """The paged decode workload (same lengths, block table and q) over FP8
    (E4M3) caches with per-(page, KV head) fp32 scales.  Algorithmic bytes:
    each valid token's K and V row of every KV head once (1 byte per element)
    plus the scales of the pages in use."""
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    p4, stream = w["p4"], w["stream"]
    t0 = time.time()
    pf = gen.make_paged_fp8(p4.seq_lens, p4.A, p4.A_kv, p4.d, p4.page_size, seed=1008)
    log(f"fp8 decode inputs ready ({time.time() - t0:.1f}s)")
    p = pf.base
    q = to_dev(p.q, "bf16")
    kc, vc = torch.from_numpy(pf.k_codes).cuda(), torch.from_numpy(pf.v_codes).cuda()
    ks, vs = torch.from_numpy(pf.k_scale).cuda(), torch.from_numpy(pf.v_scale).cuda()
    bt, sl = to_dev(p.block_table, "i32"), to_dev(p.seq_lens, "i32")
    o = torch.empty_like(q)
    lse = torch.empty((p.B, p.A), dtype=torch.float32, device="cuda")
    nbytes = ea.attn_decode_paged_workspace_bytes(p.B, p.A, p.A_kv, p.d, p.page_size, p.seq_lens)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def run():
        ea.attn_decode_paged_fp8(q, kc, vc, ks, vs, bt, sl, p.seq_lens, o, lse, ws, scale=p.scale, stream=stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    tokens = int(np.sum(p.seq_lens, dtype=np.int64))
    pages = int(np.sum((p.seq_lens.astype(np.int64) + p.page_size - 1) // p.page_size))
    kv_bytes = 2.0 * p.A_kv * p.d * tokens + 2.0 * 4 * p.A_kv * pages
    gbs = kv_bytes / (ms.mean() * 1e-3) / 1e9
    return {"metric": "paged-decode FP8 KV GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBPS, 4)},
            "avg_ms": round(float(ms.mean()), 5), "median_ms": round(float(np.median(ms)), 5),
            "min_ms": round(float(ms.min()), 5), "kv_bytes": kv_bytes, "total_tokens": tokens,
            "speedup_vs_bf16_cache": round(bf16_ms / float(ms.mean()), 3),
            "workload": "the paged decode workload (64 seqs, A=32 A_kv=8 d=128, page 16) with E4M3 caches "
                        "quantised per (page, KV head)"}


def bench_fp8_prefill(steps: int, warmup: int, stream) -> dict:
    """Causal prefill with FP8 (E4M3) queries and keys, one scale per 128 tokens
    (attn_fwd_fp8): the MHA and long GQA workloads' shapes.  Half of the FLOPs
    (QK^T) run on the FP8 matrix cores, half (PV) on the bf16 ones, so beside
    the 5.0 PF fp8 peak the line gives the mixed peak those two halves allow,
    2 / (1/5.0 + 1/2.5) = 3.33 PF."""
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    mixed = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
    out = {"metric": "FP8-QK causal prefill TFLOP/s (causal-adjusted)", "unit": "TFLOP/s",
           "peak_fp8": PEAK_FP8_TFLOPS, "peak_mixed": round(mixed, 1)}
    for name, (B, A, A_kv, S) in (("mha", (4, 32, 32, 2048)), ("gqa_long", (1, 32, 8, 16384))):
        t0 = time.time()
        p = gen.make_dense_fp8(B, A, A_kv, S, S, 128, causal=True, seed=1010 + S)
        log(f"fp8 prefill {name} inputs ready ({time.time() - t0:.1f}s)")
        q, k = torch.from_numpy(p.q_codes).cuda(), torch.from_numpy(p.k_codes).cuda()
        v = to_dev(p.v, "bf16")
        qs, ks = torch.from_numpy(p.q_scale).cuda(), torch.from_numpy(p.k_scale).cuda()
        o = torch.empty((B, A, S, 128), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, A, S), dtype=torch.float32, device="cuda")
        ms = _event_times(lambda: ea.attn_fwd_fp8(q, k, v, o, lse, qs, ks, scale=p.scale, causal=True,
                                                  stream=stream), steps, warmup, stream)
        tf = p.flops() / (ms.mean() * 1e-3) / 1e12
        out[name] = {"value": round(tf, 2), "frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4),
                     "frac_of_mixed_peak": round(tf / mixed, 4), "avg_ms": round(float(ms.mean()), 5),
                     "median_ms": round(float(np.median(ms)), 5), "min_ms": round(float(ms.min()), 5),
                     "flops": p.flops(),
                     "workload": f"causal B={B} A={A} A_kv={A_kv} S={S} d=128, E4M3 Q/K, bf16 V"}
        del q, k, v, o, lse, qs, ks
    torch.cuda.empty_cache()
    out["value"] = out["mha"]["value"]
    out["roofline"] = {"bound": "mfma", "achieved": out["mha"]["value"], "peak": PEAK_FP8_TFLOPS,
                       "unit": "TFLOP/s", "frac": out["mha"]["frac_of_fp8_peak"]}
    return out


def bench_decode_low_kv(w, steps: int, warmup: int) -> dict:
    """Paged decode with few KV heads: the decode workload's 64 lengths and
    page size with A = 32 query heads on A_kv = 1 (MQA: 32 query-head columns
    per KV head, two column groups) and on A_kv = 2 (one-wave workgroups).
    KV GB/s = 2 A_kv d 2 bytes x total tokens / time (split + merge)."""
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    p4, stream = w["p4"], w["stream"]
    out = {"metric": "paged-decode KV GB/s at few KV heads", "unit": "GB/s"}
    for A_kv in (1, 2):
        t0 = time.time()
        p = gen.make_paged(p4.seq_lens, 32, A_kv, 128, 16, dtype="bf16", seed=1030 + A_kv)
        log(f"decode A_kv={A_kv} inputs ready ({time.time() - t0:.1f}s)")
        q, kc, vc = to_dev(p.q, "bf16"), to_dev(p.k_cache, "bf16"), to_dev(p.v_cache, "bf16")
        bt, sl = to_dev(p.block_table, "i32"), to_dev(p.seq_lens, "i32")
        o = torch.empty_like(q)
        lse = torch.empty((p.B, p.A), dtype=torch.float32, device="cuda")
        nb = ea.attn_decode_paged_workspace_bytes(p.B, p.A, p.A_kv, p.d, p.page_size, p.seq_lens)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        ms = _event_times(lambda: ea.attn_decode_paged(q, kc, vc, bt, sl, p.seq_lens, o, lse, ws, scale=p.scale,
                                                       stream=stream), steps, warmup, stream)
        kvb = p.kv_bytes()
        gbs = kvb / (ms.mean() * 1e-3) / 1e9
        out[f"A_kv={A_kv}"] = {"value": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBPS, 4),
                               "avg_ms": round(float(ms.mean()), 5), "median_ms": round(float(np.median(ms)), 5),
                               "kv_bytes": kvb, "workload": f"64 seqs, A=32 A_kv={A_kv} d=128 page 16, "
                                                            "lengths ~U{512..32768}"}
        del q, kc, vc, bt, sl, o, lse, ws
    torch.cuda.empty_cache()
    return out


DECODE_WINDOW = 4096


def bench_decode_window(w, steps: int, warmup: int) -> dict:
    """The paged decode workload with a sliding window: each query sees its own
    token and the 4095 before it.  KV GB/s = 2 A_kv d 2 bytes x visible tokens
    / time (split + merge)."""
    import torch
    import exact_attention_108_amd as ea
    p4, stream = w["p4"], w["stream"]
    kc, vc, bt, sl = w["dev4"]
    q = to_dev(p4.q, "bf16")
    o = torch.empty_like(q)
    lse = torch.empty((p4.B, p4.A), dtype=torch.float32, device="cuda")
    nb = ea.attn_decode_paged_workspace_bytes(p4.B, p4.A, p4.A_kv, p4.d, p4.page_size, p4.seq_lens)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    ms = _event_times(lambda: ea.attn_decode_paged_window(q, kc, vc, bt, sl, p4.seq_lens, o, lse, ws, scale=p4.scale,
                                                          window_left=DECODE_WINDOW - 1, stream=stream),
                      steps, warmup, stream)
    visible = int(np.minimum(p4.seq_lens.astype(np.int64), DECODE_WINDOW).sum())
    kvb = 2.0 * p4.A_kv * p4.d * 2 * visible
    gbs = kvb / (ms.mean() * 1e-3) / 1e9
    return {"metric": "sliding-window paged-decode KV GB/s", "value": round(gbs, 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBPS, 4), "avg_ms": round(float(ms.mean()), 5),
            "median_ms": round(float(np.median(ms)), 5), "kv_bytes": kvb, "visible_tokens": visible,
            "workload": f"the paged decode workload (64 seqs, A=32 A_kv=8 d=128 page 16) with a {DECODE_WINDOW}-token "
                        "window (each query sees its own token and the ones before it)"}


def bench_block_sparse(w, steps: int, warmup: int) -> dict:
    """The MHA causal prefill workload with a block mask: half of the 128 x 128
    blocks kept (seeded, one mask per batch row shared by the heads).  FLOPs =
    4 d A x (causal (row, key) pairs inside kept blocks)."""
    import torch
    import exact_attention_108_amd as ea
    p2, stream = w["p2"], w["stream"]
    q, k, v, o, lse = w["dev2"]
    nb = (p2.S_q + 127) // 128
    rng = np.random.default_rng(1009)
    bk = (rng.random((p2.B, 1, nb, nb)) < 0.5).astype(np.uint8)
    bkd = torch.from_numpy(bk).cuda()

    def run():
        ea.attn_fwd(q, k, v, o, lse, scale=p2.scale, causal=True, block_keep=bkd, stream=stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    # causal pairs per block: below-diagonal blocks 128^2, diagonal blocks 128 * 129 / 2 (S = 2048 = 16 blocks)
    bi, bj = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    per_block = np.where(bj < bi, 128 * 128, np.where(bj == bi, 128 * 129 // 2, 0))
    pairs = int(sum((bk[b, 0] * per_block).sum() for b in range(p2.B)))
    flops = 4.0 * p2.d * p2.A * pairs
    tf = flops / (ms.mean() * 1e-3) / 1e12
    return {"metric": "block-sparse causal prefill TFLOP/s (kept causal pairs)", "value": round(tf, 2),
            "unit": "TFLOP/s", "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "avg_ms": round(float(ms.mean()), 5), "median_ms": round(float(np.median(ms)), 5),
            "min_ms": round(float(ms.min()), 5), "flops": flops, "blocks_kept": int(bk.sum()),
            "blocks_total": int(bk.size),
            "workload": "causal MHA B=4 A=32 S=2048 d=128 bf16 with a seeded 50% block mask (128 x 128 blocks)"}


def decode_sweep_configs():
    """(label, lengths, page size) of the decode sweep: the decode workload's
    shape (A = 32, A_kv = 8, d = 128, bf16 cache) at other page sizes, batch
    sizes and length mixes, all lengths seeded."""
    from synth import gen
    ld = gen.config_lengths_decode()
    rng = np.random.default_rng(1041)
    return [
        ("page 16, the decode workload's 64 lengths U{512..32768}", ld, 16),
        ("page 64, the same lengths", ld, 64),
        ("page 256, the same lengths", ld, 256),
        ("8 sequences, lengths U{512..32768}", rng.integers(512, 32769, 8).astype(np.int32), 16),
        ("256 sequences, lengths U{512..8192}", rng.integers(512, 8193, 256).astype(np.int32), 16),
        ("256 sequences of 1024 tokens", np.full(256, 1024, np.int32), 16),
        ("16 sequences, log-normal lengths (median 8192, sigma 1, 512..131072)",
         gen.lognormal_lengths(16, 8192.0, 1.0, 512, 131072, 1042).astype(np.int32), 16),
    ]


def decode_sweep(steps: int, warmup: int):
    """The paged decode by page size, batch size and length mix (the pages ask
    for these reported separately): KV GB/s = 2 A_kv d 2 bytes x tokens / time
    (split + merge).  Caches and queries are seeded N(0, 1) drawn on the GPU,
    pages a seeded permutation of the pool.  Prints a markdown table, then one
    JSON line."""
    import torch
    import exact_attention_108_amd as ea
    assert torch.cuda.is_available(), "the decode sweep needs a GPU"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    A, A_kv, d = 32, 8, 128
    g = torch.Generator(device="cuda").manual_seed(1043)
    rows = []
    for label, lens, ps in decode_sweep_configs():
        lens = np.asarray(lens, np.int32)
        B = len(lens)
        n_pages = (lens.astype(np.int64) + ps - 1) // ps
        P = int(n_pages.sum())
        perm = np.random.default_rng(1044).permutation(P).astype(np.int32)
        bt = np.full((B, int(n_pages.max())), -1, np.int32)
        at = 0
        for b in range(B):
            bt[b, :n_pages[b]] = perm[at:at + n_pages[b]]
            at += int(n_pages[b])
        kc = torch.randn((P, ps, A_kv, d), generator=g, device="cuda").to(torch.bfloat16)
        vc = torch.randn((P, ps, A_kv, d), generator=g, device="cuda").to(torch.bfloat16)
        q = torch.randn((B, A, d), generator=g, device="cuda").to(torch.bfloat16)
        btd, sld = torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda()
        o = torch.empty_like(q)
        lse = torch.empty((B, A), dtype=torch.float32, device="cuda")
        nb = ea.attn_decode_paged_workspace_bytes(B, A, A_kv, d, ps, lens)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        ms = _event_times(lambda: ea.attn_decode_paged(q, kc, vc, btd, sld, lens, o, lse, ws, scale=d ** -0.5,
                                                       stream=stream), steps, warmup, stream)
        tokens = int(lens.astype(np.int64).sum())
        kvb = 2.0 * A_kv * d * 2 * tokens
        gbs = kvb / (ms.mean() * 1e-3) / 1e9
        rows.append({"workload": label, "sequences": B, "tokens": tokens, "page_size": ps,
                     "value": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBPS, 4),
                     "avg_ms": round(float(ms.mean()), 5), "median_ms": round(float(np.median(ms)), 5),
                     "kv_bytes": kvb})
        log(f"decode sweep: {label}: {gbs:.0f} GB/s")
        del kc, vc, q, o, lse, ws, btd, sld
        torch.cuda.empty_cache()
    print(f"| workload (A = 32, A_kv = 8, d = 128, bf16 cache) | sequences | tokens | page | avg ms | KV GB/s | of "
          f"{PEAK_HBM_GBPS:.0f} |")
    print("|---|---|---|---|---|---|---|")
    for r in rows:
        print(f"| {r['workload']} | {r['sequences']} | {r['tokens']} | {r['page_size']} | {r['avg_ms']:.3f} | "
              f"{r['value']:.0f} | {100 * r['frac_of_hbm_peak']:.1f}% |")
    print(json.dumps({"metric": "paged-decode KV GB/s by page size, batch size and length mix", "unit": "GB/s",
                      "steps": steps, "warmup": warmup, "rows": rows}), flush=True)


def _event_times(run, steps: int, warmup: int, stream) -> np.ndarray:
    import torch
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def bench_dense_mask(w, steps: int, warmup: int) -> dict:
    """The MHA causal prefill workload with a general dense additive mask M
    (fp32 [B, heads, S, S]), two ways:
      - packed documents (log-normal lengths, median 200 tokens) given as M in
        {0, -inf} shared by the heads, with the block mask derived from it
        (attn_block_keep_from_bias, timed separately) so that tiles the
        documents exclude are skipped; FLOPs = 4 d A x (kept causal pairs);
      - a finite per-head distance penalty -2^(-8(h+1)/A) |i - j| (every pair
        kept, 2.1 GB of fp32 terms read once per launch); FLOPs = the causal
        count, and the term's bytes / time as a bandwidth."""
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    p2, stream = w["p2"], w["stream"]
    q, k, v, o, lse = w["dev2"]
    B, A, S, d = p2.B, p2.A, p2.S_q, p2.d
    doc = gen.make_bias(B, 1, S, S, "document", 1011)
    causal_pairs = np.tril(np.ones((S, S), bool))
    kept = int(sum(((doc[b, 0] == 0) & causal_pairs).sum() for b in range(B)))
    bias_doc = ea.pad_bias(torch.from_numpy(doc).cuda())
    bk = torch.empty((B, 1, (S + 127) // 128, (S + 127) // 128), dtype=torch.uint8, device="cuda")
    ms_blk = _event_times(lambda: ea.attn_block_keep_from_bias(bias_doc, bk, stream=stream), steps, warmup, stream)
    ms_doc = _event_times(lambda: ea.attn_fwd(q, k, v, o, lse, scale=p2.scale, causal=True, bias=bias_doc,
                                              block_keep=bk, stream=stream), steps, warmup, stream)
    flops_doc = 4.0 * d * A * kept
    tf_doc = flops_doc / (ms_doc.mean() * 1e-3) / 1e12
    del bias_doc
    pos = torch.arange(S, device="cuda", dtype=torch.float32)
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / A) for h in range(A)], device="cuda")
    dist = (pos[:, None] - pos[None, :]).abs()
    bias_pen = (-slopes[:, None, None] * dist[None]).unsqueeze(0).expand(B, A, S, S).contiguous()
    ms_pen = _event_times(lambda: ea.attn_fwd(q, k, v, o, lse, scale=p2.scale, causal=True, bias=bias_pen,
                                              stream=stream), steps, warmup, stream)
    flops_pen = 4.0 * d * A * B * (S * (S + 1) // 2)
    tf_pen = flops_pen / (ms_pen.mean() * 1e-3) / 1e12
    pen_bytes = 4.0 * B * A * (S * (S + 1) // 2)  # the causal part of M is what the kernel reads
    del bias_pen
    torch.cuda.empty_cache()
    return {"metric": "dense additive mask causal prefill TFLOP/s (kept pairs)", "value": round(tf_doc, 2),
            "unit": "TFLOP/s", "frac_of_bf16_peak": round(tf_doc / PEAK_BF16_TFLOPS, 4),
            "avg_ms": round(float(ms_doc.mean()), 5), "median_ms": round(float(np.median(ms_doc)), 5),
            "flops": flops_doc, "kept_pairs": kept, "blocks_kept": int(bk.sum().item()), "blocks_total": bk.numel(),
            "block_mask_from_bias_ms": round(float(ms_blk.mean()), 5),
            "workload": "causal MHA B=4 A=32 S=2048 d=128 bf16, packed documents (median 200 tokens) as an fp32 "
                        "{0, -inf} term shared by the heads, with its derived block mask",
            "per_head_penalty": {"value": round(tf_pen, 2), "unit": "TFLOP/s",
                                 "frac_of_bf16_peak": round(tf_pen / PEAK_BF16_TFLOPS, 4),
                                 "avg_ms": round(float(ms_pen.mean()), 5),
                                 "term_GB/s": round(pen_bytes / (ms_pen.mean() * 1e-3) / 1e9, 1),
                                 "workload": "the same prefill with a finite fp32 per-head distance penalty "
                                             "[4, 32, 2048, 2048] (every causal pair kept)"}}


def bench_key_range(w, steps: int, warmup: int, doc_term_ms: float) -> dict:
    """The MHA causal prefill workload with per-row key ranges:
      - packed documents as ranges (each row keeps its own document, the
        causal flag cuts it; the same documents as the dense-mask leg, seed
        1011), forward and backward; FLOPs = 4 d A x (kept causal pairs), the
        backward 2.5x that;
      - prefix-LM with a 512-token prefix (rows keep 0 .. max(i, 511), no
        causal flag); FLOPs over the kept pairs."""
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    p2, stream = w["p2"], w["stream"]
    q, k, v, o, lse = w["dev2"]
    B, A, S, d = p2.B, p2.A, p2.S_q, p2.d
    kr_np = gen.make_key_ranges(B, S, S, "document", 1011)
    i = np.arange(S)
    last = np.minimum(kr_np[..., 1], i[None])                       # causal cut
    kept = int(np.maximum(last - kr_np[..., 0] + 1, 0).sum())
    kr = torch.from_numpy(kr_np).cuda()
    ms_doc = _event_times(lambda: ea.attn_fwd(q, k, v, o, lse, scale=p2.scale, causal=True, key_range=kr,
                                              stream=stream), steps, warmup, stream)
    flops_doc = 4.0 * d * A * kept
    tf_doc = flops_doc / (ms_doc.mean() * 1e-3) / 1e12
    # backward of the documents forward
    ea.attn_fwd(q, k, v, o, lse, scale=p2.scale, causal=True, key_range=kr, stream=stream)
    do = to_dev(gen.make_dout(p2, 2002), "bf16")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(B, A, S), dtype=torch.uint8, device="cuda")
    ms_bwd = _event_times(lambda: ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale=p2.scale, causal=True,
                                              key_range=kr, stream=stream), steps, warmup, stream)
    tf_bwd = 2.5 * flops_doc / (ms_bwd.mean() * 1e-3) / 1e12
    del do, dq, dk, dv, ws
    # the same documents as packed sequences (each document of each batch row
    # its own sequence; q, k, v copied into the packed [A, T, d] layout
    # outside the timed region)
    lens = np.concatenate([np.bincount(gen.document_ids(S, 1011, b)) for b in range(B)])
    lens = lens[lens > 0]
    cu_host = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    qp, kp, vp = (x.permute(1, 0, 2, 3).reshape(A, B * S, d).contiguous() for x in (q, k, v))
    op, lp = torch.empty_like(qp), torch.empty((A, B * S), dtype=torch.float32, device="cuda")
    cu = torch.from_numpy(cu_host).cuda()
    ms_pk = _event_times(lambda: ea.attn_fwd_varlen(qp, kp, vp, op, lp, cu, cu_host, scale=p2.scale, causal=True,
                                                    stream=stream), steps, warmup, stream)
    del qp, kp, vp, op, lp
    P = 512
    pre_np = gen.make_key_ranges(B, S, S, "prefix", 0, prefix=P)
    kept_pre = int((np.maximum(i, P - 1) + 1).sum()) * B
    pre = torch.from_numpy(pre_np).cuda()
    ms_pre = _event_times(lambda: ea.attn_fwd(q, k, v, o, lse, scale=p2.scale, causal=False, key_range=pre,
                                              stream=stream), steps, warmup, stream)
    tf_pre = 4.0 * d * A * kept_pre / (ms_pre.mean() * 1e-3) / 1e12
    return {"metric": "key-range causal prefill TFLOP/s (kept pairs)", "value": round(tf_doc, 2), "unit": "TFLOP/s",
            "frac_of_bf16_peak": round(tf_doc / PEAK_BF16_TFLOPS, 4), "avg_ms": round(float(ms_doc.mean()), 5),
            "median_ms": round(float(np.median(ms_doc)), 5), "flops": flops_doc, "kept_pairs": kept,
            "speedup_over_dense_term": round(doc_term_ms / float(ms_doc.mean()), 2),
            "workload": "causal MHA B=4 A=32 S=2048 d=128 bf16, packed documents (median 200 tokens) as per-row "
                        "key ranges (the dense-mask leg's documents)",
            "backward": {"value": round(tf_bwd, 2), "unit": "TFLOP/s (2.5x the kept-pair forward FLOPs)",
                         "frac_of_bf16_peak": round(tf_bwd / PEAK_BF16_TFLOPS, 4),
                         "avg_ms": round(float(ms_bwd.mean()), 5)},
            "as_packed_sequences": {"value": round(flops_doc / (ms_pk.mean() * 1e-3) / 1e12, 2),
                                    "unit": "TFLOP/s (kept pairs)", "avg_ms": round(float(ms_pk.mean()), 5),
                                    "sequences": int(lens.size),
                                    "workload": "the same documents through attn_fwd_varlen, one sequence each"},
            "prefix_lm": {"value": round(tf_pre, 2), "unit": "TFLOP/s (kept pairs)",
                          "frac_of_bf16_peak": round(tf_pre / PEAK_BF16_TFLOPS, 4),
                          "avg_ms": round(float(ms_pre.mean()), 5), "kept_pairs": kept_pre,
                          "workload": "the same prefill, prefix-LM with a 512-token prefix (no causal flag)"}}


def bench_alibi(w, steps: int, warmup: int, term_ms: float, plain_bwd_ms: float) -> dict:
    """The MHA causal prefill workload with ALiBi computed in the kernels: the
    per-head distance penalty of the dense-mask leg (slopes 2^(-8 (h + 1) / A))
    without its 2.1 GB term, forward and backward; FLOPs = the causal count
    (every causal pair kept), the backward 2.5x that."""
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    p2, stream = w["p2"], w["stream"]
    q, k, v, o, lse = w["dev2"]
    B, A, S, d = p2.B, p2.A, p2.S_q, p2.d
    slopes = torch.tensor([2.0 ** (-8.0 * (h + 1) / A) for h in range(A)], dtype=torch.float32, device="cuda")
    ms = _event_times(lambda: ea.attn_fwd(q, k, v, o, lse, scale=p2.scale, causal=True, alibi_slopes=slopes,
                                          stream=stream), steps, warmup, stream)
    flops = p2.flops()
    tf = flops / (ms.mean() * 1e-3) / 1e12
    ea.attn_fwd(q, k, v, o, lse, scale=p2.scale, causal=True, alibi_slopes=slopes, stream=stream)
    do = to_dev(gen.make_dout(p2, 2002), "bf16")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(ea.attn_bwd_workspace_bytes(B, A, S), dtype=torch.uint8, device="cuda")
    ms_b = _event_times(lambda: ea.attn_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, scale=p2.scale, causal=True,
                                            alibi_slopes=slopes, stream=stream), steps, warmup, stream)
    tf_b = 2.5 * flops / (ms_b.mean() * 1e-3) / 1e12
    del do, dq, dk, dv, ws
    # the paged decode workload with the same slopes
    p4 = w["p4"]
    kc, vc, bt, sl = w["dev4"]
    q4 = to_dev(p4.q, "bf16")
    o4 = torch.empty_like(q4)
    lse4 = torch.empty((p4.B, p4.A), dtype=torch.float32, device="cuda")
    nb = ea.attn_decode_paged_workspace_bytes(p4.B, p4.A, p4.A_kv, p4.d, p4.page_size, p4.seq_lens)
    ws4 = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    ms_d = _event_times(lambda: ea.attn_decode_paged_alibi(q4, kc, vc, bt, sl, p4.seq_lens, o4, lse4, ws4,
                                                           scale=p4.scale, alibi_slopes=slopes, stream=stream),
                        steps, warmup, stream)
    kvb = p4.kv_bytes()
    gbs = kvb / (ms_d.mean() * 1e-3) / 1e9
    return {"metric": "ALiBi causal prefill TFLOP/s", "value": round(tf, 2), "unit": "TFLOP/s",
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "avg_ms": round(float(ms.mean()), 5),
            "median_ms": round(float(np.median(ms)), 5), "flops": flops,
            "speedup_over_dense_term": round(term_ms / float(ms.mean()), 2),
            "workload": "causal MHA B=4 A=32 S=2048 d=128 bf16 with ALiBi, slopes 2^(-8(h+1)/32) (the dense-mask "
                        "leg's per-head penalty, computed in the kernel)",
            "backward": {"value": round(tf_b, 2), "unit": "TFLOP/s (2.5x the forward FLOPs)",
                         "frac_of_bf16_peak": round(tf_b / PEAK_BF16_TFLOPS, 4),
                         "avg_ms": round(float(ms_b.mean()), 5),
                         "plain_backward_avg_ms": plain_bwd_ms},
            "decode": {"value": round(gbs, 1), "unit": "GB/s of KV", "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBPS, 4),
                       "avg_ms": round(float(ms_d.mean()), 5),
                       "workload": "the paged decode workload (64 seqs, A=32 A_kv=8 d=128 page 16) with the same "
                                   "slopes (attn_decode_paged_alibi, split + merge)"}}


PAGED_CHUNK = 256


def bench_paged_prefill(w, steps: int, warmup: int) -> dict:
    """Chunked prefill over the paged decode cache: each of the 64 sequences
    (A=32, A_kv=8, d=128, page 16, lengths ~U{512..32768}) gets its last 256
    tokens as a new query chunk, all in one call.  FLOPs = 4 d A x (causal
    (row, key) pairs): row i of a chunk of q rows over L keys sees L - q + i + 1."""
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    p4, stream = w["p4"], w["stream"]
    kc, vc, bt, sl = w["dev4"]
    n = p4.B
    q_lens = np.full(n, PAGED_CHUNK, np.int32)
    cu = np.zeros(n + 1, np.int32)
    cu[1:] = np.cumsum(q_lens)
    q = to_dev(gen.draw((p4.A, int(cu[-1]), p4.d), 1007, 0, "normal", "bf16"), "bf16")
    cud = to_dev(cu, "i32")
    o = torch.empty_like(q)
    lse = torch.empty((p4.A, int(cu[-1])), dtype=torch.float32, device="cuda")

    def run():
        ea.attn_prefill_paged(q, kc, vc, bt, sl, p4.seq_lens, cud, cu, o, lse, scale=p4.scale, causal=True,
                              stream=stream)

    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    L = p4.seq_lens.astype(np.int64)
    ql = q_lens.astype(np.int64)
    pairs = int(np.sum(ql * (L - ql) + ql * (ql + 1) // 2))
    flops = 4.0 * p4.d * p4.A * pairs
    tf = flops / (ms.mean() * 1e-3) / 1e12
    return {"metric": "paged chunked prefill TFLOP/s (causal pairs)", "value": round(tf, 2), "unit": "TFLOP/s",
            "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "avg_ms": round(float(ms.mean()), 5),
            "median_ms": round(float(np.median(ms)), 5), "min_ms": round(float(ms.min()), 5), "flops": flops,
            "workload": f"{n} sequences of the paged decode cache (A=32 A_kv=8 d=128 page 16, lengths "
                        f"~U{{512..32768}}), each with its last {PAGED_CHUNK} tokens as the query chunk"}


def bench_paged_prefill_fp8(w, steps: int, warmup: int) -> dict:
    """The chunked-prefill leg over the E4M3 form of the decode workload's cache
    (per-(page, KV head) scales; the same lengths, block table and 256-token
    chunks, seeded queries): the FP8 bytes are widened to bf16 on the way into
    LDS.  FLOPs as the bf16 leg."""
    import torch
    import exact_attention_108_amd as ea
    from synth import gen
    p4, stream = w["p4"], w["stream"]
    n = p4.B
    q_lens = np.full(n, PAGED_CHUNK, np.int32)
    t0 = time.time()
    pf, qh, cu = gen.make_paged_prefill_fp8(p4.seq_lens, q_lens, p4.A, p4.A_kv, p4.d, p4.page_size, seed=1012)
    log(f"fp8 paged prefill inputs ready ({time.time() - t0:.1f}s)")
    p = pf.base
    q = to_dev(qh, "bf16")
    kc, vc = torch.from_numpy(pf.k_codes).cuda(), torch.from_numpy(pf.v_codes).cuda()
    ks, vs = torch.from_numpy(pf.k_scale).cuda(), torch.from_numpy(pf.v_scale).cuda()
    bt, sl, cud = to_dev(p.block_table, "i32"), to_dev(p.seq_lens, "i32"), to_dev(cu, "i32")
    o = torch.empty_like(q)
    lse = torch.empty((p.A, int(cu[-1])), dtype=torch.float32, device="cuda")
    ms = _event_times(lambda: ea.attn_prefill_paged_fp8(q, kc, vc, ks, vs, bt, sl, p.seq_lens, cud, cu, o, lse,
                                                        scale=p.scale, causal=True, stream=stream),
                      steps, warmup, stream)
    L = p.seq_lens.astype(np.int64)
    ql = q_lens.astype(np.int64)
    pairs = int(np.sum(ql * (L - ql) + ql * (ql + 1) // 2))
    flops = 4.0 * p.d * p.A * pairs
    tf = flops / (ms.mean() * 1e-3) / 1e12
    del q, kc, vc, ks, vs, o, lse
    torch.cuda.empty_cache()
    return {"metric": "paged chunked prefill over an E4M3 cache TFLOP/s (causal pairs)", "value": round(tf, 2),
            "unit": "TFLOP/s", "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "avg_ms": round(float(ms.mean()), 5), "median_ms": round(float(np.median(ms)), 5), "flops": flops,
            "workload": f"{n} sequences of the paged decode workload's E4M3 cache, last {PAGED_CHUNK} tokens each"}


def measured_ceilings(stream) -> dict:
    """What this GPU sustains on plain library work, as a second reference
    beside the spec peaks: a bf16 GEMM through torch.matmul, a 2 GiB
    device-to-device copy and a read-only stream (row sums over 4 GiB)."""
    import torch
    out = {}
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(10):
        torch.matmul(a, b)
    e1.record(stream)
    torch.cuda.synchronize()
    out["gemm_tflops"] = round(2.0 * n ** 3 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
    del a, b
    src = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    out["copy_gbps"] = round(2.0 * src.numel() * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del src, dst
    # read-only stream: row sums over 4 GiB of fp32 in rows of 4096 (what decode
    # does: read, little written).  A whole-tensor x.sum() reads at only ~4 TB/s
    # on this GPU; the row form streams at ~6.3 TB/s, about what a plain
    # grid-stride kernel of 16-byte loads reaches.
    x = torch.ones(1 << 30, dtype=torch.float32, device="cuda")
    rows = x.view(-1, 4096)
    for _ in range(2):
        rows.sum(1)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(5):
        rows.sum(1)
    e1.record(stream)
    torch.cuda.synchronize()
    out["read_gbps"] = round(4.0 * x.numel() * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del x, rows
    torch.cuda.empty_cache()
    return out


def cpu_baseline_decode(p4, kv_bytes: float, target_s: float) -> dict:
    """The fp64 oracle on uniformly drawn (sequence, head) rows of the paged
    decode workload, extrapolated by the rows' share of the KV tokens."""
    import oracle
    orc = oracle.default()
    total_rows = p4.B * p4.A
    rng = np.random.default_rng(2025)
    order = rng.permutation(total_rows)
    lens = np.repeat(p4.seq_lens.astype(np.float64), p4.A)
    spent, done, work = 0.0, 0, 0.0
    while done < total_rows and spent < target_s:
        rows = order[done:done + 16]
        t0 = time.perf_counter()
        orc.decode_paged(p4.q, p4.k_cache, p4.v_cache, p4.block_table, p4.seq_lens, dtype="bf16",
                         scale=p4.scale, rows=rows)
        spent += time.perf_counter() - t0
        done += len(rows)
        work += lens[rows].sum()
    est = spent * lens.sum() / work
    log(f"oracle decode: {done} rows in {spent:.1f}s")
    return {"value": round(kv_bytes / est / 1e9, 3), "unit": "GB/s", "cores": orc.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{done} uniformly drawn (sequence, head) rows of the paged decode ({spent:.1f}s), "
                      f"extrapolated by their share of KV tokens to all {total_rows} rows ({est:.0f}s)"}


def cpu_baseline_varlen(p5, target_s: float) -> dict:
    """The fp64 oracle on uniformly drawn query rows of the varlen workload,
    extrapolated by the rows' share of visible keys (causal within a sequence)."""
    import oracle
    orc = oracle.default()
    cu = p5.cu_seqlens.astype(np.int64)
    pos = np.arange(p5.T, dtype=np.int64) - np.repeat(cu[:-1], np.diff(cu))  # position within the sequence
    cost = np.tile((pos + 1).astype(np.float64), p5.A)  # keys each (head, row) sees
    total_rows = p5.A * p5.T
    rng = np.random.default_rng(2026)
    order = rng.permutation(total_rows)
    spent, done, work = 0.0, 0, 0.0
    while done < total_rows and spent < target_s:
        rows = order[done:done + 256]
        t0 = time.perf_counter()
        orc.attn_fwd_varlen(p5.q, p5.k, p5.v, p5.cu_seqlens, dtype="bf16", scale=p5.scale, causal=True,
                            q_keep=p5.q_keep, rows=rows)
        spent += time.perf_counter() - t0
        done += len(rows)
        work += cost[rows].sum()
    est = spent * cost.sum() / work
    log(f"oracle varlen: {done} rows in {spent:.1f}s")
    return {"value": round(p5.flops() / est / 1e12, 6), "unit": "TFLOP/s", "cores": orc.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{done} uniformly drawn query rows of the varlen workload ({spent:.1f}s), extrapolated "
                      f"by their share of visible keys to all {total_rows} rows ({est:.0f}s)"}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_dense_rows(p, target_s: float, seed: int, what: str) -> dict:
    """The fp64 oracle on query rows of a causal dense workload drawn without
    replacement (one seeded permutation, taken in order), extrapolated by the
    rows' share of visible keys (row i of a causal head sees i + 1 keys)."""
    import oracle
    orc = oracle.default()
    total_rows = p.B * p.A * p.S_q
    cost = np.tile(np.arange(1, p.S_q + 1, dtype=np.float64), p.B * p.A)
    order = np.random.default_rng(seed).permutation(total_rows)
    n, spent, done, work = 256, 0.0, 0, 0.0
    while done < total_rows and spent < target_s:
        rows = np.sort(order[done:done + n])
        t0 = time.perf_counter()
        orc.attn_fwd(p.q, p.k, p.v, dtype="bf16", scale=p.scale, causal=True, rows=rows)
        dt = time.perf_counter() - t0
        spent += dt
        done += rows.size
        work += cost[rows].sum()
        log(f"oracle {what}: {done} rows in {spent:.1f}s")
        n = int(max(64, min(total_rows - done, n * max(1.0, (target_s - spent) / max(dt, 1e-3)))))
    est = spent * cost.sum() / work
    return {"value": round(p.flops() / est / 1e12, 6), "unit": "TFLOP/s", "cores": orc.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{done} query rows of the {what} drawn without replacement ({spent:.1f}s), extrapolated "
                      f"by their share of visible keys to all {total_rows} rows ({est:.0f}s)"}


def cpu_baseline(p2, target_s: float) -> dict:
    """The fp64 oracle on sampled query rows of the MHA prefill workload (same
    causal-adjusted FLOP count as `value`)."""
    return _oracle_dense_rows(p2, target_s, 2024, "causal B=4 A=32 S=2048 d=128 prefill")


def cpu_baseline_gqa(p3, target_s: float) -> dict:
    """The fp64 oracle on sampled query rows of the long GQA prefill workload."""
    return _oracle_dense_rows(p3, target_s, 2027, "GQA causal B=1 A=32 A_kv=8 S=16384 d=128 prefill")


if __name__ == "__main__":
    main()
