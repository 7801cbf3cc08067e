#!/usr/bin/env python3
"""Benchmark: encode + decode of paged KV blocks on one MI355X.

Workload (default): TurboQuant-4 K + uniform-4 V on a Llama-3-8B-shaped
cache -- 32 layers, 8 KV heads, head_dim 128, BF16, separate K/V tensors,
16-token pages, a pool of 8192 blocks of which 4096 (64K tokens) are picked
at random; layers 0, 1, 30, 31 are protected (stored raw).  Inputs are
synthetic (seeded N(0,1) K with lognormal channel scales, N(0,1) V) and
resident in HBM before timing starts.

One step = kvc_encode_pages over all 4096 pages x 32 layers (one launch)
+ kvc_decode_pages of the result into a second pool (one launch).
value = original KV bytes / step time (GB/s of original KV round-tripped).

Prints one JSON line.  --gpus N > 1 is not supported (single-GPU path).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_tq4_u4_llama3.md")
KERNEL_SOURCES = [os.path.join(ROOT, "kv_cache_page_kvc_amd", "csrc", f)
                  for f in ("kvc_kernels.hip", "kvc_arch.h", "kvc_internal.h")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or
    None when there is none or the kernels changed since it was taken."""
    import re
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    b = re.search(rf"{kernel}_hbm_bytes_per_launch:\s*([0-9]+)", text)
    if not m or not b or m.group(1) != kernel_source_hash():
        return None
    return int(b.group(1))


def calibrate_copy(gib):
    """A plain device-to-device copy of known size, for scaling the byte
    counters: each launch reads and writes `gib` GiB once."""
    import torch
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)


def algorithmic_bytes(desc):
    """Bytes one launch must move (either direction), from the encode
    descriptors: per segment the source elements, the 32-byte header and the
    stored payload (codes and metadata, or the raw bytes of a raw segment)."""
    return int(desc["original_len"].astype(np.int64).sum() + 32 * len(desc) +
               desc["stored_len"].astype(np.int64).sum())


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """Worker threads for the oracle's parallel leg: the CPUs this process
    may run on, at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, out_gpu, threads, pages_parallel, pages_single):
    """The CPU oracle, as it stands, on bounded samples of the workload's
    pages (all layers, K and V, encode then decode): once on `threads`
    threads over the first `pages_parallel` pages and once on one thread over
    the first `pages_single`.  Outside any timed region, the parallel leg's
    slots and decoded pages are compared with the GPU's (`out_gpu`: the GPU's
    encoded buffer; w["dst"]: the pages the GPU decoded it into), segment by
    segment: slot bytes identical, decoded values bit-identical (TurboQuant:
    up to the sign of a zero)."""
    import torch

    from oracle import kvc_oracle as O
    ks, vs, ids, H, T, D = w["ks"], w["vs"], w["ids"], w["H"], w["T"], w["D"]
    L, prot, seed = len(ks), w["protected"], w["seed"]
    protl = [1 if l in prot else 0 for l in range(L)]

    def u16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)

    def run(n_pages, nthreads):
        sample = ids[:n_pages]
        idx = torch.tensor(sorted(set(int(p) for p in sample)), dtype=torch.long, device=ks[0].device)
        remap = {int(b): j for j, b in enumerate(idx.tolist())}
        host = O.HostLayout(O.BF16, L, H, D, T, len(remap), T * H * D, H * D, D,
                            [u16(t.index_select(0, idx)) for t in ks], [u16(t.index_select(0, idx)) for t in vs])
        mapped = np.array([remap[int(p)] for p in sample], np.int32)
        t0 = time.perf_counter()
        buf, st, offs, total = O.encode_pages(host, O.TQ4, O.UNIFORM4, seed, mapped, protected=protl,
                                              threads=nthreads)
        t1 = time.perf_counter()
        out = O.HostLayout(O.BF16, L, H, D, T, len(remap), T * H * D, H * D, D,
                           [np.zeros_like(a) for a in host.k], [np.zeros_like(a) for a in host.v])
        O.decode_pages(buf, out, O.TQ4, O.UNIFORM4, seed, mapped, protected=protl, threads=nthreads)
        t2 = time.perf_counter()
        orig = L * len(sample) * 2 * T * H * D * 2
        return {"orig": orig, "enc_s": t1 - t0, "dec_s": t2 - t1, "buf": buf, "offs": offs, "out": out,
                "idx": idx, "remap": remap, "sample": sample}

    par = run(pages_parallel, threads)
    one = run(pages_single, 1)

    # parity of the parallel sample against the GPU's bytes and pages
    n_all = len(ids)
    offs_gpu, sizes, effs, _ = O.plan(L, H, D, T, O.TQ4, O.UNIFORM4, protl, n_all)
    gbuf = out_gpu.cpu().numpy()
    seg_all, seg_s = O.segment_list(L, n_all), O.segment_list(L, pages_parallel)
    pos = {key: s for s, key in enumerate(seg_all)}
    mism = 0
    checked = 0
    for s, (l, i, c) in enumerate(seg_s):
        g = pos[(l, i, c)]
        a = gbuf[offs_gpu[g]:offs_gpu[g] + sizes[g]]
        b = par["buf"][par["offs"][s]:par["offs"][s] + sizes[g]]
        bad = not np.array_equal(a, b)
        checked += 1
        mism += int(bad)
    dst_k, dst_v = w["dst"]
    idx = par["idx"]
    for l in range(L):
        for c, (gl, hl) in enumerate(((dst_k, par["out"].k), (dst_v, par["out"].v))):
            got = u16(gl[l].index_select(0, idx)).reshape(len(idx), T * H, D)
            want = hl[l].reshape(len(idx), T * H, D)
            tq = c == 0 and not protl[l]
            same = got == want
            if tq:
                same |= ((got & 0x7FFF) == 0) & ((want & 0x7FFF) == 0)
            mism += int((~same.reshape(len(idx), -1).all(1)).sum())
    def rate(r):
        return round(r["orig"] / (r["enc_s"] + r["dec_s"]) / 1e9, 4)
    return {"value": rate(par), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{pages_parallel} pages x {L} layers x K,V ({par['orig'] / 2**20:.0f} MiB of original KV), "
                      f"encode {par['enc_s']:.2f} s + decode {par['dec_s']:.2f} s wall on {threads} threads",
            "single_thread": {"value": rate(one), "unit": "GB/s", "cores": 1,
                              "sample": f"{pages_single} pages x {L} layers x K,V "
                                        f"({one['orig'] / 2**20:.0f} MiB), encode {one['enc_s']:.2f} s + "
                                        f"decode {one['dec_s']:.2f} s wall"},
            "cpu_model": cpu_model(), "host_logical_cpus": os.cpu_count(),
            "parity": {"segments": checked, "mismatches": mism,
                       "checked": "slot bytes of every sampled segment and its decoded page, GPU vs oracle"}}


DEFAULT_WORKLOAD = "tq4_u4_llama3"
WORKLOADS = {
    "tq4_u4_llama3": "TurboQuant-4 K + uniform-4 V, Llama-3-8B shape: 32 layers, 8 KV heads, D=128, BF16, "
                     "separate K/V, 16-token pages, 4096 random pages of an 8192-block pool (64K tokens), "
                     "layers 0,1,30,31 raw",
    "tq4_u4_llama3_tp8": "one 8-way tensor-parallel shard of the TurboQuant-4 K + uniform-4 V Llama-3-8B workload: "
                         "32 layers, 1 KV head, D=128, BF16, separate K/V, 16-token pages (4 KiB segments), "
                         "4096 random pages of an 8192-block pool, layers 0,1,30,31 raw",
    "fp8_dynamic_small": "FP8 E4M3FN dynamic per-token/head K and V: 2 layers, 8 KV heads, D=128, BF16, "
                         "separate K/V, 64 pages of 16 tokens",
    "k16v8_packed": "K raw, V FP8 ({vcodec}), Qwen3-8B shape: 36 layers, 8 KV heads, D=128, FP16, vLLM packed "
                    "[2048 blocks, 8, 16, 256] (4 sequences x 8192 tokens)",
    "tq3_u3_dsweep": "TurboQuant-3 K (2% outlier channels x20) + uniform-3 V: 28 layers, 4 KV heads, D={dim}, "
                     "BF16, separate K/V, 2048 pages (32K tokens)",
    "int8_fp8_stress": "{codec} K and V with 1% of segments holding NaN/Inf/+-450/+-1000: 32 layers, 8 KV heads, "
                       "D=128, BF16, separate K/V, 8192 pages (128K tokens), decoded into shuffled pages",
    "int8_records_qwen3": "INT8 host-pool records (BF16 scales, 1,152-byte token rows) K and V, Qwen3-8B shape: "
                          "36 layers, 8 KV heads, D=128, BF16, separate K/V, 3392 random pages of a 4096-block "
                          "pool (54,272 tokens)",
    "ans16_llama3": "lossless rANS of the byte planes (ANS16) K and V, Llama-3-8B shape: 32 layers, 8 KV heads, "
                    "D=128, BF16, separate K/V, 4096 random pages of an 8192-block pool (64K tokens)",
    "k8v8_packed": "K8/V8: FP8 E4M3FN K and V with per-token/head scales, Qwen3-8B shape: 36 layers, 8 KV heads, "
                   "D=128, FP16, vLLM packed [2048 blocks, 8, 16, 256]",
}


def build_workload(args, seed=0):
    """Synthetic engine tensors, page lists and codec of one workload (seed:
    the data and page-id seed of this copy)."""
    import torch

    import kv_cache_page_kvc_amd as kvc
    from kv_cache_page_kvc_amd import inputs
    name = args.workload
    cfg = inputs.CONFIGS[name]
    L, H, T, pool = cfg["layers"], cfg["heads"], cfg["tokens"], cfg["pool"]
    D = args.dim if name == "tq3_u3_dsweep" else cfg["dim"]
    td = inputs.torch_dtype(cfg["dtype"])
    w = {"L": L, "H": H, "D": D, "T": T, "pool": pool, "seed": seed, "protected": list(cfg.get("protected", ())),
         "describe": WORKLOADS[name].format(dim=D, vcodec=args.vcodec, codec=args.codec)}
    if cfg["layout"] == "separate":
        ks, vs = inputs.separate_kv(L, pool, T, H, D, td, seed=seed, device="cuda",
                                    k_kind=cfg.get("k_kind", "lognormal"))
        w["ks"], w["vs"] = ks, vs
        w["lay"] = kvc.Layout.separate(ks, vs, H, D, T)
        dst = ([torch.empty_like(t) for t in ks], [torch.empty_like(t) for t in vs])
        w["dst"] = dst
        w["dlay"] = kvc.Layout.separate(dst[0], dst[1], H, D, T)
    else:
        pk = inputs.packed_kv(L, pool, H, T, D, td, seed=seed, device="cuda")
        w["ks"] = pk
        w["lay"] = kvc.Layout.packed(pk, H, D, T)
        dst = [torch.empty_like(t) for t in pk]
        w["dst"] = dst
        w["dlay"] = kvc.Layout.packed(dst, H, D, T)
    n = cfg["pages"]
    ids = inputs.random_page_ids(pool, n, seed=seed) if cfg.get("random_pages") else np.arange(n, dtype=np.int32)
    w["ids"], w["dst_ids"] = ids, ids
    fixed = None
    if name == "k16v8_packed":
        k, v = "RAW", args.vcodec
        if v == "FP8_FIXED":      # per-layer scale from the first sequence's V absmax (calibration stand-in)
            amax = np.array([float(t[:512, :, :, D:].abs().max()) for t in w["ks"]])
            fixed = np.stack([np.ones(L), amax / 448.0], 1).astype(np.float32)
    elif name == "int8_fp8_stress":
        k = v = args.codec
        inputs.inject_specials(w["ks"], w["vs"], ids, frac=cfg["inject"], seed=seed)
        w["dst_ids"] = inputs.permutation(n, seed)
    else:
        k, v = cfg["k"], cfg["v"]
    # the entropy stage always carries the segment CRC32
    w["crc"] = bool(args.crc) or "ANS16" in (k, v)
    w["codec"] = kvc.Codec(k, v, seed=seed, fixed_scales=fixed, protected_layers=w["protected"], layers=L,
                           crc=w["crc"])
    return w


def lane(args):
    """Offload lane: kvc_offload_pages (encode with a CRC32 per segment, then
    the slot region, the used spill bytes and the descriptors to pinned host
    memory) and kvc_restore_pages (host to device per layer on the
    library's copy stream, each layer checked and decoded as it lands),
    timed with HIP events on the caller's stream.  Rates are GB/s of original
    KV, host link included."""
    import torch

    import kv_cache_page_kvc_amd as kvc

    torch.cuda.set_device(0)
    w = build_workload(args)
    L, H, D, T, n = w["L"], w["H"], w["D"], w["T"], len(w["ids"])
    codec, lay, dlay = w["codec"], w["lay"], w["dlay"]
    slot, spill, _ = kvc.kvc_plan(lay, codec, n)
    total = slot + spill
    host = torch.empty(total, dtype=torch.uint8, pin_memory=True)
    hdesc = torch.empty(L * n * 2 * 32, dtype=torch.uint8, pin_memory=True)
    ctx = kvc.kvc_create(0, 0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    off_ms, res_ms = [], []
    for k in range(args.warmup + args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        used = kvc.kvc_offload_pages(ctx, lay, codec, w["ids"], host.data_ptr(), total, hdesc.data_ptr(), sh)
        e[1].record(stream)
        kvc.kvc_restore_pages(ctx, dlay, codec, host.data_ptr(), used, w["dst_ids"], 0, L, 0, None, sh)
        e[2].record(stream)
        torch.cuda.synchronize()
        if k >= args.warmup:
            off_ms.append(e[0].elapsed_time(e[1]))
            res_ms.append(e[1].elapsed_time(e[2]))
        print(f"[lane] step {k}: offload {e[0].elapsed_time(e[1]):.2f} ms, restore {e[1].elapsed_time(e[2]):.2f} ms",
              file=sys.stderr, flush=True)
    kvc.kvc_destroy(ctx)
    orig = L * n * 2 * T * H * D * 2
    om, rm = float(np.mean(off_ms)), float(np.mean(res_ms))
    print(json.dumps({
        "metric": "offload lane GB/s of original KV (encode + device-to-host, host-to-device + decode)",
        "value": round(orig / ((om + rm) / 1e3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": True, "data": "synthetic",
        "config": {"workload": w["describe"], "original_bytes": orig, "host_bytes": used, "crc32": True},
        "offload_ms": round(om, 3), "restore_ms": round(rm, 3),
        "offload_GBps_original": round(orig / om / 1e6, 1), "restore_GBps_original": round(orig / rm / 1e6, 1),
        "offload_GBps_host_link": round(used / om / 1e6, 1), "restore_GBps_host_link": round(used / rm / 1e6, 1),
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-sample-pages", type=int, default=512,
                    help="pages of the oracle's multi-threaded leg (all layers, K and V)")
    ap.add_argument("--cpu-single-pages", type=int, default=256,
                    help="pages of the oracle's single-thread leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="GIB",
                    help="only run a plain GIB-GiB device copy (byte-counter calibration)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS),
                    help="the timed workload (the others are the parity-test shapes, timed on request)")
    ap.add_argument("--dim", type=int, default=256, choices=[32, 64, 256], help="head_dim for tq3_u3_dsweep")
    ap.add_argument("--vcodec", default="FP8_FIXED", choices=["FP8_FIXED", "FP8_DYNAMIC"],
                    help="V codec for k16v8_packed")
    ap.add_argument("--codec", default="INT8", choices=["INT8", "FP8_DYNAMIC", "FP8_DIRECT"],
                    help="codec for int8_fp8_stress")
    ap.add_argument("--lane", action="store_true",
                    help="time the offload lane instead: encode + copy to pinned host memory, then copy back "
                         "+ layer-by-layer decode (PCIe-inclusive; not the headline value)")
    ap.add_argument("--crc", action="store_true",
                    help="store a CRC32 per segment on encode and verify it on decode")
    ap.add_argument("--replicas", type=int, default=1, metavar="R",
                    help="R copies of the workload (seeds 0..R-1), step k on copy k mod R: inputs of a small "
                         "call then come from HBM rather than the 256 MB last-level cache")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this path runs on one GPU only (no multi-GPU sharding is built); "
              "use --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.lane:
        lane(args)
        return

    import torch

    import kv_cache_page_kvc_amd as kvc

    torch.cuda.set_device(0)
    if args.replicas < 1:
        sys.exit("bench.py: --replicas must be at least 1")
    reps = [build_workload(args, seed=r) for r in range(args.replicas)]
    w = reps[0]
    L, H, D, T, n = w["L"], w["H"], w["D"], w["T"], len(w["ids"])
    codec = w["codec"]
    slot, spill, bpt = kvc.kvc_plan(w["lay"], codec, n)
    total = slot + spill
    for r in reps:
        r["out"] = torch.empty(total, dtype=torch.uint8, device="cuda")
        r["desc"] = torch.empty(L * n * 2 * 32, dtype=torch.uint8, device="cuda")
    ctx = kvc.kvc_create(0, 0)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def step(k, ev=None):
        r = reps[k % len(reps)]
        if ev:
            ev[0].record(stream)
        kvc.kvc_encode_pages(ctx, r["lay"], r["codec"], r["ids"], r["out"].data_ptr(), total, r["desc"].data_ptr(), sh)
        if ev:
            ev[1].record(stream)
        kvc.kvc_decode_pages(ctx, r["dlay"], r["codec"], r["out"].data_ptr(), total, r["dst_ids"], 0, sh)
        if ev:
            ev[2].record(stream)

    print(f"[bench] {args.workload}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for k in range(max(args.warmup, len(reps))):
        step(k)
    torch.cuda.synchronize()
    d = w["desc"].cpu().numpy().view(kvc.DESC_DTYPE)
    n_raw_data = int((d["status"] == kvc.KVC_SEG_RAW_DATA).sum() + (d["status"] == kvc.KVC_SEG_CAPACITY).sum())

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    enc_all = [e[0].elapsed_time(e[1]) for e in evs]
    dec_all = [e[1].elapsed_time(e[2]) for e in evs]
    enc_ms, dec_ms = float(np.mean(enc_all)), float(np.mean(dec_all))
    ms_per_step = wall * 1e3 / args.steps

    orig = L * n * 2 * T * H * D * 2
    alg = algorithmic_bytes(d)
    enc_gbps, dec_gbps = alg / enc_ms / 1e6, alg / dec_ms / 1e6
    dom = "encode" if enc_ms >= dec_ms else "decode"
    dom_ms = max(enc_ms, dec_ms)
    achieved = alg / dom_ms / 1e6
    default = args.workload == DEFAULT_WORKLOAD and not args.crc and len(reps) == 1
    result = {
        "metric": "encode+decode GB/s of original KV and % of HBM peak, TurboQuant-4 D=128",
        "value": round(orig / (ms_per_step / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": w["describe"], "layers": L, "kv_heads": H, "head_dim": D, "tokens_per_page": T,
                   "pages": n, "pool_blocks": w["pool"], "original_bytes": orig, "crc32": w["crc"],
                   "replicas": len(reps), "parallelism": "none"},
        "encode_ms": round(enc_ms, 4), "decode_ms": round(dec_ms, 4),
        "encode_ms_median": round(float(np.median(enc_all)), 4),
        "decode_ms_median": round(float(np.median(dec_all)), 4),
        "timing": "HIP events recorded on the launch stream around each launch; means (and medians) over "
                  "the timed steps; rocprofv3 kernel-trace averages of the same launches are in profiles/",
        "encode_GBps_original": round(orig / enc_ms / 1e6, 1),
        "decode_GBps_original": round(orig / dec_ms / 1e6, 1),
        "encode_hbm_frac": round(enc_gbps / HBM_PEAK_GBPS, 4),
        "decode_hbm_frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_launch": alg, "bytes_per_token_encoded": bpt,
        "raw_data_segments": n_raw_data,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(dom) if default else None},
    }
    if not default:
        result["metric"] = "encode+decode GB/s of original KV and % of HBM peak"
    kvc.kvc_destroy(ctx)
    if default and not args.no_cpu_baseline:
        threads = host_threads()
        print(f"[bench] cpu baseline ({threads} threads, then 1)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, w["out"], threads, args.cpu_sample_pages,
                                              args.cpu_single_pages)
        result["parity"] = result["cpu_baseline"]["parity"]
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
