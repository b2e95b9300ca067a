#!/usr/bin/env python3
"""Throughput of lossless KV-cache coding on one MI355X.

A step is one pass of the whole coding path over the cache: encode
(symbolize, table lookup, 32-lane rANS, index + compaction) and decode (rANS
decode, reconstruction) of the Qwen3-8B-shaped e4m3 cache, 36 layers x K,V
x 32768 tokens x 1024 channels, with inputs resident in HBM.  The tables are
fitted once before timing (their fit is not part of a step).

Prints one JSON line: uncompressed GB/s of the round trip, encode and decode
rates, the ratio, per-kernel times from HIP events recorded on the launch
stream, the roofline position of the dominant kernel and the CPU oracle
timed on a bounded sample of the same workload.
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

METRIC = "KV rANS encode/decode GB/s (uncompressed) + ratio, % HBM roofline, 1 GPU"
HBM_PEAK_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "lossless_kv_cache_amd", "csrc", "skv_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_sha() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=2, help="workload id (2 = Qwen3-8B-shaped e4m3)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target length of the CPU-oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tables", choices=["channel", "exponent", "map"], default="channel",
                    help="residual tables per channel (default) or per slab and predictor exponent class; "
                         "for the DCKV workload, 'map' adds the rank-64 decoded-neighbour map")
    ap.add_argument("--transfer-layers", type=int, default=4,
                    help="layers per chunk of the transfer-pipeline measurement (0 = skip it)")
    ap.add_argument("--no-copy-probe", action="store_true",
                    help="skip timing a plain device copy of the cache (HBM ceiling; counter scale reference)")
    ap.add_argument("--no-store-probe", action="store_true",
                    help="skip the prefix-cache store measurement (put, shared-prefix decode, hit-rate trace)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the coding path has no multi-GPU part "
              "(streams are independent, so a cache shards by slab with no exchange). Run with --gpus 1.",
              flush=True)
        return 2

    import numpy as np
    import torch

    from lossless_kv_cache_amd import skv
    from workloads import gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", flush=True)
        return 1
    torch.cuda.set_device(0)
    cfg = gen.CONFIGS[args.config]
    cb = cfg.dtype == "int16"                  # DCKV coefficients (checkerboard mode)

    use_map = cb and args.tables == "map"
    if args.tables == "map" and not cb:
        print("--tables map applies to the DCKV coefficient workload (--config 4)", flush=True)
        return 2
    wl = cfg.name + ("-exponent-tables" if args.tables == "exponent" and not cb else "") + \
        ("-neighbour-map" if use_map else "")
    log(f"generating {cfg.name}: {cfg.values} values on the GPU")
    t0 = time.perf_counter()
    nmap = gen.dckv_map_weights(cfg) if use_map else None
    if cb:
        tgt, prd = gen.dckv_draw(cfg, device="cuda", nbr_map=nmap)
        ct, cp = gen.dckv_draw(cfg, gen.CALIB, tokens=gen.CALIB_TOKENS, device="cuda", nbr_map=nmap)
    else:
        tgt, prd = gen.residual_array(cfg, device="cuda")
        ct, cp = gen.residual_array(cfg, gen.CALIB, tokens=gen.CALIB_TOKENS, device="cuda")
    torch.cuda.synchronize()
    log(f"generated in {time.perf_counter() - t0:.1f} s; fitting tables")
    t0 = time.perf_counter()
    if use_map:
        V, U, sh_h, sh_m = nmap
        tabs = skv.fit_tables_map(cfg.channels, ct.cpu().numpy(), cp.cpu().numpy(), gen.CALIB_TOKENS, V, U, sh_h, sh_m)
    elif cb:
        tabs = skv.fit_tables(skv.INT16, skv.CHECKERBOARD, 1, 1, cfg.channels, ct.cpu().numpy(), cp.cpu().numpy(),
                              gen.CALIB_TOKENS)
    else:
        dt = skv.E4M3 if cfg.dtype == "e4m3" else skv.BF16
        mode = skv.RESIDUAL_EXP if args.tables == "exponent" else skv.RESIDUAL
        tabs = skv.fit_tables(dt, mode, cfg.layers, cfg.kv, cfg.channels, ct.cpu().numpy(),
                              cp.cpu().numpy(), gen.CALIB_TOKENS)
    fit_s = time.perf_counter() - t0
    del ct, cp
    log(f"fit {tabs.nbytes} B of tables in {fit_s:.2f} s")

    enc = skv.Encoder(tabs, cfg.tokens)
    out = torch.empty_like(tgt)
    raw_bytes = cfg.raw_bytes

    def step():
        a = time.perf_counter()
        cont = enc(tgt, prd)
        b = time.perf_counter()
        ke = skv.kernel_times()
        skv.decode_into(tabs, cont, prd, out)
        c = time.perf_counter()
        kd = skv.kernel_times()
        return cont.numel(), b - a, c - b, ke + kd

    skv.kernel_timing(True)
    for i in range(args.warmup):
        step()
        log(f"warmup {i + 1}/{args.warmup} done")
    torch.cuda.synchronize()
    enc_s, dec_s, ktot, kcnt = [], [], {}, {}
    cont_bytes = 0
    t_start = time.perf_counter()
    for i in range(args.steps):
        cont_bytes, e, d, ks = step()
        enc_s.append(e)
        dec_s.append(d)
        for name, ms in ks:
            ktot[name] = ktot.get(name, 0.0) + ms
            kcnt[name] = kcnt.get(name, 0) + 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {wall:.3f} s")

    # partial decode: the first half of every slab's tokens through the container's offset index
    part = None
    t1 = (cfg.tokens // 2) // 128 * 128
    if t1 > 0 and not cb:
        cont = enc(tgt, prd)
        pr = prd[:, :, :t1].contiguous()
        orr = torch.empty_like(pr)
        skv.decode_range_into(tabs, cont, 0, t1, pr, orr)
        pms = []
        for _ in range(5):
            skv.decode_range_into(tabs, cont, 0, t1, pr, orr)
            pms += [ms for name, ms in skv.kernel_times() if name == "decode_streams"]
        rb = pr.numel() * pr.element_size()
        pk = sorted(pms)[len(pms) // 2]
        part = {"tokens": [0, t1], "raw_bytes": rb, "kernel_ms": round(pk, 4),
                "GBps_uncompressed": round(rb / (pk / 1e3) / 1e9, 1),
                "verified": bool(torch.equal(orr, tgt[:, :, :t1]))}
        log(f"range decode of tokens [0, {t1}): {pk:.3f} ms, verified {part['verified']}")
        del pr, orr
    skv.kernel_timing(False)

    ok = bool(torch.equal(out, tgt))
    if not ok:
        log("RECONSTRUCTION MISMATCH")
    n_streams = cfg.layers * cfg.kv * (cfg.tokens // 128) * (cfg.channels // 32)
    head = 64 + 8 * (n_streams + 1)
    payload = cont_bytes - head
    ratio = raw_bytes / cont_bytes
    ms_per_step = wall / args.steps * 1e3
    enc_ms = 1e3 * sum(enc_s) / len(enc_s)
    dec_ms = 1e3 * sum(dec_s) / len(dec_s)
    kavg = {k: ktot[k] / kcnt[k] for k in ktot}

    # algorithmic bytes per launch (what the method itself must move)
    alg = {
        "encode_streams": 2 * raw_bytes + payload,               # target + predictor read, coded streams out
        "place_streams": 8 * (n_streams + 1) + 64,              # index + header written
        "copy_streams": payload,                                 # the stream payload written
        # predictor (or G) + container read, reconstruction out; checkerboard decodes in two launches
        "decode_streams": (raw_bytes + cont_bytes + raw_bytes) // (2 if cb else 1),
        "stream_block_sums": 0, "stream_block_scan": 0,
        # decoded-neighbour map (once per encode, once per decode): the even rows read, the odd
        # rows' side input read and their mapped side input written
        "nbr_map": 3 * (raw_bytes // 2) if use_map else 0,
    }
    dom = max(ktot, key=lambda k: ktot[k] / args.steps)
    dur_s = kavg[dom] / 1e3
    achieved = alg.get(dom, 0) / dur_s / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)                                   # {workload: {kernel: counters}}
        ent = tr.get(wl, {}).get(dom)
        if ent and ent.get("kernel_sha") == kernel_sha():
            traffic = ent["bytes_per_launch"]
    roofline = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "algorithmic_bytes": alg.get(dom, 0), "avg_ms": round(kavg[dom], 4)}
    # whole calls (every kernel of the op and its host read-backs), against HBM peak
    enc_alg = 2 * raw_bytes + cont_bytes
    dec_alg = 2 * raw_bytes + cont_bytes
    op_roofline = {
        "encode": {"ms": round(enc_ms, 4), "algorithmic_bytes": enc_alg,
                   "achieved_GBps": round(enc_alg / (enc_ms / 1e3) / 1e9, 1),
                   "frac": round(enc_alg / (enc_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "decode": {"ms": round(dec_ms, 4), "algorithmic_bytes": dec_alg,
                   "achieved_GBps": round(dec_alg / (dec_ms / 1e3) / 1e9, 1),
                   "frac": round(dec_alg / (dec_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)},
    }
    per_kernel = {k: {"avg_ms": round(kavg[k], 4), "algorithmic_bytes": alg.get(k, 0),
                      "achieved_GBps": round(alg.get(k, 0) / (kavg[k] / 1e3) / 1e9, 1),
                      "frac": round(alg.get(k, 0) / (kavg[k] / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}
                  for k in kavg if alg.get(k, 0)}

    copy = None
    if not args.no_copy_probe:
        src = tgt.view(-1).view(torch.uint8)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        cgbps = 2 * src.numel() / (ms / 1e3) / 1e9
        copy = {"bytes_copied": src.numel(), "ms": round(ms, 4), "GBps_read_plus_write": round(cgbps, 1),
                "frac_of_peak": round(cgbps / HBM_PEAK_GBPS, 4),
                "decode_kernel_frac_of_copy": round(achieved / cgbps, 4) if dom.startswith("decode") else None}
        del dst

    xfer = None
    if not cb and args.transfer_layers > 0:
        del out
        xfer = transfer_probe(skv, cfg, tabs, tgt, prd, min(args.transfer_layers, cfg.layers))

    store = None
    if not cb and not args.no_store_probe:
        store = store_probe(skv, cfg, tabs, tgt, prd)
        log(f"prefix store: put {store['put_ms']} ms, shared-prefix decode {store['lookup_and_decode_ms']} ms, "
            f"hit rate coded {store['trace']['coded']['hit_rate']} vs raw {store['trace']['raw']['hit_rate']}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = (cpu_baseline_cb if cb else cpu_baseline)(cfg, tabs, tgt, prd, args.cpu_seconds)

    res = {
        "metric": METRIC,
        "value": round(raw_bytes / (ms_per_step / 1e3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": "synthetic",
        "config": {"workload": wl, "tables": ("neighbour-map rank 64" if use_map else None) if cb else args.tables, "shape": f"[{cfg.layers}][{cfg.kv}][{cfg.tokens}][{cfg.channels}]",
                   "element": cfg.dtype, "values": cfg.values, "raw_bytes": raw_bytes, "streams": n_streams,
                   "step": "encode + decode of the whole cache", "container_bytes": cont_bytes},
        "ratio": round(ratio, 4),
        "encode_GBps": round(raw_bytes / (enc_ms / 1e3) / 1e9, 2),
        "decode_GBps": round(raw_bytes / (dec_ms / 1e3) / 1e9, 2),
        "encode_ms": round(enc_ms, 3),
        "decode_ms": round(dec_ms, 3),
        "kernels_ms": {k: round(v, 4) for k, v in kavg.items()},
        "table_fit_s": round(fit_s, 3),
        "verified_roundtrip": ok,
        "roofline": roofline,
        "op_roofline": op_roofline,
        "kernels_roofline": per_kernel,
        "copy_ceiling": copy,
        "range_decode": part,
        "transfer": xfer,
        "prefix_store": store,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0 if ok and (store is None or store["verified"]) else 1


def transfer_probe(skv, cfg, tabs, tgt, prd, layers_per_chunk, reps=3):
    """Wall time of the transfer pipeline (chunked encode -> page-locked host
    -> device -> decode, overlapped on separate streams) against moving the
    raw cache the same way (device -> page-locked host -> device, one copy
    each way); both read the cache from and write it back to HBM."""
    import torch

    tr = skv.Transfer(tabs, cfg.tokens, layers_per_chunk)
    out = torch.empty_like(tgt)
    wire, offs = tr(tgt, prd, prd, out)                       # warm: tables of every chunk, buffers
    ok = bool(torch.equal(out, tgt))
    times = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        wire, offs = tr(tgt, prd, prd, out)
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t0) * 1e3)
    ok = ok and bool(torch.equal(out, tgt))
    raw = tgt.numel() * tgt.element_size()
    host = torch.empty(raw, dtype=torch.uint8, pin_memory=True)
    src = tgt.view(-1).view(torch.uint8)
    dst = out.view(-1).view(torch.uint8)
    raw_times = []
    for _ in range(reps + 1):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        host.copy_(src, non_blocking=True)
        dst.copy_(host, non_blocking=True)
        torch.cuda.synchronize()
        raw_times.append((time.perf_counter() - t0) * 1e3)
    raw_ms = min(raw_times[1:])
    # the raw cache in the same layer chunks, with the two copy directions
    # overlapped on two streams (default priority), as the pipeline does
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    step = raw // cfg.layers * layers_per_chunk
    spans = [(a, min(raw, a + step)) for a in range(0, raw, step)]
    piped_times = []
    for _ in range(reps + 1):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs = []
        with torch.cuda.stream(s1):
            for a, b in spans:
                host[a:b].copy_(src[a:b], non_blocking=True)
                ev = torch.cuda.Event()
                ev.record(s1)
                evs.append(ev)
        with torch.cuda.stream(s2):
            for (a, b), ev in zip(spans, evs):
                s2.wait_event(ev)
                dst[a:b].copy_(host[a:b], non_blocking=True)
        torch.cuda.synchronize()
        piped_times.append((time.perf_counter() - t0) * 1e3)
    ok = ok and bool(torch.equal(out, tgt))
    piped_ms = min(piped_times[1:])
    ms = min(times)
    del host, tr
    return {"layers_per_chunk": layers_per_chunk, "chunks": len(offs) - 1, "wire_bytes": int(wire.numel()),
            "ms": round(ms, 3), "GBps": round(raw / (ms / 1e3) / 1e9, 2),
            "raw_copy_ms": round(raw_ms, 3), "raw_copy_GBps": round(raw / (raw_ms / 1e3) / 1e9, 2),
            "raw_overlapped_copy_ms": round(piped_ms, 3),
            "raw_overlapped_copy_GBps": round(raw / (piped_ms / 1e3) / 1e9, 2),
            "speedup_vs_raw_copy": round(raw_ms / ms, 3),
            "speedup_vs_raw_overlapped_copy": round(piped_ms / ms, 3), "verified": ok}


def store_probe(skv, cfg, tabs, tgt, prd, prefix_tokens=4096, prompts=64, requests=2000, zipf=1.0, seed=7,
                reps=5):
    """The prefix-cache store on the same cache: putting a prefix of
    `prefix_tokens` tokens (encode straight into the arena), looking up and
    decoding the part of it a new request shares (half its blocks), and a
    seeded request trace -- `prompts` prefixes drawn with Zipf popularity,
    a miss inserting the prefix -- replayed against two arenas of the same
    size (four raw prefixes), one holding coded prefixes and one holding raw
    ones (bookkeeping only), for the hit rate each reaches."""
    import numpy as np
    import torch

    T = min(prefix_tokens, cfg.tokens)
    t = tgt[:, :, :T].contiguous()
    p = prd[:, :, :T].contiguous()
    raw = t.numel() * t.element_size()
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, 150000, T)
    h = skv.block_hashes(ids)
    arena_bytes = -(-4 * raw // 256) * 256
    st = skv.Store(arena_bytes=arena_bytes)
    put_ms = []
    for _ in range(reps + 1):
        torch.cuda.synchronize()
        a = time.perf_counter()
        entry, nbytes = st.put(tabs, t, p, h)
        put_ms.append((time.perf_counter() - a) * 1e3)
        if len(put_ms) <= reps:
            st.erase(entry)
    put = sorted(put_ms[1:])[len(put_ms[1:]) // 2]
    # a request sharing the first half of the prefix's blocks
    q = ids.copy()
    q[T // 2 + 5] += 1
    half = T // 2
    pr = p[:, :, :half].contiguous()
    out = torch.empty_like(pr)
    dec_ms = []
    ok = True
    for _ in range(reps + 1):
        torch.cuda.synchronize()
        a = time.perf_counter()
        hit = st.lookup(skv.block_hashes(q))
        st.decode_into(tabs, hit.entry, pr, out, 0, 128 * hit.matched_blocks)
        st.release(hit.entry)
        torch.cuda.synchronize()
        dec_ms.append((time.perf_counter() - a) * 1e3)
        ok = ok and hit.matched_blocks == half // 128
    ok = ok and bool(torch.equal(out, t[:, :, :half]))
    dec = sorted(dec_ms[1:])[len(dec_ms[1:]) // 2]
    cont = st.container(st.lookup(h)).clone()
    # the trace: the same requests against coded and raw prefixes in arenas of one size
    ranks = np.arange(1, prompts + 1, dtype=np.float64)
    pop = ranks ** -zipf
    pop /= pop.sum()
    draws = rng.choice(prompts, size=requests, p=pop)
    keys = [skv.block_hashes(rng.integers(0, 150000, T)) for _ in range(prompts)]
    coded = skv.Store(arena_bytes=arena_bytes)
    base = torch.empty(arena_bytes + 256, dtype=torch.uint8)
    off = (-base.data_ptr()) % 256
    rawst = skv.Store(arena=base[off:off + arena_bytes])
    res = {}
    for name, store in (("coded", coded), ("raw", rawst)):
        hits = 0
        for k in draws:
            hit = store.lookup(keys[k])
            if hit.matched_blocks == len(keys[k]):
                hits += 1
                store.release(hit.entry)
                continue
            if hit.entry:
                store.release(hit.entry)
            if name == "coded":
                store.insert(cont, keys[k])
            else:
                e, _ = store.reserve(raw, keys[k])
                store.commit(e, raw, tokens=T)
        res[name] = {"hit_rate": round(hits / requests, 4), "entries_resident": store.stats()["entries"],
                     "evictions": store.stats()["evictions"]}
    st.close()
    coded.close()
    rawst.close()
    return {"prefix_tokens": T, "prefix_raw_bytes": raw, "container_bytes": int(nbytes),
            "put_ms": round(put, 3), "put_GBps": round(raw / (put / 1e3) / 1e9, 1),
            "shared_prefix_tokens": half, "lookup_and_decode_ms": round(dec, 3),
            "lookup_and_decode_GBps": round(t.numel() * t.element_size() / 2 / (dec / 1e3) / 1e9, 1),
            "verified": ok,
            "trace": {"arena_bytes": arena_bytes, "prompts": prompts, "requests": requests, "zipf": zipf,
                      "coded": res["coded"], "raw": res["raw"]}}


def host_cpus() -> dict:
    """The host's CPU inventory: logical CPUs, the ones this process may run
    on, and lscpu's sockets, cores per socket and threads per core."""
    import subprocess

    info = {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0))}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        keys = {"Socket(s)": "sockets", "Core(s) per socket": "cores_per_socket",
                "Thread(s) per core": "threads_per_core", "Model name": "model"}
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in keys:
                v = v.strip()
                info[keys[k.strip()]] = int(v) if v.isdigit() else v
    except (OSError, subprocess.SubprocessError):
        pass
    return info


def oracle_threads() -> int:
    """OpenMP threads for the oracle: every CPU this process may use, up to
    the 16-CPU share of one GPU on the test machines (OMP_NUM_THREADS there)."""
    cap = int(os.environ.get("OMP_NUM_THREADS", "16") or 16)
    return max(1, min(cap, 16, len(os.sched_getaffinity(0))))


def cpu_baseline(cfg, tabs, tgt, prd, seconds):
    """The oracle (plain C, OpenMP over streams) on the host: encode + decode
    of whole layers of the same workload until about `seconds` of work, on
    every thread it may use, then the first layer again on one thread."""
    import numpy as np
    import oracle

    threads = oracle_threads()
    blob = tabs.bytes()
    exp = tabs.mode == oracle.RESIDUAL_EXP
    per_layer_tables = cfg.kv * (16 if exp else cfg.channels)
    rec = 514
    n_tables = cfg.layers * per_layer_tables
    done_bytes, spent, layers = 0, 0.0, 0
    one = None
    for layer in range(cfg.layers):
        hdr = bytearray(blob[:64])
        hdr[8:12] = per_layer_tables.to_bytes(4, "little")
        hdr[12:16] = (1).to_bytes(4, "little")
        total = 64 + per_layer_tables * rec + (cfg.kv if exp else 0)
        hdr[32:40] = total.to_bytes(8, "little")
        sub = bytes(hdr) + blob[64 + layer * per_layer_tables * rec:64 + (layer + 1) * per_layer_tables * rec]
        if exp:                                                   # the layer's class bases
            b0 = 64 + n_tables * rec + layer * cfg.kv
            sub += blob[b0:b0 + cfg.kv]
        t = tgt[layer:layer + 1].cpu().numpy()
        p = prd[layer:layer + 1].cpu().numpy()
        dt = oracle.E4M3 if cfg.dtype == "e4m3" else oracle.BF16
        shape = oracle.make_shape(dt, oracle.RESIDUAL_EXP if exp else oracle.RESIDUAL, 1, cfg.kv, cfg.tokens,
                                  cfg.channels)
        a = time.perf_counter()
        c = oracle.encode(sub, shape, t, p, threads=threads)
        back = oracle.decode(sub, c, p, t, threads=threads)
        spent += time.perf_counter() - a
        if not np.array_equal(back, t):
            raise RuntimeError("oracle round trip failed")
        if one is None:                                           # the same layer on one thread
            a = time.perf_counter()
            c1 = oracle.encode(sub, shape, t, p, threads=1)
            oracle.decode(sub, c1, p, t, threads=1)
            s1 = time.perf_counter() - a
            one = {"value": round(t.nbytes / s1 / 1e9, 4), "unit": "GB/s", "threads": 1,
                   "sample": f"encode + decode of layer 0 ({t.nbytes} B)", "seconds": round(s1, 2)}
            log(f"cpu oracle: layer 0 on one thread in {s1:.1f} s")
        done_bytes += t.nbytes
        layers += 1
        log(f"cpu oracle: layer {layer} done, {spent:.1f} s so far")
        if spent >= seconds:
            break
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"encode + decode of {layers} of {cfg.layers} layers (K and V, {done_bytes} B of "
                      f"{cfg.dtype} codes) of the same workload and tables, {threads} OpenMP threads",
            "seconds": round(spent, 2), "one_thread": one, "host": host_cpus()}


def cpu_baseline_cb(cfg, tabs, coef, G, seconds):
    """The oracle on the host for the checkerboard workload: encode + decode of
    leading token spans of the same matrix (same tables) until about `seconds`."""
    import numpy as np
    import oracle

    threads = oracle_threads()
    blob = tabs.bytes()
    span = min(cfg.tokens, 8192)
    done_bytes, spent, spans = 0, 0.0, 0
    one = None
    for a in range(0, cfg.tokens, span):
        c = coef[a:a + span].cpu().numpy()
        g = G[a:a + span].cpu().numpy()
        shape = oracle.make_shape(oracle.INT16, tabs.mode, 1, 1, span, cfg.channels)
        t0 = time.perf_counter()
        cont = oracle.encode(blob, shape, c, g, threads=threads)
        back = oracle.decode(blob, cont, g, c, threads=threads)
        spent += time.perf_counter() - t0
        if not np.array_equal(back, c):
            raise RuntimeError("oracle round trip failed")
        if one is None:                                           # the same span on one thread
            t0 = time.perf_counter()
            cont1 = oracle.encode(blob, shape, c, g, threads=1)
            oracle.decode(blob, cont1, g, c, threads=1)
            s1 = time.perf_counter() - t0
            one = {"value": round(c.nbytes / s1 / 1e9, 4), "unit": "GB/s", "threads": 1,
                   "sample": f"encode + decode of the first span ({c.nbytes} B)", "seconds": round(s1, 2)}
        done_bytes += c.nbytes
        spans += 1
        log(f"cpu oracle: span {spans} done, {spent:.1f} s so far")
        if spent >= seconds:
            break
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"encode + decode of {spans} spans of {span} tokens x {cfg.channels} int16 coefficients "
                      f"({done_bytes} B) of the same matrix and tables, {threads} OpenMP threads",
            "seconds": round(spent, 2), "one_thread": one, "host": host_cpus()}


if __name__ == "__main__":
    sys.exit(main())
