"""Helpers for the rocprofv3 measurements of the Kara kernels.

    python -m decode_kv_cache_amd.profiling copy --mib 2048
        a plain device copy of a known size (an elementwise torch kernel that
        reads and writes every byte once), run under ``rocprofv3 --pmc`` to
        calibrate FETCH_SIZE / WRITE_SIZE against bytes actually moved;
    python -m decode_kv_cache_amd.profiling peaks
        achievable peaks on this GPU from libkara_probes.so (MFMA bf16 loop,
        v_exp_f32 and fp32 FMA rates, HBM read and copy bandwidth), as JSON;
    python -m decode_kv_cache_amd.profiling counters <rocprofv3 --pmc output dirs>
        per-kernel means of every collected counter, with MFMA busy and VALU
        issue shares per SIMD;
    python -m decode_kv_cache_amd.profiling stats <rocprofv3 output dir>
        markdown table of per-kernel dispatch counts and durations;
    python -m decode_kv_cache_amd.profiling traffic --workload W --fetch D1 --write D2 \\
            --copy-fetch D3 --copy-write D4 --copy-mib M
        per-launch HBM bytes of every kernel from FETCH_SIZE / WRITE_SIZE runs,
        each scaled by what the same counter reads for the copy; updates
        profiles/traffic.json (keyed by workload and the kernel-source hash)
        and prints a markdown summary.

FETCH_SIZE and WRITE_SIZE are rocprofv3's derived L2-to-memory counters, in
KiB per dispatch.
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def code_only(src: str) -> str:
    """C++ source without its comments, whitespace runs collapsed to one
    space; string and character literals are kept as they are."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            while i < n and src[i] != "\n":
                i += 1
        elif src.startswith("/*", i):
            k = src.find("*/", i + 2)
            i = n if k < 0 else k + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(read=None) -> str:
    """Hash of the code (comments and layout aside) of every source that goes
    into the library's kernels: all of csrc but the host-only ABI layer
    (api.hip, no device code) and the probes (tools, not part of the
    library).  A stored measurement is valid for this hash only.  `read`
    (name -> text) replaces the working tree, e.g. to hash another revision."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "decode_kv_cache_amd", "csrc")
    if read is None:
        names = os.listdir(csrc)

        def read(f):
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                return fh.read()
    else:
        names = read(None)
    for f in sorted(names):
        if f in ("probes.hip", "api.hip"):
            continue
        h.update(f.encode() + b"\0" + code_only(read(f)).encode())
    return h.hexdigest()[:16]


_TYPES = {"DF16b": "__bf16", "f": "float", "d": "double", "i": "int"}


def _demangle_kara(name: str) -> str:
    """Readable form of the simple mangled names of this library's kernels
    (namespace kara, optional template arguments of types and integers)."""
    import re
    m = re.match(r"_ZN4kara(?:12_GLOBAL__N_1)?(\d+)", name)
    if not m:
        return name
    n = int(m.group(1))
    ident = name[m.end():m.end() + n]
    rest = name[m.end() + n:]
    if rest.startswith("I"):
        args, i = [], 1
        while i < len(rest) and rest[i] != "E":
            if rest.startswith("Li", i):
                j = rest.index("E", i)
                args.append(rest[i + 2:j])
                i = j + 1
                continue
            for code, tname in _TYPES.items():
                if rest.startswith(code, i):
                    args.append(tname)
                    i += len(code)
                    break
            else:
                break
        ident += "<" + ", ".join(args) + ">"
    return ident


def short_name(name: str) -> str:
    if name.startswith("_Z"):
        return _demangle_kara(name)
    s = name.replace("void ", "").split("(")[0]
    for pre in ("kara::(anonymous namespace)::", "kara::"):
        s = s.replace(pre, "")
    return s.strip() or "(unnamed probe kernel)"


def _files(d, pattern):
    return sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))


def counter_means(d: str, counter: str) -> dict:
    """Mean over dispatches of `counter` per kernel (summing the rows of one dispatch)."""
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for f in _files(d, "*counter_collection.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") != counter:
                    continue
                per[short_name(r.get("Kernel_Name", ""))][r.get("Dispatch_Id")] += float(r["Counter_Value"])
    return {k: sum(v.values()) / len(v) for k, v in per.items() if v}


def kernel_stats(d: str) -> list:
    rows = []
    for f in _files(d, "*kernel_stats.csv"):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                             float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
    return rows


def achievable_peaks(device=0) -> dict:
    """Time the probes of libkara_probes.so with HIP events on one stream."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "decode_kv_cache_amd", "libkara_probes.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m decode_kv_cache_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    for name, args in (("kara_probe_mfma", [vp, i32, i32, vp]), ("kara_probe_exp", [vp, i32, i32, vp]),
                       ("kara_probe_fma", [vp, i32, i32, vp]), ("kara_probe_read", [vp, sz, vp, i32, vp]),
                       ("kara_probe_copy", [vp, vp, sz, i32, vp]), ("kara_probe_rewrite", [vp, sz, vp])):
        getattr(lib, name).argtypes = args
        getattr(lib, name).restype = i32
    dev = torch.device("cuda", device)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    st = torch.cuda.Stream(device=dev)
    sptr = ctypes.c_void_p(st.cuda_stream)

    def timed(launch, reps=3):
        launch()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(st)
        for _ in range(reps):
            if launch() != 0:
                raise RuntimeError("probe launch failed")
        ev[1].record(st)
        torch.cuda.synchronize(dev)
        return ev[0].elapsed_time(ev[1]) / reps / 1e3

    blocks, iters = cus * 8, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    o = ctypes.c_void_p(out.data_ptr())
    t = timed(lambda: lib.kara_probe_mfma(o, blocks, iters, sptr))
    mfma = blocks * 4 * iters * 4 * 32768.0 / t / 1e12
    t = timed(lambda: lib.kara_probe_exp(o, blocks, iters, sptr))
    exps = blocks * 256 * iters * 8.0 / t
    t = timed(lambda: lib.kara_probe_fma(o, blocks, iters, sptr))
    fmas = blocks * 256 * iters * 8.0 / t
    nbytes = 4 << 30
    grid = cus * 8
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(grid * 256, dtype=torch.float32, device=dev)
    sp, dp, kp = (ctypes.c_void_p(x.data_ptr()) for x in (src, dst, sink))
    torch.cuda.synchronize(dev)                    # filled on the default stream, read on the probe stream
    t = timed(lambda: lib.kara_probe_read(sp, nbytes, kp, grid, sptr))
    read = nbytes / t / 1e9
    t = timed(lambda: lib.kara_probe_copy(sp, dp, nbytes, grid, sptr))
    copy = 2 * nbytes / t / 1e9
    t = timed(lambda: lib.kara_probe_rewrite(dp, nbytes, sptr))
    rewrite = 2 * nbytes / t / 1e9
    del src, dst
    return {"mfma_bf16_tflops": round(mfma, 1), "v_exp_f32_per_s": float(f"{exps:.4g}"),
            "fma_f32_per_s": float(f"{fmas:.4g}"), "hbm_read_GBps": round(read, 1),
            "hbm_copy_GBps_read_plus_write": round(copy, 1),
            "hbm_rewrite_in_place_GBps_read_plus_write": round(rewrite, 1),
            "how": "libkara_probes.so: MFMA 32x32x16 bf16 loop, v_exp_f32 / v_fma_f32 chains (8 per lane per "
                   "iteration), 4 GiB non-temporal read (64 KiB chunks per workgroup, grid-stride), copy "
                   "(grid-stride) and in-place rewrite (one workgroup per 16 KiB); HIP events over "
                   "3 launches after one warm-up"}


def cmd_peaks(a):
    print(json.dumps(achievable_peaks()), flush=True)


def cmd_counters(a):
    """Mean per dispatch of every counter found in the given rocprofv3 --pmc
    output directories, for this library's kernels, with the derived
    utilisations (SQ counters are totals over the chip's 1024 SIMDs; GRBM
    counters over its 8 XCDs)."""
    per = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
    for d in a.dirs:
        for f in _files(d, "*counter_collection.csv"):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    k = short_name(r.get("Kernel_Name", ""))
                    per[k][r["Counter_Name"]][(d, r.get("Dispatch_Id"))] += float(r["Counter_Value"])
    for k in sorted(per):
        if not any(t in k for t in ("score", "select", "compact", "finalize", "decode_attn", "pipeline", "row_lse",
                                    "col_mass")):
            continue
        c = {name: sum(v.values()) / len(v) for name, v in per[k].items()}
        print(f"### {k}")
        print()
        print("| Counter | Mean per dispatch |")
        print("|---|---|")
        for name in sorted(c):
            print(f"| {name} | {c[name]:.4g} |")
        simds, xcds = 1024.0, 8.0
        if "GRBM_GUI_ACTIVE" in c:
            cyc = c["GRBM_GUI_ACTIVE"] / xcds
            print(f"| kernel cycles (GRBM_GUI_ACTIVE / 8 XCDs) | {cyc:.4g} |")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
                print(f"| MFMA busy per SIMD (SQ_VALU_MFMA_BUSY_CYCLES / 1024 / cycles) | "
                      f"{c['SQ_VALU_MFMA_BUSY_CYCLES'] / simds / cyc:.3f} |")
            if "SQ_INSTS_VALU" in c and "SQ_INSTS_VALU_TRANS_F32" in c:
                # a wave64 VALU instruction holds a 16-lane SIMD for 4 cycles, a
                # transcendental one (quarter rate) for 16
                tr = c["SQ_INSTS_VALU_TRANS_F32"]
                busy = ((c["SQ_INSTS_VALU"] - tr) * 4 + tr * 16) / simds / cyc
                print(f"| VALU busy per SIMD ((SQ_INSTS_VALU - TRANS) x 4 + TRANS x 16 cycles / 1024 / cycles) | "
                      f"{busy:.3f} |")
        print()


def cmd_copy(a):
    import torch
    n = a.mib * 1024 * 1024 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(a.reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(f"copied {a.mib} MiB x {a.reps} with torch.neg (reads and writes every byte once)", flush=True)


def cmd_stats(a):
    print("| Kernel | Calls | Avg (us) | Min (us) | Max (us) | % of GPU time |")
    print("|---|---|---|---|---|---|")
    for name, calls, avg, mn, mx, pct in kernel_stats(a.dir):
        print(f"| {name} | {calls} | {avg:.1f} | {mn:.1f} | {mx:.1f} | {pct:.2f} |")


def cmd_traffic(a):
    fetch = counter_means(a.fetch, "FETCH_SIZE")
    write = counter_means(a.write, "WRITE_SIZE")
    cf = counter_means(a.copy_fetch, "FETCH_SIZE")
    cw = counter_means(a.copy_write, "WRITE_SIZE")
    kib = a.copy_mib * 1024.0
    ck = [k for k in cf if "neg" in k.lower()] or list(cf)
    f_fac = max(cf[k] for k in ck) / kib
    w_fac = max(cw[k] for k in ck if k in cw) / kib
    print(f"copy calibration ({a.copy_mib} MiB read + written): FETCH_SIZE reads {f_fac:.4f} x, "
          f"WRITE_SIZE {w_fac:.4f} x the bytes moved")
    print()
    print("| Kernel | FETCH_SIZE (KiB/dispatch) | WRITE_SIZE (KiB/dispatch) | HBM bytes per launch (scaled) |")
    print("|---|---|---|---|")
    rec = {}
    for k in sorted(set(fetch) | set(write)):
        if "kara" not in k and not any(t in k for t in ("score", "select", "compact", "finalize", "decode_attn",
                                                         "row_lse", "col_mass")):
            continue
        fb = fetch.get(k, 0.0) * 1024 / f_fac
        wb = write.get(k, 0.0) * 1024 / w_fac
        rec[k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes": fb + wb}
        print(f"| {k} | {fetch.get(k, 0.0):.0f} | {write.get(k, 0.0):.0f} | {fb + wb:.4g} |")
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    score = [v["bytes"] for k, v in rec.items() if "score" in k or "row_lse" in k or "col_mass" in k]
    data[a.workload] = {"kernel_hash": kernel_source_hash(), "copy_factor_fetch": f_fac,
                        "copy_factor_write": w_fac, "kernels": rec,
                        "score_bytes_per_launch": sum(score) if score else None}
    with open(path, "w") as f:
        json.dump(data, f, indent=1)


def cmd_coissue(a):
    """Time kara_probe_coissue's four modes at 1, 2 and 4 waves per SIMD and
    print ns per wave-iteration per SIMD, with the overlap of the MFMA and
    VALU parts: (t_mfma + t_valu - t_both) / min(t_mfma, t_valu)."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "decode_kv_cache_amd", "libkara_probes.so")
    lib = ctypes.CDLL(path)
    lib.kara_probe_coissue.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]
    lib.kara_probe_coissue.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    simds = 4 * cus
    st = torch.cuda.Stream()
    sp = ctypes.c_void_p(st.cuda_stream)
    out = torch.empty(4 * cus * 512, dtype=torch.float32, device="cuda")
    o = ctypes.c_void_p(out.data_ptr())
    iters = a.iters

    def ns(mode, blocks, threads):
        f = lambda: lib.kara_probe_coissue(mode, o, blocks, threads, iters, sp)
        if f() != 0:
            raise RuntimeError("probe launch failed")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(st)
        f()
        ev[1].record(st)
        torch.cuda.synchronize()
        waves_per_simd = blocks * threads / 64 / simds
        return ev[0].elapsed_time(ev[1]) * 1e6 / iters / waves_per_simd

    print("| Waves per SIMD | 4 MFMA | 16 FMA | 4 MFMA + 16 FMA | overlap | 16 (mul + v_exp_f32) "
          "| 4 MFMA + 16 (mul + v_exp_f32) | overlap | 16 bare v_exp_f32 | 16 v_exp_f32 + 16 FMA | overlap |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for label, blocks, threads in (("1", cus, 256), ("2", cus, 512), ("4", 4 * cus, 256)):
        tm, tf, tb, tmx, tx, te, tef = (ns(m, blocks, threads) for m in (0, 1, 2, 3, 4, 5, 6))
        ov = (tm + tf - tb) / min(tm, tf)
        ox = (tm + tx - tmx) / min(tm, tx)
        oe = (te + tf - tef) / min(te, tf)
        print(f"| {label} | {tm:.1f} ns | {tf:.1f} ns | {tb:.1f} ns | {100 * ov:.0f} % | {tx:.1f} ns | {tmx:.1f} ns "
              f"| {100 * ox:.0f} % | {te:.1f} ns | {tef:.1f} ns | {100 * oe:.0f} % |", flush=True)


def cmd_coissue_cu(a):
    """Time kara_probe_coissue_cu's modes at exactly one and two waves per
    SIMD (one workgroup per compute unit) and print ns per wave-iteration."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "decode_kv_cache_amd", "libkara_probes.so")
    lib = ctypes.CDLL(path)
    lib.kara_probe_coissue_cu.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p]
    lib.kara_probe_coissue_cu.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.Stream()
    sp = ctypes.c_void_p(st.cuda_stream)
    out = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    o = ctypes.c_void_p(out.data_ptr())
    names = ["16 MFMA", "64 FMA", "16 MFMA + 16 FMA (M v)", "16 MFMA + 32 FMA (M vv)", "16 MFMA + 64 FMA (M vvvv)",
             "32 v_exp_f32", "16 MFMA + 32 v_exp_f32 (M ee)"]
    print("| Per iteration | 1 wave per SIMD | 2 waves per SIMD |")
    print("|---|---|---|")
    for mode, name in enumerate(names):
        row = []
        for threads in (256, 512):
            if lib.kara_probe_coissue_cu(mode, o, cus, threads, 10, sp) != 0:
                raise RuntimeError("probe launch failed")
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(st)
            lib.kara_probe_coissue_cu(mode, o, cus, threads, a.iters, sp)
            ev[1].record(st)
            torch.cuda.synchronize()
            row.append(ev[0].elapsed_time(ev[1]) * 1e6 / a.iters / (threads // 256))
        print(f"| {name} | {row[0]:.1f} ns | {row[1]:.1f} ns |", flush=True)
    # the MFMAs and the vector work in the two different waves of each SIMD
    print()
    print("| Waves 0-3 / waves 4-7 of each workgroup (2 per SIMD) | Time per iteration | Waves placed one of each kind per SIMD |")
    print("|---|---|---|")
    for mode, name in ((7, "16 MFMA / 64 FMA"), (8, "16 MFMA / 32 v_exp_f32")):
        if lib.kara_probe_coissue_cu(mode, o, cus, 512, 10, sp) != 0:
            raise RuntimeError("probe launch failed")
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(st)
        lib.kara_probe_coissue_cu(mode, o, cus, 512, a.iters, sp)
        ev[1].record(st)
        torch.cuda.synchronize()
        tags = out.view(cus, 8, 64)[:, :, 0].cpu().numpy().astype(int) - 1000
        ok = all(sorted(t.tolist()) == [0, 1, 10, 11, 20, 21, 30, 31] for t in tags)
        print(f"| {name} | {ev[0].elapsed_time(ev[1]) * 1e6 / a.iters:.1f} ns | {'yes' if ok else 'no'} |",
              flush=True)


def cmd_compact_patterns(a):
    """Time kara_compact_paged on one workload with several kept patterns: the
    selection the step makes, and synthetic ones with the same budget (dense
    in place, dense shifted, strided, uniformly random).  Only the block
    tables are restored between launches; pool contents do not change the
    work.  Rate = 2 pools x B rows x row bytes x (read + write) x units."""
    import numpy as np
    import torch

    from decode_kv_cache_amd import kara as K
    from decode_kv_cache_amd.workloads import make_workload, shape_by_name
    shape = shape_by_name(a.workload)
    wl = make_workload(shape, "cuda")
    cfg = K.make_config(shape, max_blocks_per_seq=wl.max_blocks, num_blocks=wl.num_blocks)
    S, Lyr, Hkv, W, B = shape.num_seqs, shape.num_layers, shape.num_kv_heads, shape.window, shape.budget
    dev = wl.q.device
    st = torch.cuda.Stream()
    scores = torch.empty((S, Lyr, Hkv, W), dtype=torch.float32, device=dev)
    ws = torch.empty(max(K.kara_workspace_bytes(cfg) // 4, 1), dtype=torch.float32, device=dev)
    sel = torch.empty((S, Lyr, Hkv, B), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    K.kara_score_window(cfg, wl.q, wl.k_pool, wl.block_tables, wl.prior_lens, scores, ws, st)
    K.kara_select_chunks(cfg, scores, sel, None, st)
    st.synchronize()
    gen = np.random.default_rng(1234)
    units = S * Lyr * Hkv
    rnd = np.sort(np.argsort(gen.random((units, W)), axis=1)[:, :B], axis=1).astype(np.int32)
    r = torch.arange(B, dtype=torch.int32, device=dev)
    patterns = {
        "selection made by the step": sel,
        "dense in place (kept[r] = r)": r.expand(S, Lyr, Hkv, B).contiguous(),
        "dense shifted (kept[r] = r + W - B)": (r + (W - B)).expand(S, Lyr, Hkv, B).contiguous(),
        f"strided (kept[r] = {W // B} r)": (r * (W // B)).expand(S, Lyr, Hkv, B).contiguous(),
        "uniform random subset": torch.from_numpy(rnd).to(dev).view(S, Lyr, Hkv, B),
    }
    tables0 = wl.block_tables.clone()
    seq = torch.empty(S, dtype=torch.int32, device=dev)
    freed = torch.empty((S, K.kara_max_freed(cfg)), dtype=torch.int32, device=dev)
    nfreed = torch.empty(S, dtype=torch.int32, device=dev)
    esize = 2 if shape.dtype == "bf16" else 4
    nbytes = 2 * 2 * B * shape.head_dim * esize * units
    torch.cuda.synchronize()
    print(f"| Kept pattern ({a.workload}, {units} units, B = {B} of W = {W}) | ms per launch | GB/s |")
    print("|---|---|---|")
    for name, kept in patterns.items():
        ts = []
        for _ in range(a.reps + 1):
            with torch.cuda.stream(st):
                wl.block_tables.copy_(tables0)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(st)
            K.kara_compact_paged(cfg, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, seq, kept, freed,
                                 nfreed, st)
            ev[1].record(st)
            st.synchronize()
            ts.append(ev[0].elapsed_time(ev[1]))
        ms = float(np.median(ts[1:]))
        print(f"| {name} | {ms:.3f} | {nbytes / ms / 1e6:.0f} |", flush=True)
    with torch.cuda.stream(st):
        wl.block_tables.copy_(tables0)
    st.synchronize()


def main(argv=None):
    p = argparse.ArgumentParser(prog="python -m decode_kv_cache_amd.profiling")
    sub = p.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=2048)
    c.add_argument("--reps", type=int, default=3)
    sub.add_parser("peaks")
    cn = sub.add_parser("counters")
    cn.add_argument("dirs", nargs="+")
    s = sub.add_parser("stats")
    s.add_argument("dir")
    t = sub.add_parser("traffic")
    t.add_argument("--workload", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-fetch", required=True)
    t.add_argument("--copy-write", required=True)
    t.add_argument("--copy-mib", type=int, required=True)
    ci = sub.add_parser("coissue")
    ci.add_argument("--iters", type=int, default=20000)
    cc = sub.add_parser("coissue_cu")
    cc.add_argument("--iters", type=int, default=4000)
    cp = sub.add_parser("compact_patterns")
    cp.add_argument("--workload", default="llama8b_b64")
    cp.add_argument("--reps", type=int, default=5)
    a = p.parse_args(argv)
    {"coissue": cmd_coissue, "coissue_cu": cmd_coissue_cu, "compact_patterns": cmd_compact_patterns, "copy": cmd_copy, "peaks": cmd_peaks, "stats": cmd_stats, "traffic": cmd_traffic,
     "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    sys.exit(main())
