#!/usr/bin/env python3
"""Benchmark of the Kara window-compression step on one MI355X.

One step = kara_score_window + kara_select_chunks + kara_compact_paged over
every (sequence, layer, KV head) of the workload, inputs resident in HBM.
Between steps the blocks that compaction writes (those holding the slots
[L, L+B) of each window) and the block tables are restored from a pristine
copy (outside the timed events; compaction is in place), and once, before the
timed steps, every window block is checked against that copy.

After the timed steps, the consumer of the cache (one decode step of paged
attention, kara_decode_attention) is timed over the compacted cache (L + B
slots per sequence) and over the same cache before compaction (L + W slots),
and reported with its HBM roofline beside the step.

Prints ONE JSON line: metric, value (window tokens per second), per-stage
times, the roofline of the dominant kernel, and the fp64 CPU oracle timed on
a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "window tokens compressed/sec (score+select+compact), 8B shape; % of roofline"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="llama8b_b64")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU work of the oracle sample")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-peaks", action="store_true", help="skip the achievable-peak probes")
    p.add_argument("--consumer-reps", type=int, default=10,
                   help="timed decode-attention passes over the cache before and after compaction (0: skip)")
    return p.parse_args()


def run_environment(dev) -> dict:
    """What the line was measured on: GPU, its compute units and clock, the
    HIP runtime and torch builds, the library's source hash."""
    import torch
    p = torch.cuda.get_device_properties(dev)
    env = {"gpu": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
           "hip": torch.version.hip, "torch": torch.__version__}
    clock = getattr(p, "clock_rate", None)
    if clock:
        env["max_clock_mhz"] = round(clock / 1000.0)
    return env


def scorer_kernel(shape, passes: int) -> str:
    """The kernel(s) kara_score_window launches for this shape."""
    if passes == 2:
        return "row_lse_kernel + col_mass_kernel"
    resident = shape.dtype == "bf16" and shape.head_dim == 128 and shape.window <= 1024
    return "fused_score_kernel" if resident else "small_score_kernel"


def kernel_source_hash():
    from decode_kv_cache_amd.profiling import kernel_source_hash as h
    return h()


def measured_traffic(workload, kernel_hash):
    """HBM bytes per launch of the scoring call from committed PMC runs, if the
    kernels have not changed since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(workload)
    if not rec or rec.get("kernel_hash") != kernel_hash:
        return None
    return rec.get("score_bytes_per_launch")


# ----------------------------------------------------------------------------- CPU oracle baseline
def _oracle_unit(args):
    import numpy as np
    import oracle
    qg, kw, krows, vrows, B, s, r = args
    t0 = time.perf_counter()
    c = oracle.window_scores(qg, kw)
    sel = oracle.token2chunk_select(c, B, s, r)
    oracle.compact_window_rows(krows, sel.kept)
    oracle.compact_window_rows(vrows, sel.kept)
    return time.perf_counter() - t0


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def cpu_workers():
    """Worker processes of the oracle pool: one per CPU this process may run
    on, at most 16 (the host's CPU share per GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, shape, target_s):
    """Time the oracle (score + select + compact per unit) on a seeded sample."""
    import multiprocessing as mp

    import numpy as np
    import torch
    procs = cpu_workers()
    rng = np.random.default_rng(1234)
    G, W, bs = shape.group, shape.window, shape.block_size

    def unit_args(u):
        n, rest = divmod(int(u), shape.num_layers * shape.num_kv_heads)
        layer, g = divmod(rest, shape.num_kv_heads)
        L = int(wl.host_prior_lens[n])
        pos = np.arange(L, L + W)
        blk = torch.from_numpy(wl.host_tables[n, pos // bs].astype(np.int64)).to(wl.k_pool.device)
        off = torch.from_numpy((pos % bs).astype(np.int64)).to(wl.k_pool.device)
        kr = wl.k_pool[layer][blk, g, off, :]
        vr = wl.v_pool[layer][blk, g, off, :]
        qg = wl.q[n, layer, :, g * G:(g + 1) * G, :].permute(1, 0, 2)
        bits = torch.int16 if kr.dtype == torch.bfloat16 else torch.int32
        return (qg.double().cpu().numpy(), kr.double().cpu().numpy(), kr.view(bits).cpu().numpy(),
                vr.view(bits).cpu().numpy(), shape.budget, shape.seeds, shape.radius)

    units = shape.units
    t1 = _oracle_unit(unit_args(0))                    # calibration (single unit, this process)
    n = int(max(procs, min(units, round(target_s * procs / max(t1, 1e-6)))))
    n = min(n, units, 4096)
    sample = rng.choice(units, size=n, replace=False)
    work = [unit_args(u) for u in sample]
    ctx = mp.get_context("fork")
    with ctx.Pool(procs, initializer=_pool_init) as pool:
        t0 = time.perf_counter()
        pool.map(_oracle_unit, work, chunksize=1)
        wall = time.perf_counter() - t0
    est_total = wall * units / n
    tokens = shape.num_seqs * shape.window
    return {"value": tokens / est_total, "unit": "window tokens/s", "cores": procs, "kind": "oracle",
            "cpu_model": cpu_model(), "cpus_visible": len(os.sched_getaffinity(0)),
            "sample": f"{n} of {units} units (seeded), fp64 numpy score+select+compact per unit, "
                      f"{procs} worker processes x 1 BLAS thread, {wall:.1f} s wall; extrapolated linearly "
                      f"to all units"}


# ----------------------------------------------------------------------------- main
def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only: the step has no cross-GPU work (units shard with no exchange); "
              f"got --gpus {a.gpus}", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from decode_kv_cache_amd import kara as K
    from decode_kv_cache_amd.workloads import make_workload, shape_by_name

    shape = shape_by_name(a.workload)
    dev = torch.device("cuda:0")
    log(f"[bench] generating {shape.name} ({shape.description})")
    t0 = time.time()
    wl = make_workload(shape, dev)
    torch.cuda.synchronize()
    log(f"[bench] generated in {time.time() - t0:.1f} s; pool {wl.k_pool.numel() * wl.k_pool.element_size() / 1e9:.1f} GB x2")
    cfg = K.make_config(shape, max_blocks_per_seq=wl.max_blocks, num_blocks=wl.num_blocks)
    S, Lyr, Hkv, W, B = shape.num_seqs, shape.num_layers, shape.num_kv_heads, shape.window, shape.budget
    scores = torch.empty((S, Lyr, Hkv, W), dtype=torch.float32, device=dev)
    kept = torch.empty((S, Lyr, Hkv, B), dtype=torch.int32, device=dev)
    ws = torch.empty((K.kara_workspace_bytes(cfg) + 255) // 4 + 64, dtype=torch.float32, device=dev)
    seq_lens = torch.empty(S, dtype=torch.int32, device=dev)
    freed = torch.empty((S, K.kara_max_freed(cfg)), dtype=torch.int32, device=dev)
    nfreed = torch.empty(S, dtype=torch.int32, device=dev)

    # pristine copy of every block a window touches, and of the tables.  A
    # step writes only the slots [L, L+B) of each window (compaction), so the
    # restore before each step copies back just the blocks that hold them; a
    # check after the warm-up compares every window block with the copy.
    bs = shape.block_size
    blocks, written = [], []
    for n in range(S):
        L = int(wl.host_prior_lens[n])
        blocks.extend(wl.host_tables[n, L // bs: -(-(L + W) // bs)].tolist())
        written.extend(wl.host_tables[n, L // bs: -(-(L + B) // bs)].tolist())
    blk_idx = torch.tensor(blocks, dtype=torch.int64, device=dev)
    k_save = wl.k_pool.index_select(1, blk_idx)
    v_save = wl.v_pool.index_select(1, blk_idx)
    pos_in_save = {b: i for i, b in enumerate(blocks)}
    wr_idx = torch.tensor(written, dtype=torch.int64, device=dev)
    wr_sel = torch.tensor([pos_in_save[b] for b in written], dtype=torch.int64, device=dev)
    k_wsave = k_save.index_select(1, wr_sel)
    v_wsave = v_save.index_select(1, wr_sel)
    tables_save = wl.block_tables.clone()
    # everything above ran on the default stream; the bench stream must not
    # start (restores read these copies) before it has finished
    torch.cuda.synchronize()

    st = torch.cuda.Stream(device=dev)
    def restore():
        with torch.cuda.stream(st):
            wl.k_pool.index_copy_(1, wr_idx, k_wsave)
            wl.v_pool.index_copy_(1, wr_idx, v_wsave)
            wl.block_tables.copy_(tables_save)

    def pools_pristine():
        """Every window block equals its pristine copy (after a restore)."""
        with torch.cuda.stream(st):
            ok = torch.equal(wl.k_pool.index_select(1, blk_idx), k_save) and \
                torch.equal(wl.v_pool.index_select(1, blk_idx), v_save)
        torch.cuda.synchronize()
        return ok

    def step(e=None):
        if e:
            e[0].record(st)
        K.kara_score_window(cfg, wl.q, wl.k_pool, wl.block_tables, wl.prior_lens, scores, ws, st)
        if e:
            e[1].record(st)
        K.kara_select_chunks(cfg, scores, kept, None, st)
        if e:
            e[2].record(st)
        K.kara_compact_paged(cfg, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, seq_lens, kept, freed,
                             nfreed, st)
        if e:
            e[3].record(st)

    def tables_match(upto_budget):
        """Device block tables equal the workload's host copy over every
        sequence's window blocks (after a restore) or over the blocks that
        hold only kept slots (after a step)."""
        got = wl.block_tables.cpu().numpy()
        for n in range(S):
            L = int(wl.host_prior_lens[n])
            upto = (L + B) // bs if upto_budget else -(-(L + W) // bs)
            if not np.array_equal(got[n, :upto], wl.host_tables[n, :upto]):
                return False
        return True

    restore()
    torch.cuda.synchronize()
    if not tables_match(False):
        sys.exit("bench: block tables differ from the workload after a restore")
    # the library's own check of the addressing data before any step trusts it
    bad = torch.full((1,), -1, dtype=torch.int32, device=dev)
    K.kara_validate_tables(cfg, wl.block_tables, wl.prior_lens, bad, st)
    torch.cuda.synchronize()
    if int(bad.item()) != 0:
        sys.exit(f"bench: kara_validate_tables reports {int(bad.item())} sequences with out-of-range entries")
    for _ in range(a.warmup):
        restore()
        step()
    restore()
    torch.cuda.synchronize()
    if not pools_pristine():
        sys.exit("bench: a restore does not return the window blocks to their pristine contents")
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(a.steps)]
    log(f"[bench] timing {a.steps} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(a.steps):
        restore()
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    if not tables_match(True):
        sys.exit("bench: block tables of the kept slots changed during the timed steps")
    t_score = [e[0].elapsed_time(e[1]) for e in events]
    t_sel = [e[1].elapsed_time(e[2]) for e in events]
    t_cmp = [e[2].elapsed_time(e[3]) for e in events]
    ms = [x + y + z for x, y, z in zip(t_score, t_sel, t_cmp)]
    ms_step = float(np.mean(ms))
    tokens = S * W
    value = tokens / (ms_step / 1e3)
    log(f"[bench] step {ms_step:.3f} ms (score {np.mean(t_score):.3f}, select {np.mean(t_sel):.3f}, "
        f"compact {np.mean(t_cmp):.3f}); wall incl. restores {wall / a.steps * 1e3:.3f} ms/step")

    # roofline of the dominant call (scoring: one Q K^T per unit)
    G, d = shape.group, shape.head_dim
    flops = 2.0 * G * W * W * d * shape.units
    t_s = float(np.mean(t_score)) / 1e3
    achieved = flops / t_s / 1e12
    peak = PEAK_TFLOPS[shape.dtype]
    khash = kernel_source_hash()
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": measured_traffic(shape.name, khash),
            "kernel": scorer_kernel(shape, K.kara_score_passes(cfg)) + " (kara_score_window)",
            "algorithmic": f"2*G*W^2*d = {2 * G * W * W * d:.4g} FLOP per unit x {shape.units} units"}
    cbytes = 4.0 * B * d * shape.elem_bytes * shape.units
    t_c = float(np.mean(t_cmp)) / 1e3
    compact_roof = {"bound": "hbm", "achieved": round(cbytes / t_c / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(cbytes / t_c / 1e9 / PEAK_HBM_GBS, 4),
                    "algorithmic": f"4*B*d*elem = {4 * B * d * shape.elem_bytes} B per unit x {shape.units} units"}

    # the same step in one launch (kara_compress_fused), where offered
    fused = None
    if K.kara_compress_fused_supported(cfg):
        done = torch.zeros(S, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()                   # the counters are zero before the bench stream reads them

        def fused_step():
            K.kara_compress_fused(cfg, wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, scores, kept,
                                  seq_lens, freed, nfreed, done, stream=st)

        for _ in range(a.warmup):
            restore()
            fused_step()
        torch.cuda.synchronize()
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(a.steps)]
        for i in range(a.steps):
            restore()
            fev[i][0].record(st)
            fused_step()
            fev[i][1].record(st)
        torch.cuda.synchronize()
        ms_fused = float(np.mean([e[0].elapsed_time(e[1]) for e in fev]))
        fused = {"call": "kara_compress_fused (score + select + compact + table rewrite, one launch)",
                 "ms_per_step": round(ms_fused, 4), "value": round(tokens / (ms_fused / 1e3), 1),
                 "vs_three_calls": round(ms_step / ms_fused, 4)}
        log(f"[bench] one-launch pipeline {ms_fused:.3f} ms/step ({ms_step / ms_fused:.3f}x the three calls)")

    # the bridging variant of the selection (largest gap the budget admits, up to 16)
    bridged = None
    gap = max([g_ for g_ in range(0, 17) if 0 <= K.kara_chunk_bound(cfg, g_) <= B], default=0)
    if shape.seeds > 1 and gap > 0:
        kept_b = torch.empty_like(kept)

        def sel_ms(fn, reps=10):
            fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(st)
            for _ in range(reps):
                fn()
            ev[1].record(st)
            torch.cuda.synchronize()
            return ev[0].elapsed_time(ev[1]) / reps

        t_plain = sel_ms(lambda: K.kara_select_chunks(cfg, scores, kept_b, None, st))
        t_bridge = sel_ms(lambda: K.kara_select_chunks_bridged(cfg, gap, scores, kept_b, None, st))
        bridged = {"call": "kara_select_chunks_bridged", "gap": gap, "ms": round(t_bridge, 4),
                   "ms_plain_select": round(t_plain, 4)}
        log(f"[bench] bridged selection (gap {gap}) {t_bridge:.3f} ms, plain {t_plain:.3f} ms")

    consumer = None
    if a.consumer_reps > 0:
        from decode_kv_cache_amd.workloads import decode_queries
        q_dec = decode_queries(shape, dev)
        torch.cuda.synchronize()                   # drawn on the default stream, read on the bench stream
        att = torch.empty((S, Lyr, shape.num_q_heads, d), dtype=torch.float32, device=dev)
        aws = torch.empty(K.kara_decode_attention_workspace_bytes(cfg) // 4 + 64, dtype=torch.float32, device=dev)

        def attend_ms(lens):
            for _ in range(2):
                K.kara_decode_attention(cfg, q_dec, wl.k_pool, wl.v_pool, wl.block_tables, lens, att, aws, st)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(st)
            for _ in range(a.consumer_reps):
                K.kara_decode_attention(cfg, q_dec, wl.k_pool, wl.v_pool, wl.block_tables, lens, att, aws, st)
            ev[1].record(st)
            torch.cuda.synchronize()
            return ev[0].elapsed_time(ev[1]) / a.consumer_reps

        kv_row = Lyr * Hkv * d * shape.elem_bytes * 2          # K and V bytes per slot over all layers
        res = {}
        for tag, lens in (("compacted", seq_lens), ("full", None)):
            if lens is None:
                restore()
                torch.cuda.synchronize()
                lens = (wl.prior_lens + W).to(torch.int32)
            n_slots = int(lens.sum().item())
            t_ms = attend_ms(lens)
            res[tag] = (t_ms, n_slots * kv_row)
        (tc, bc), (tf, bf) = res["compacted"], res["full"]
        consumer = {"call": "kara_decode_attention (one decode step, every sequence, layer and query head)",
                    "ms_compacted": round(tc, 4), "ms_full": round(tf, 4), "speedup": round(tf / tc, 4),
                    "kv_bytes_compacted": bc, "kv_bytes_full": bf,
                    "roofline": {"bound": "hbm", "achieved": round(bc / tc / 1e6, 1), "peak": PEAK_HBM_GBS,
                                 "unit": "GB/s", "frac": round(bc / tc / 1e6 / PEAK_HBM_GBS, 4),
                                 "algorithmic": "2 * seq_len * num_layers * num_kv_heads * head_dim * elem bytes "
                                                "(each cached K and V row read once)"},
                    "splits": K.kara_decode_attention_splits(cfg)}
        log(f"[bench] decode attention: compacted {tc:.3f} ms ({bc / tc / 1e6:.0f} GB/s), full {tf:.3f} ms")

    achievable = None
    if not a.no_peaks:
        from decode_kv_cache_amd.profiling import achievable_peaks
        achievable = achievable_peaks()
        log(f"[bench] achievable peaks: {achievable}")
        roof["frac_of_achievable"] = round(roof["achieved"] / achievable["mfma_bf16_tflops"], 4) \
            if shape.dtype == "bf16" else None
        # the softmax around the MFMA: per logit one v_exp_f32 and four full-rate
        # fp32 VALU operations (scale-and-shift, row sum, column update, max)
        logits = float(G) * W * W * shape.units
        floor_s = logits * (4.0 / achievable["fma_f32_per_s"] + 1.0 / achievable["v_exp_f32_per_s"])
        roof["alu_floor"] = {"bound": "alu", "floor_ms": round(floor_s * 1e3, 3),
                             "frac": round(floor_s / t_s, 4),
                             "basis": "G*W^2 logits per unit x (4 fp32 VALU ops at the probed FMA rate + 1 "
                                      "v_exp_f32 at the probed exp rate); packed fp32 is not used"}
        compact_roof["frac_of_achievable"] = round(compact_roof["achieved"] / max(
            achievable["hbm_copy_GBps_read_plus_write"], achievable["hbm_rewrite_in_place_GBps_read_plus_write"]), 4)
        if consumer:
            consumer["roofline"]["frac_of_achievable"] = round(consumer["roofline"]["achieved"] /
                                                               achievable["hbm_read_GBps"], 4)

    cpu = None
    if not a.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on a CPU sample")
        cpu = cpu_baseline(wl, shape, a.cpu_seconds)
        log(f"[bench] cpu baseline {cpu['value']:.1f} tokens/s ({cpu['sample']})")

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "window tokens/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": shape.dtype, "data": "synthetic",
        "config": {"workload": shape.name, "num_seqs": S, "num_layers": Lyr, "num_q_heads": shape.num_q_heads,
                   "num_kv_heads": Hkv, "head_dim": d, "window": W, "budget": B, "seeds": shape.seeds,
                   "radius": shape.radius, "block_size": bs, "prior": list(shape.prior),
                   "key_model": shape.key_model, "plants": shape.plants, "parallelism": "single GPU"},
        "stages_ms": {"score": round(float(np.mean(t_score)), 4), "select": round(float(np.mean(t_sel)), 4),
                      "compact": round(float(np.mean(t_cmp)), 4)},
        "step_ms_median": round(float(np.median(ms)), 4), "step_ms_min": round(float(np.min(ms)), 4),
        "roofline": roof,
        "compact_roofline": compact_roof,
        "fused_pipeline": fused,
        "select_bridged": bridged,
        "decode_attention": consumer,
        "cpu_baseline": cpu,
        "achievable_peaks": achievable,
        "kernel_hash": khash,
        "wall_ms_per_step_incl_restore": round(wall / a.steps * 1e3, 3),
        "env": run_environment(dev),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
