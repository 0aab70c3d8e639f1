"""Full-size parity over every unit of one sequence, in the launch
configuration the benchmark times (the three calls over the whole workload).

For the last sequence of each full-size workload:
  - scores of every (layer, KV head) unit against the fp64 oracle (2e-3
    relative, floor 1e-30); on the 80-layer shape, whose oracle takes about
    2.5 s per unit, every unit of the sequence's last layer;
  - the kept list of every unit equal to the oracle's selection on the GPU
    scores, and any difference from the oracle's selection on its own scores
    a near-tie at a cutoff;
  - every byte of the sequence's window blocks, in every layer, K and V,
    equal to the oracle's in-place compaction of the pre-step blocks with the
    GPU kept lists: the compacted rows, the stale tail rows, the prior rows
    that share the first block and the contents of the freed blocks;
  - the sequence's table row, freed list and length.
The oracle runs in a process pool of one worker per visible CPU (at most 16),
one BLAS thread each.
"""
import multiprocessing as mp
import os

import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_amd.workloads import make_workload, shape_by_name
from tests.kara_harness import SCORE_RTOL, near_cutoff_ok, run_step, score_errors

pytestmark = pytest.mark.gpu

_UNITS = {}          # inputs of the oracle workers (inherited through fork)


def _pool_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _scores_of(key):
    qg, kw = _UNITS[key]
    return key, oracle.window_scores(qg, kw)


def _bits(t):
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).cpu().numpy()


@pytest.mark.parametrize("name", ["llama8b_b1", "llama8b_b64", "gqa7b", "large"])
def test_every_unit_of_one_sequence(name):
    s = shape_by_name(name)
    print(f"[{name}] generating", flush=True)
    wl = make_workload(s, "cuda")
    S, Lyr, Hkv, W, B, G, bs = s.num_seqs, s.num_layers, s.num_kv_heads, s.window, s.budget, s.group, s.block_size
    n = S - 1
    L = int(wl.host_prior_lens[n])
    lb0, lb1 = L // bs, -(-(L + W) // bs)                 # logical blocks holding [L - L % bs, L + W)
    blocks = wl.host_tables[n, lb0:lb1].astype(np.int64)
    blk_t = torch.from_numpy(blocks).cuda()
    k_before = _bits(wl.k_pool.index_select(1, blk_t))    # [layers][window blocks][Hkv][bs][d]
    v_before = _bits(wl.v_pool.index_select(1, blk_t))
    layers = range(Lyr) if name != "large" else [Lyr - 1]
    _UNITS.clear()
    pos = torch.from_numpy(np.arange(L, L + W)).cuda()
    kb = torch.from_numpy(wl.host_tables[n].astype(np.int64)).cuda()[pos // bs]
    ko = pos % bs
    for layer in layers:
        qn = wl.q[n, layer].float().double().cpu().numpy()                 # [W][Hq][d]
        kn = wl.k_pool[layer][kb, :, ko, :].float().double().cpu().numpy()  # [W][Hkv][d]
        for g in range(Hkv):
            _UNITS[(layer, g)] = (np.ascontiguousarray(np.transpose(qn[:, g * G:(g + 1) * G, :], (1, 0, 2))),
                                  np.ascontiguousarray(kn[:, g, :]))
    print(f"[{name}] running the step", flush=True)
    cfg, out = run_step(wl, with_mask=False)
    assert out.guards_intact()
    sc = out["scores"].cpu().numpy()[n]
    kept = out["kept"].cpu().numpy()[n]
    # scores and the selection band, in a process pool
    procs = max(1, min(16, len(os.sched_getaffinity(0)), len(_UNITS)))
    print(f"[{name}] oracle scores of {len(_UNITS)} units of sequence {n} on {procs} processes", flush=True)
    with mp.get_context("fork").Pool(procs, initializer=_pool_init) as pool:
        for (layer, g), c_orc in pool.imap_unordered(_scores_of, list(_UNITS), chunksize=1):
            err = score_errors(sc[layer, g], c_orc)
            assert err.max() <= SCORE_RTOL, (layer, g, float(err.max()))
            ok, nd = near_cutoff_ok(c_orc, kept[layer, g], B, s.seeds, s.radius)
            assert ok, (layer, g, nd)
    _UNITS.clear()
    # exact selection on the GPU scores, every unit of the sequence
    for layer in range(Lyr):
        for g in range(Hkv):
            sel = oracle.token2chunk_select(sc[layer, g].astype(np.float64), B, s.seeds, s.radius)
            assert kept[layer, g].tolist() == sel.kept.tolist(), (layer, g)
    # every byte of the window blocks: the oracle compacts a copy of them
    # through a table that maps the sequence's logical blocks onto the copy
    print(f"[{name}] compaction of {Lyr * Hkv} units against the oracle", flush=True)
    sub_table = np.full(lb1, -1, dtype=np.int64)
    sub_table[lb0:lb1] = np.arange(lb1 - lb0)
    k_ref, v_ref = k_before.copy(), v_before.copy()
    oracle.compact_paged_sequence(k_ref, v_ref, sub_table, L, kept.astype(np.int64), bs)
    assert np.array_equal(_bits(wl.k_pool.index_select(1, blk_t)), k_ref)
    assert np.array_equal(_bits(wl.v_pool.index_select(1, blk_t)), v_ref)
    # the sequence's table row, freed list and length
    row, fr, new_len = oracle.rewrite_block_table(wl.host_tables[n], L, W, B, bs)
    assert np.array_equal(wl.block_tables.cpu().numpy()[n], row)
    assert int(out["seq_lens"].cpu()[n]) == new_len and int(out["num_freed"].cpu()[n]) == fr.size
    assert out["freed"].cpu().numpy()[n, :fr.size].tolist() == fr.tolist()
    del wl, out
    torch.cuda.empty_cache()
