"""GPU parity of kara_compact_paged_tail against the fp64 oracle.

When the compressed window is the oldest part of the context not yet
compressed (reading R28, the gist.science explainer's periodic schedule), T
newer tokens follow it; they slide in order right behind the kept rows and
the table keeps the blocks of the first L + B + T slots.  The workloads are
generated with a longer window, so that real rows sit behind the compressed
one; every pool byte, table, length and freed list must equal the oracle's
compaction (compress_step with tail_lens) given the GPU kept lists.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_amd import kara as K
from decode_kv_cache_amd.workloads import KaraShape, make_workload
from tests.kara_harness import Outputs, bits

pytestmark = pytest.mark.gpu

CASES = [
    # (shape of the generated context, compressed window, budget, seeds, radius, tails)
    (KaraShape("tail_bf16", 971, num_seqs=4, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
               window=300 + 90, budget=60, seeds=3, radius=4, prior=("uniform", 5, 80)), 300, 60, 3, 4,
     [0, 1, 37, 90]),
    (KaraShape("tail_f32_bs4", 972, num_seqs=3, num_layers=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
               window=128 + 40, budget=32, seeds=2, radius=3, prior=("fixed", 10), block_size=4, dtype="f32"),
     128, 32, 2, 3, [40, 3, 0]),
    (KaraShape("tail_bs1", 973, num_seqs=2, num_layers=1, num_q_heads=2, num_kv_heads=1, head_dim=64,
               window=64 + 30, budget=9, seeds=1, radius=4, prior=("fixed", 7), block_size=1), 64, 9, 1, 4,
     [30, 29]),
    (KaraShape("tail_keep_all", 974, num_seqs=2, num_layers=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
               window=48 + 20, budget=48, seeds=1, radius=0, prior=("fixed", 16), block_size=16), 48, 48, 1, 0,
     [20, 5]),
]


@pytest.mark.parametrize("shape,W,B,s,r,tails", CASES, ids=[c[0].name for c in CASES])
def test_compaction_with_tail_matches_oracle(shape, W, B, s, r, tails):
    print(f"[tail] {shape.name} W={W} B={B} tails={tails}", flush=True)
    wl = make_workload(shape, "cuda")
    S = shape.num_seqs
    small = shape.with_(window=W, budget=B, seeds=s, radius=r)
    cfg = K.make_config(small, max_blocks_per_seq=wl.max_blocks, num_blocks=wl.num_blocks)
    q = wl.q[:, :, :W].contiguous()
    out = Outputs(cfg, "cuda")
    k_before, v_before = bits(wl.k_pool), bits(wl.v_pool)
    tables_before = wl.block_tables.cpu().numpy()
    tail_t = torch.tensor(tails, dtype=torch.int32, device="cuda")
    K.kara_score_window(cfg, q, wl.k_pool, wl.block_tables, wl.prior_lens, out["scores"], out.ws)
    K.kara_select_chunks(cfg, out["scores"], out["kept"])
    K.kara_compact_paged_tail(cfg, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, tail_t, out["seq_lens"],
                              out["kept"], out["freed"], out["num_freed"])
    torch.cuda.synchronize()
    assert out.guards_intact()
    ref = oracle.compress_step(np.zeros((S, small.num_layers, W, small.num_q_heads, 1)), k_before, v_before,
                               tables_before, wl.host_prior_lens, window=W, budget=B, seeds=s, radius=r,
                               block_size=small.block_size, scores_override=out["scores"].cpu().numpy(),
                               tail_lens=np.array(tails))
    assert np.array_equal(out["kept"].cpu().numpy(), ref["kept"])
    assert np.array_equal(bits(wl.k_pool), ref["k_pool"])
    assert np.array_equal(bits(wl.v_pool), ref["v_pool"])
    assert np.array_equal(wl.block_tables.cpu().numpy(), ref["block_tables"])
    assert np.array_equal(out["seq_lens"].cpu().numpy(), ref["seq_lens"])
    nf = out["num_freed"].cpu().numpy()
    fr = out["freed"].cpu().numpy()
    for n in range(S):
        assert nf[n] == ref["num_freed"][n] and fr[n, :nf[n]].tolist() == ref["freed"][n].tolist()
        assert np.all(fr[n, nf[n]:] == -1)


def test_zero_tails_equal_the_plain_compaction():
    shape = CASES[0][0]
    W, B, s, r = 300, 60, 3, 4
    res = []
    for with_tail in (False, True):
        wl = make_workload(shape, "cuda")
        small = shape.with_(window=W, budget=B, seeds=s, radius=r)
        cfg = K.make_config(small, max_blocks_per_seq=wl.max_blocks, num_blocks=wl.num_blocks)
        out = Outputs(cfg, "cuda")
        K.kara_score_window(cfg, wl.q[:, :, :W].contiguous(), wl.k_pool, wl.block_tables, wl.prior_lens,
                            out["scores"], out.ws)
        K.kara_select_chunks(cfg, out["scores"], out["kept"])
        args = (cfg, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens)
        rest = (out["seq_lens"], out["kept"], out["freed"], out["num_freed"])
        if with_tail:
            K.kara_compact_paged_tail(*args, torch.zeros(shape.num_seqs, dtype=torch.int32, device="cuda"), *rest)
        else:
            K.kara_compact_paged(*args, *rest)
        torch.cuda.synchronize()
        res.append([bits(wl.k_pool), bits(wl.v_pool), wl.block_tables.cpu().numpy()] +
                   [bits(out[k]) for k in ("seq_lens", "freed", "num_freed")])
    for a, b in zip(*res):
        assert np.array_equal(a, b)
