"""Multi-round run of the periodic scheduler on the GPU path, every tick
checked against the fp64 oracle applied to the cache as it was before that
tick: scores within the score tolerance, kept lists, pools, block tables,
lengths and freed blocks bit for bit.  The windows are the oldest uncompressed
tokens, and the newer tokens behind them move down with the compaction."""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_amd.scheduler import TRACES, run_trace
from tests.kara_harness import SCORE_RTOL, score_errors

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()


def test_tiny_trace_every_tick_matches_the_oracle():
    spec = TRACES["tiny_trace"]
    rec = []
    rep = run_trace(spec, "cuda", record=rec)
    print(rep, flush=True)
    assert rep["compressions"] >= 4 and len(rec) >= 2
    # the schedule really carries tails: some windows had newer tokens behind them
    assert any(int(t) > 0 for r in rec for t in r["tail"])
    assert rep["blocks_in_use_at_end"] == 0
    assert rep["peak_saving"] > 0
    G = spec.num_q_heads // spec.num_kv_heads
    for r in rec:
        q = r["q"].float().double().numpy()
        k64 = r["pre_k"].float().double().numpy()
        for i, n in enumerate(r["seqs"]):
            for layer in range(spec.num_layers):
                for g in range(spec.num_kv_heads):
                    qg = np.transpose(q[i, layer, :, g * G:(g + 1) * G, :], (1, 0, 2))
                    kw = oracle.gather_window_rows(k64, r["pre_tables"][i], layer, g, int(r["prior"][i]),
                                                   spec.window, spec.block_size)
                    err = score_errors(r["scores"][i, layer, g].numpy(), oracle.window_scores(qg, kw))
                    assert err.max() <= SCORE_RTOL
        ref = oracle.compress_step(np.zeros((len(r["seqs"]), spec.num_layers, spec.window, spec.num_q_heads, 1)),
                                   _bits(r["pre_k"]), _bits(r["pre_v"]), r["pre_tables"], r["prior"],
                                   window=spec.window, budget=spec.budget, seeds=spec.seeds, radius=spec.radius,
                                   block_size=spec.block_size, scores_override=r["scores"].numpy(),
                                   tail_lens=r["tail"])
        assert np.array_equal(ref["kept"], r["kept"].numpy())
        assert np.array_equal(ref["k_pool"], _bits(r["post_k"]))
        assert np.array_equal(ref["v_pool"], _bits(r["post_v"]))
        assert np.array_equal(ref["block_tables"], r["post_tables"])
        assert np.array_equal(ref["seq_lens"], r["seq_lens"])
        for a, b in zip(ref["freed"], r["freed"]):
            assert a.tolist() == b.tolist()
