"""Reentrancy through the C ABI: the library keeps no state between calls,
so two independent steps enqueued at the same time on two streams give,
bit for bit, what the same steps give one after the other."""
import numpy as np
import pytest
import torch

from decode_kv_cache_amd import kara as K
from decode_kv_cache_amd.workloads import KaraShape, make_workload
from tests.kara_harness import Outputs, bits, config_of, run_step

pytestmark = pytest.mark.gpu

# one shape per scorer: the single-pass kernel (bf16, d 128) and the two passes (fp32, d 64)
SHAPES = (
    KaraShape("streams_fused", 301, num_seqs=3, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
              window=512, budget=100, seeds=4, radius=3, prior=("uniform", 10, 400)),
    KaraShape("streams_two_pass", 302, num_seqs=2, num_layers=2, num_q_heads=6, num_kv_heads=2, head_dim=64,
              window=700, budget=150, seeds=5, radius=4, prior=("uniform", 0, 300), block_size=8, dtype="f32"),
)


def _state(wl, out):
    return dict(scores=out["scores"].cpu().numpy(), kept=out["kept"].cpu().numpy(), mask=out["mask"].cpu().numpy(),
                seq_lens=out["seq_lens"].cpu().numpy(), freed=out["freed"].cpu().numpy(),
                num_freed=out["num_freed"].cpu().numpy(), k=bits(wl.k_pool), v=bits(wl.v_pool),
                tables=wl.block_tables.cpu().numpy())


def test_two_steps_on_two_streams_match_serial_runs():
    # serial reference: each step alone on the default stream
    serial = []
    for s in SHAPES:
        wl = make_workload(s, "cuda")
        _, out = run_step(wl)
        serial.append(_state(wl, out))
    # the same inputs again (the generators are seeded), now interleaved on two streams
    wls = [make_workload(s, "cuda") for s in SHAPES]
    cfgs = [config_of(wl) for wl in wls]
    outs = [Outputs(cfg, "cuda") for cfg in cfgs]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()                 # inputs and guard fills were written on the default stream
    for i in range(2):
        wl, cfg, out, st = wls[i], cfgs[i], outs[i], streams[i]
        K.kara_score_window(cfg, wl.q, wl.k_pool, wl.block_tables, wl.prior_lens, out["scores"], out.ws, st)
    for i in range(2):
        cfg, out, st = cfgs[i], outs[i], streams[i]
        K.kara_select_chunks(cfg, out["scores"], out["kept"], out["mask"], st)
    for i in range(2):
        wl, cfg, out, st = wls[i], cfgs[i], outs[i], streams[i]
        K.kara_compact_paged(cfg, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, out["seq_lens"],
                             out["kept"], out["freed"], out["num_freed"], st)
    torch.cuda.synchronize()
    for i, s in enumerate(SHAPES):
        assert outs[i].guards_intact(), s.name
        got = _state(wls[i], outs[i])
        for key, ref in serial[i].items():
            assert np.array_equal(got[key], ref, equal_nan=True) if ref.dtype.kind == "f" else \
                np.array_equal(got[key], ref), (s.name, key)
