"""Parity at the full workload sizes, in the launch configuration the
benchmark times: sampled units against the fp64 oracle, and properties that
must hold for every unit."""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_amd.workloads import make_workload, shape_by_name
from tests.kara_harness import SCORE_RTOL, near_cutoff_ok, oracle_unit_attention, run_step, score_errors

pytestmark = pytest.mark.gpu


def _unit_rows(wl, pool, n, layer, g, start, count):
    bs = wl.shape.block_size
    pos = np.arange(start, start + count)
    blk = torch.from_numpy(wl.host_tables[n, pos // bs].astype(np.int64)).to(pool.device)
    off = torch.from_numpy((pos % bs).astype(np.int64)).to(pool.device)
    return pool[layer][blk, g, off, :]


def _bits(t):
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)).cpu().numpy()


@pytest.mark.parametrize("name", ["llama8b_b1", "llama8b_b64", "gqa7b", "large"])
def test_full_size_sampled(name):
    s = shape_by_name(name)
    print(f"[{name}] generating", flush=True)
    wl = make_workload(s, "cuda")
    S, Lyr, Hkv, W, B, G = s.num_seqs, s.num_layers, s.num_kv_heads, s.window, s.budget, s.group
    rng = np.random.default_rng(s.shape_id)
    units = {(0, 0, 0), (S - 1, Lyr - 1, Hkv - 1)}
    while len(units) < 6:
        units.add((int(rng.integers(S)), int(rng.integers(Lyr)), int(rng.integers(Hkv))))
    units = sorted(units)
    saved = {}
    for (n, layer, g) in units:
        L = int(wl.host_prior_lens[n])
        head = L % s.block_size
        qg = wl.q[n, layer, :, g * G:(g + 1) * G, :].float().double().permute(1, 0, 2).cpu().numpy()
        kw = _unit_rows(wl, wl.k_pool, n, layer, g, L, W)
        saved[(n, layer, g)] = dict(
            qg=qg, kw=kw.float().double().cpu().numpy(), kbits=_bits(kw),
            vbits=_bits(_unit_rows(wl, wl.v_pool, n, layer, g, L, W)),
            khead=_bits(_unit_rows(wl, wl.k_pool, n, layer, g, L - head, head)),
            vhead=_bits(_unit_rows(wl, wl.v_pool, n, layer, g, L - head, head)))
    print(f"[{name}] running the step", flush=True)
    cfg, out = run_step(wl)
    assert out.guards_intact()
    sc, kept, mask = out["scores"], out["kept"], out["mask"]
    # properties of every unit
    assert torch.isfinite(sc).all() and (sc >= 0).all()
    tot = sc.double().sum(-1)
    assert torch.allclose(tot, torch.full_like(tot, G * W), rtol=1e-4, atol=0)
    assert (kept[..., 1:] > kept[..., :-1]).all() and int(kept.min()) >= 0 and int(kept.max()) < W
    assert (mask.sum(-1, dtype=torch.int64) == B).all()
    assert (mask.gather(-1, kept.long()) == 1).all()
    # tables, lengths, freed lists of every sequence
    tables = wl.block_tables.cpu().numpy()
    freed = out["freed"].cpu().numpy()
    nfreed = out["num_freed"].cpu().numpy()
    lens = out["seq_lens"].cpu().numpy()
    for n in range(S):
        row, fr, new_len = oracle.rewrite_block_table(wl.host_tables[n], int(wl.host_prior_lens[n]), W, B,
                                                      s.block_size)
        assert np.array_equal(tables[n], row) and lens[n] == new_len and nfreed[n] == fr.size
        assert freed[n, :fr.size].tolist() == fr.tolist() and np.all(freed[n, fr.size:] == -1)
    # exact selection for a sample of units
    sc_h = sc.cpu().numpy()
    kept_h = kept.cpu().numpy()
    flat = rng.choice(S * Lyr * Hkv, size=min(64, S * Lyr * Hkv), replace=False)
    for u in flat:
        n, rest = divmod(int(u), Lyr * Hkv)
        layer, g = divmod(rest, Hkv)
        sel = oracle.token2chunk_select(sc_h[n, layer, g].astype(np.float64), B, s.seeds, s.radius)
        assert kept_h[n, layer, g].tolist() == sel.kept.tolist()
    # sampled units against the oracle: scores, selection band, compacted rows
    for (n, layer, g) in units:
        d = saved[(n, layer, g)]
        print(f"[{name}] oracle on unit {(n, layer, g)}", flush=True)
        c_orc = oracle.window_scores(d["qg"], d["kw"])
        err = score_errors(sc_h[n, layer, g], c_orc)
        assert err.max() <= SCORE_RTOL, (n, layer, g, float(err.max()))
        ok, nd = near_cutoff_ok(c_orc, kept_h[n, layer, g], B, s.seeds, s.radius)
        assert ok, (n, layer, g, nd)
        L = int(wl.host_prior_lens[n])
        head = L % s.block_size
        ka = _bits(_unit_rows(wl, wl.k_pool, n, layer, g, L, W))
        va = _bits(_unit_rows(wl, wl.v_pool, n, layer, g, L, W))
        kk = kept_h[n, layer, g]
        assert np.array_equal(ka, oracle.compact_window_rows(d["kbits"], kk))
        assert np.array_equal(va, oracle.compact_window_rows(d["vbits"], kk))
        assert np.array_equal(_bits(_unit_rows(wl, wl.k_pool, n, layer, g, L - head, head)), d["khead"])
        assert np.array_equal(_bits(_unit_rows(wl, wl.v_pool, n, layer, g, L - head, head)), d["vhead"])
    del wl, out
    torch.cuda.empty_cache()


def _sample_units(s, rng, k=6):
    S, Lyr, Hkv = s.num_seqs, s.num_layers, s.num_kv_heads
    units = {(0, 0, 0), (S - 1, Lyr - 1, Hkv - 1)}
    while len(units) < k:
        units.add((int(rng.integers(S)), int(rng.integers(Lyr)), int(rng.integers(Hkv))))
    return sorted(units)


@pytest.mark.parametrize("name", ["llama8b_b1", "llama8b_b64"])
def test_full_size_pipeline(name):
    """kara_compress_fused at full size: scores and kept lists equal to the
    separate calls on the same input, every table and length exact, and
    sampled units' compacted rows exact against the oracle."""
    from decode_kv_cache_amd import kara as K
    from tests.kara_harness import Outputs, config_of
    s = shape_by_name(name)
    print(f"[{name}] generating", flush=True)
    wl = make_workload(s, "cuda")
    S, Lyr, Hkv, W, B = s.num_seqs, s.num_layers, s.num_kv_heads, s.window, s.budget
    cfg = config_of(wl)
    ref = Outputs(cfg, "cuda")
    K.kara_score_window(cfg, wl.q, wl.k_pool, wl.block_tables, wl.prior_lens, ref["scores"], ref.ws)
    K.kara_select_chunks(cfg, ref["scores"], ref["kept"])
    rng = np.random.default_rng(s.shape_id + 17)
    units = _sample_units(s, rng)
    saved = {u: (_bits(_unit_rows(wl, wl.k_pool, *u, int(wl.host_prior_lens[u[0]]), W)),
                 _bits(_unit_rows(wl, wl.v_pool, *u, int(wl.host_prior_lens[u[0]]), W))) for u in units}
    out = Outputs(cfg, "cuda")
    done = torch.zeros(S, dtype=torch.int32, device="cuda")
    print(f"[{name}] one-launch pipeline", flush=True)
    K.kara_compress_fused(cfg, wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, out["scores"],
                          out["kept"], out["seq_lens"], out["freed"], out["num_freed"], done)
    torch.cuda.synchronize()
    assert torch.all(done == 0)
    assert torch.equal(out["scores"], ref["scores"]) and torch.equal(out["kept"], ref["kept"])
    tables, lens = wl.block_tables.cpu().numpy(), out["seq_lens"].cpu().numpy()
    freed, nfreed = out["freed"].cpu().numpy(), out["num_freed"].cpu().numpy()
    for n in range(S):
        row, fr, new_len = oracle.rewrite_block_table(wl.host_tables[n], int(wl.host_prior_lens[n]), W, B,
                                                      s.block_size)
        assert np.array_equal(tables[n], row) and lens[n] == new_len and nfreed[n] == fr.size
        assert freed[n, :fr.size].tolist() == fr.tolist()
    kept_h = out["kept"].cpu().numpy()
    for u in units:
        L = int(wl.host_prior_lens[u[0]])
        kk = kept_h[u]
        assert np.array_equal(_bits(_unit_rows(wl, wl.k_pool, *u, L, W)), oracle.compact_window_rows(saved[u][0], kk))
        assert np.array_equal(_bits(_unit_rows(wl, wl.v_pool, *u, L, W)), oracle.compact_window_rows(saved[u][1], kk))
    del wl, out, ref
    torch.cuda.empty_cache()


def test_full_size_decode_attention_after_compaction():
    """Decode attention over the compacted 64-sequence 8B cache (random prior
    context) against the oracle for every query head of sampled units."""
    from decode_kv_cache_amd import kara as K
    from decode_kv_cache_amd.workloads import decode_queries, fill_prior_context
    from tests.test_gpu_attention import ATTN_ATOL, ATTN_RTOL
    s = shape_by_name("llama8b_b64")
    print("[attention] generating", flush=True)
    wl = make_workload(s, "cuda")
    fill_prior_context(wl)
    q_dec = decode_queries(s, "cuda")
    print("[attention] compressing", flush=True)
    cfg, out = run_step(wl, with_mask=False)
    att = torch.full((s.num_seqs, s.num_layers, s.num_q_heads, s.head_dim), float("nan"), device="cuda")
    wsb = K.kara_decode_attention_workspace_bytes(cfg)
    ws = torch.empty(wsb // 4 + 64, dtype=torch.float32, device="cuda") if wsb else None
    K.kara_decode_attention(cfg, q_dec, wl.k_pool, wl.v_pool, wl.block_tables, out["seq_lens"], att, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(att).all()
    att_h = att.cpu().numpy().astype(np.float64)
    G, d = s.group, s.head_dim
    rng = np.random.default_rng(99)
    for (n, layer, g) in _sample_units(s, rng):
        T = int(wl.host_prior_lens[n]) + s.budget
        print(f"[attention] oracle on unit {(n, layer, g)}, {T} slots", flush=True)
        Kd = _unit_rows(wl, wl.k_pool, n, layer, g, 0, T).float().double().cpu().numpy()
        Vd = _unit_rows(wl, wl.v_pool, n, layer, g, 0, T).float().double().cpu().numpy()
        qh = q_dec[n, layer, g * G:(g + 1) * G].float().double().cpu().numpy()
        o = oracle_unit_attention(qh, Kd, Vd)
        got = att_h[n, layer, g * G:(g + 1) * G]
        assert np.all(np.abs(got - o) <= ATTN_ATOL + ATTN_RTOL * np.abs(o)), (n, layer, g)
    del wl, out
    torch.cuda.empty_cache()
