"""Unit records for offline re-checks (decode_kv_cache_amd.unit_dump): a
record of a step re-checks clean against the oracle, and every kind of wrong
output in a record is caught.  The CPU tests build the outputs with the oracle
itself; the GPU test records real kernel outputs."""
import numpy as np
import pytest
import torch

import oracle
from decode_kv_cache_amd.unit_dump import load_unit, save_unit, unit_inputs, unit_outputs
from decode_kv_cache_amd.workloads import KaraShape, make_workload
from tests.kara_harness import config_of
from tests.unit_recheck import _values, recheck

SHAPE = KaraShape("dump_bf16", 401, num_seqs=2, num_layers=2, num_q_heads=4, num_kv_heads=2, head_dim=64,
                  window=40, budget=12, seeds=2, radius=2, prior=("uniform", 3, 30), block_size=8)
UNITS = [(0, 0, 0), (1, 1, 1), (1, 0, 1)]


def _bits_of(t):
    return t.view(torch.int16).numpy() if t.dtype == torch.bfloat16 else t.view(torch.int32).numpy()


def _oracle_step(wl, cfg):
    """The step on the host with the oracle: scores rounded to fp32 (as the
    GPU writes them), selection and compaction from those scores."""
    s = wl.shape
    qv = _values(_bits_of(wl.q), cfg.dtype)
    kv = _values(_bits_of(wl.k_pool), cfg.dtype)
    sc = np.zeros((s.num_seqs, s.num_layers, s.num_kv_heads, s.window))
    for n in range(s.num_seqs):
        for layer in range(s.num_layers):
            for g in range(s.num_kv_heads):
                G = s.group
                qg = np.transpose(qv[n, layer, :, g * G:(g + 1) * G, :], (1, 0, 2))
                kw = oracle.gather_window_rows(kv, wl.host_tables[n], layer, g, int(wl.host_prior_lens[n]),
                                               s.window, s.block_size)
                sc[n, layer, g] = oracle.window_scores(qg, kw)
    sc = sc.astype(np.float32).astype(np.float64)
    o = oracle.compress_step(np.zeros((s.num_seqs, s.num_layers, s.window, s.num_q_heads, 1)),
                             _bits_of(wl.k_pool), _bits_of(wl.v_pool), wl.host_tables, wl.host_prior_lens,
                             window=s.window, budget=s.budget, seeds=s.seeds, radius=s.radius,
                             block_size=s.block_size, scores_override=sc)
    mf = (s.window + s.block_size - 1) // s.block_size + 1
    freed = torch.full((s.num_seqs, mf), -1, dtype=torch.int32)
    for n, fr in enumerate(o["freed"]):
        freed[n, :fr.size] = torch.from_numpy(fr.astype(np.int32))
    return dict(k=torch.from_numpy(o["k_pool"]).view(torch.bfloat16), v=torch.from_numpy(o["v_pool"]).view(torch.bfloat16),
                tables=torch.from_numpy(o["block_tables"].astype(np.int32)),
                seq_lens=torch.from_numpy(o["seq_lens"].astype(np.int32)),
                scores=torch.from_numpy(o["scores"].astype(np.float32)),
                kept=torch.from_numpy(o["kept"].astype(np.int32)), freed=freed,
                num_freed=torch.from_numpy(o["num_freed"].astype(np.int32)))


def _record(tmp_path, wl, cfg, step, unit):
    n, layer, g = unit
    before = unit_inputs(cfg, wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, n, layer, g)
    r = step()
    after = unit_outputs(cfg, r["k"], r["v"], r["tables"], r["seq_lens"], r["scores"], r["kept"], r["freed"],
                         r["num_freed"], n, layer, g, before["prior_len"])
    path = str(tmp_path / f"unit_{n}_{layer}_{g}.npz")
    save_unit(path, cfg, before, after, unit)
    return path


@pytest.mark.parametrize("unit", UNITS)
def test_record_of_a_correct_step_rechecks_clean(tmp_path, unit):
    wl = make_workload(SHAPE, "cpu")
    cfg = config_of(wl)
    path = _record(tmp_path, wl, cfg, lambda: _oracle_step(wl, cfg), unit)
    meta, ins, outs = load_unit(path)
    assert meta["unit"] == list(unit) and meta["window"] == SHAPE.window
    assert ins["k_window"].dtype == np.int16 and outs["k_kept"].shape == (SHAPE.budget, SHAPE.head_dim)
    assert recheck(path) == []


def _mutate(path, out_path, **changes):
    meta, ins, outs = load_unit(path)

    class C:
        pass
    cfg = C()
    for k, v in meta.items():
        setattr(cfg, k, v)
    for key, fn in changes.items():
        side, name = key.split("__")
        d = ins if side == "in" else outs
        d[name] = fn(np.array(d[name], copy=True))
    save_unit(out_path, cfg, ins, outs, tuple(meta["unit"]))
    return out_path


def _flip(a, i=0):
    a.reshape(-1)[i] ^= 1
    return a


def test_every_kind_of_wrong_output_is_caught(tmp_path):
    wl = make_workload(SHAPE, "cpu")
    cfg = config_of(wl)
    path = _record(tmp_path, wl, cfg, lambda: _oracle_step(wl, cfg), (1, 1, 1))
    assert recheck(path) == []

    def other_kept(k):
        k = k.copy()
        missing = sorted(set(range(SHAPE.window)) - set(k.tolist()))
        k[-1] = missing[-1]
        return np.sort(k)

    cases = {
        "scores": dict(out__scores=lambda a: a * np.float32(1.01)),
        "kept": dict(out__kept=other_kept),
        "k_kept": dict(out__k_kept=lambda a: _flip(a, 5)),
        "v_kept": dict(out__v_kept=lambda a: _flip(a, 77)),
        "table": dict(out__table_after=lambda a: np.roll(a, 1)),
        "freed": dict(out__freed=lambda a: a[::-1] if a.size > 1 else np.array([12345], np.int32)),
        "seq_len": dict(out__seq_len=lambda a: a + 1),
    }
    for want, ch in cases.items():
        bad = _mutate(path, str(tmp_path / f"bad_{want}.npz"), **ch)
        assert want in recheck(bad), want
    # a window whose first block starts below L keeps those bytes; changing them is caught
    meta, ins, outs = load_unit(path)
    if ins["k_head"].size:
        bad = _mutate(path, str(tmp_path / "bad_head.npz"), out__k_head_after=lambda a: _flip(a, 0))
        assert "k_head" in recheck(bad)


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [
    SHAPE,
    KaraShape("dump_fused", 402, num_seqs=2, num_layers=2, num_q_heads=8, num_kv_heads=2, head_dim=128,
              window=256, budget=51, seeds=3, radius=3, prior=("uniform", 5, 90), plants=True),
    KaraShape("dump_two_pass_f32", 403, num_seqs=1, num_layers=1, num_q_heads=4, num_kv_heads=1, head_dim=128,
              window=300, budget=60, seeds=2, radius=4, prior=("fixed", 21), dtype="f32", block_size=32),
], ids=lambda s: s.name)
def test_records_of_gpu_steps_recheck_clean(tmp_path, shape):
    from tests.kara_harness import run_step
    print(f"[dump] {shape.name}", flush=True)
    wl = make_workload(shape, "cuda")
    cfg = config_of(wl)
    units = [(0, 0, 0), (shape.num_seqs - 1, shape.num_layers - 1, shape.num_kv_heads - 1)]
    befores = [unit_inputs(cfg, wl.q, wl.k_pool, wl.v_pool, wl.block_tables, wl.prior_lens, *u) for u in units]
    _, out = run_step(wl, cfg)
    torch.cuda.synchronize()
    for u, before in zip(units, befores):
        after = unit_outputs(cfg, wl.k_pool, wl.v_pool, wl.block_tables, out["seq_lens"], out["scores"],
                             out["kept"], out["freed"], out["num_freed"], *u, before["prior_len"])
        path = str(tmp_path / f"{shape.name}_{u[0]}_{u[1]}_{u[2]}.npz")
        save_unit(path, cfg, before, after, u)
        assert recheck(path) == [], (shape.name, u)
