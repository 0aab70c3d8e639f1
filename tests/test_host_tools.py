"""Host-side tooling: bench refuses more than one GPU, kernel-name demangling
and the rocprofv3 CSV summaries used for the traffic figures; the binding
fails loudly without its library and never passes host tensors on."""
import json
import os
import subprocess
import sys

import pytest

from decode_kv_cache_amd import profiling
from tests.conftest import ROOT


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_kernel_names_are_demangled():
    f = profiling.short_name
    assert f("_ZN4kara18decode_attn_kernelIDF16bLi128ELi4EEEvNS_7AttnGeoEPKT_") == "decode_attn_kernel<__bf16, 128, 4>"
    assert f("_ZN4kara15pipeline_kernelENS_3GeoEPKDF16bPh") == "pipeline_kernel"
    assert f("void kara::fused_score_kernel(kara::Geo, __bf16 const*)") == "fused_score_kernel"
    assert f("compact_kernel<256>") == "compact_kernel<256>"


def _csv(path, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for r in rows:
            f.write(",".join(str(x) for x in r) + "\n")


def test_traffic_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    for d in ("f", "w", "cf", "cw"):
        (tmp_path / d).mkdir()
    # two dispatches of the scorer, each split over two counter rows
    _csv(tmp_path / "f" / "run_counter_collection.csv",
         [(1, "void kara::fused_score_kernel(kara::Geo)", "FETCH_SIZE", 300), (1, "void kara::fused_score_kernel(kara::Geo)", "FETCH_SIZE", 200),
          (2, "void kara::fused_score_kernel(kara::Geo)", "FETCH_SIZE", 500)])
    _csv(tmp_path / "w" / "run_counter_collection.csv",
         [(1, "void kara::fused_score_kernel(kara::Geo)", "WRITE_SIZE", 10), (2, "void kara::fused_score_kernel(kara::Geo)", "WRITE_SIZE", 30)])
    _csv(tmp_path / "cf" / "run_counter_collection.csv", [(1, "at::native::neg_kernel", "FETCH_SIZE", 1024)])
    _csv(tmp_path / "cw" / "run_counter_collection.csv", [(1, "at::native::neg_kernel", "WRITE_SIZE", 2048)])
    assert profiling.counter_means(str(tmp_path / "f"), "FETCH_SIZE") == {"fused_score_kernel": 500.0}
    monkeypatch.setattr(profiling, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    (tmp_path / "decode_kv_cache_amd" / "csrc").mkdir(parents=True)
    (tmp_path / "decode_kv_cache_amd" / "csrc" / "k.hip").write_text("x")
    profiling.main(["traffic", "--workload", "w", "--fetch", str(tmp_path / "f"), "--write", str(tmp_path / "w"),
                    "--copy-fetch", str(tmp_path / "cf"), "--copy-write", str(tmp_path / "cw"), "--copy-mib", "2"])
    rec = json.loads((tmp_path / "profiles" / "traffic.json").read_text())["w"]
    # copy of 2 MiB = 2048 KiB: FETCH reads 0.5x, WRITE 1.0x
    assert abs(rec["copy_factor_fetch"] - 0.5) < 1e-12 and abs(rec["copy_factor_write"] - 1.0) < 1e-12
    k = rec["kernels"]["fused_score_kernel"]
    assert k["fetch_bytes"] == 500 * 1024 / 0.5 and k["write_bytes"] == 20 * 1024
    assert rec["score_bytes_per_launch"] == k["bytes"]


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """No fallback: with libkara.so absent every entry point raises."""
    from decode_kv_cache_amd import kara as K
    monkeypatch.setattr(K, "_LIB_PATH", str(tmp_path / "libkara.so"))
    monkeypatch.setattr(K, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        K.lib()
    with pytest.raises(RuntimeError, match="missing"):
        K.kara_check_config(K.kara_config())


def test_binding_rejects_host_tensors():
    """Device pointers only: a CPU tensor never reaches the library."""
    import torch

    from decode_kv_cache_amd import kara as K
    from decode_kv_cache_amd.workloads import shape_by_name
    s = shape_by_name("tiny")
    cfg = K.make_config(s, max_blocks_per_seq=32, num_blocks=64)
    scores = torch.zeros((s.num_seqs, s.num_layers, s.num_kv_heads, s.window), dtype=torch.float32)
    kept = torch.zeros((s.num_seqs, s.num_layers, s.num_kv_heads, s.budget), dtype=torch.int32)
    with pytest.raises(ValueError, match="device"):
        K.kara_select_chunks(cfg, scores, kept)


def test_kernel_hash_sees_code_not_comments():
    """Stored traffic measurements stay valid across comment edits and go
    stale on any code edit; the host-only ABI layer and the probes do not
    count."""
    from decode_kv_cache_amd.profiling import code_only, kernel_source_hash

    base = {"a.hip": 'int f() { return 1; } // one\n', "b.h": "/* x */ #define S \"// kept\"\n",
            "api.hip": "int g();", "probes.hip": "int p();"}

    def reader(files):
        return lambda f: list(files) if f is None else files[f]

    h0 = kernel_source_hash(reader(base))
    assert kernel_source_hash(reader(dict(base, **{"a.hip": "int f() {\n  return 1;  /* same */ }\n"}))) == h0
    assert kernel_source_hash(reader(dict(base, **{"api.hip": "int g(int);", "probes.hip": ""}))) == h0
    assert kernel_source_hash(reader(dict(base, **{"a.hip": "int f() { return 2; }"}))) != h0
    assert kernel_source_hash(reader(dict(base, **{"b.h": '#define S "// changed"'}))) != h0
    assert code_only('x = "a//b"; // c\ny') == 'x = "a//b"; y'
