"""Host logic of bench.py (no GPU): the kernel-source hash that ties a
committed HBM-traffic measurement to the code it was taken with, and the
reading of those summaries."""
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_only_drops_comments_keeps_literals():
    src = ('int a = 1; // one\n/* two\n lines */ const char* s = "x // y /* z */";\n'
           "char q = '/'; char r = '\\''; int b;  /* tail */\n")
    assert bench._code_only(src) == ('int a = 1; const char* s = "x // y /* z */"; '
                                     "char q = '/'; char r = '\\''; int b;")


def test_hash_follows_code_not_comments(tmp_path, monkeypatch):
    csrc = tmp_path / "mixture_experts_layer_10_amd" / "csrc"
    csrc.mkdir(parents=True)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", {"x": ["k.hip"]})
    (csrc / "k.hip").write_text("// v1\n__global__ void k() { int a = 1; }\n")
    h1 = bench.kernel_source_hash("x")
    (csrc / "k.hip").write_text("/* reworded */\n__global__ void k() {\n    int a = 1;   // same code\n}\n")
    assert bench.kernel_source_hash("x") == h1
    (csrc / "k.hip").write_text("__global__ void k() { int a = 2; }\n")
    assert bench.kernel_source_hash("x") != h1


@pytest.mark.parametrize("workload,dtype", [("full_prefill_bf16", "bf16"), ("full_decode_bf16", "bf16"),
                                            ("ep8_decode_bf16", "bf16"), ("fp8_skew", "fp8"),
                                            ("full_decode_mxfp4", "mxfp4")])
def test_committed_traffic_matches_current_kernels(workload, dtype):
    """Every committed traffic summary was taken with the kernels as they are
    (else bench.py would report traffic as null)."""
    assert os.path.exists(os.path.join(ROOT, "profiles", f"gate_up_{workload}_hbm_traffic.md"))
    t = bench.stored_traffic("gate_up", workload, dtype)
    assert t is not None and t > 0
