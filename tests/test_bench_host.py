"""Host-side pieces of bench.py (no GPU): the source hash that ties stored
counter summaries to the kernels they were taken on, and the one-GPU limit."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_strip_c_comments_keeps_code_and_literals():
    src = ('int a = 1; // line\n/* block\n comment */ const char* s = "x//y/*z*/";\n'
           "char q = '\"'; int b/*in*/=2;\n  float c = a /b;\n")
    got = bench._strip_c_comments(src)
    assert got == "int a = 1; const char* s = \"x//y/*z*/\"; char q = '\"'; int b =2; float c = a /b;"


def test_strip_c_comments_escaped_quote():
    src = 'const char* s = "a\\"//b"; // gone\nint x;'
    assert bench._strip_c_comments(src) == 'const char* s = "a\\"//b"; int x;'


def test_sources_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    f = tmp_path / "k.hip"
    f.write_text("__global__ void k(int* p) { p[0] = 1; }\n")
    h0 = bench.sources_hash(["k.hip"])
    f.write_text("// a kernel\n__global__ void k(int* p) {\n  p[0] = 1;  /* store */\n}\n")
    assert bench.sources_hash(["k.hip"]) == h0
    f.write_text("__global__ void k(int* p) { p[0] = 2; }\n")
    assert bench.sources_hash(["k.hip"]) != h0


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


@pytest.mark.parametrize("name, short, call", [
    ("void losa::(anonymous namespace)::attn_bf16_kernel<128, false>(losa::Geom, ...)",
     "attn_bf16_kernel", "losa_sparse_attn"),
    ("void losa::(anonymous namespace)::attn_bf16_kernel<128, true>(losa::Geom, ...)",
     "attn_bf16_kernel (in-pass thresholding)", "losa_sparse_attn_threshold"),
    ("_ZN4losa12_GLOBAL__N_116attn_bf16_kernelILi64ELb1EEEvNS_4GeomE",
     "attn_bf16_kernel (in-pass thresholding)", "losa_sparse_attn_threshold"),
    ("_ZN4losa14pack_kv_kernelILi128ELb0EEEvNS_4GeomEPKDF16bS3_PDF16bS4_i",
     "pack_kv_kernel (K only)", "losa_block_mass"),
    ("void losa::(anonymous namespace)::dense_bf16_kernel<128, true>(losa::Geom, ...)",
     "dense_bf16_kernel (lists)", "losa_sparse_attn_mass"),
    ("void losa::(anonymous namespace)::dense_bf16_kernel<128, false>(losa::Geom, ...)",
     "dense_bf16_kernel", "losa_dense_attn_mass"),
    ("_ZN4losa12_GLOBAL__N_111pool_kernelIDF16bLi128EdEEvNS_4GeomEPKT_llliiPT1_",
     "pool_kernel (fp64 block means)", "losa_sparse_attn_threshold"),
    ("_ZN4losa12_GLOBAL__N_111pool_kernelIDF16bLi128EfEEvNS_4GeomEPKT_llliiPT1_",
     "pool_kernel", "losa_pooled_mass"),
    ("void losa::(anonymous namespace)::threshold_kernel<true>(losa::Geom, ...)",
     "threshold_kernel (indices)", "losa_select_threshold"),
])
def test_trace_kernel_names_map_to_their_calls(name, short, call):
    assert bench.kernel_label(name, bench.TRACE_KERNELS) == (short, call)


def test_clock_kernels_skip_the_in_pass_instance():
    assert bench.kernel_label("attn_bf16_kernel<128, true>(...)", bench.CLOCK_KERNELS) is None
    assert bench.kernel_label("attn_bf16_kernel<128, false>(...)", bench.CLOCK_KERNELS)[0] == "attn_bf16_kernel"
