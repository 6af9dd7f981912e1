"""Host logic of bench.py that needs no GPU: the code hash that keys the
committed counter entries, and the layout of those entries."""
import hashlib
import json
import os

import bench
from synth import CONFIGS


def test_code_only_drops_comments_and_layout():
    src = ("int a = 1;  // trailing comment\n"
           "/* block\n   comment */ int   b =\n 2;\n"
           "// whole-line comment\n")
    assert bench._code_only(src) == "int a = 1; int b = 2;"


def test_code_only_keeps_literals_that_look_like_comments():
    src = 'const char* s = "x // y /* z */"; char q = \'"\'; char r = \'\\\'\'; // gone'
    assert bench._code_only(src) == 'const char* s = "x // y /* z */"; char q = \'"\'; char r = \'\\\'\';'


def test_code_hash_ignores_comment_edits_but_not_code_edits():
    base = "__global__ void k(int* p) { p[0] = 1; }\n"
    commented = "// a kernel\n__global__ void k(int* p) {  /* store */ p[0] = 1;  }\n"
    changed = "__global__ void k(int* p) { p[0] = 2; }\n"
    h = lambda t: hashlib.sha256(bench._code_only(t).encode()).hexdigest()
    assert h(base) == h(commented)
    assert h(base) != h(changed)


def test_traffic_entries_name_known_workloads_and_kernels():
    entries = json.load(open(bench.TRAFFIC_FILE))
    for workload, kernels in entries.items():
        assert workload == bench.ATTN_WORKLOAD or workload in CONFIGS
        T = 4096 if workload == bench.ATTN_WORKLOAD else CONFIGS[workload].T
        for kernel, e in kernels.items():
            src = bench.kernel_source(kernel, T)
            assert os.path.exists(os.path.join(bench.ROOT, "sparse_mixture_experts_wave_amd", "csrc", src))
            # each scaled count is rounded on its own
            assert abs(e["bytes_per_launch"] - (e["read_bytes"] + e["write_bytes"])) <= 1
            assert e["bytes_per_launch"] > 0
            assert len(e["src_sha"]) == 16
