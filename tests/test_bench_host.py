"""Host-side logic of bench.py that needs no GPU: the one-GPU contract, argument checks
that stop a run before it starts, and the source hash that decides whether the committed
counter summary still describes the kernels."""
import importlib.util
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line for a configuration that was not measured


def test_backward_refuses_other_chunk_sizes():
    r = _run("--backward", "--chunk", "128")
    assert r.returncode == 2
    assert "C = 64" in r.stderr
    assert r.stdout.strip() == ""


def test_source_hash_covers_the_headline_kernels_and_their_headers():
    # every local header the forward kernels' translation unit includes (transitively) is part
    # of the key, so no change to the headline kernels leaves the committed figures in use;
    # the backward header, included at the end of that unit, holds only the backward kernels
    bench = _load_bench()
    csrc = os.path.join(ROOT, "chunkwise_gated_delta_amd", "csrc")
    seen, todo = set(), ["gdr_kda_split.hip"]
    while todo:
        name = todo.pop()
        if name in seen:
            continue
        seen.add(name)
        with open(os.path.join(csrc, name)) as f:
            todo += re.findall(r'^#include "([^"/]+)"', f.read(), re.M)
    keyed = {os.path.basename(rel) for rel in bench.KERNEL_SOURCES}
    assert seen - {"gdr_kda_bwd.h"} <= keyed
    # the compiler flags shape the code, so the build script is part of the key too
    assert "build.py" in keyed


def test_counter_figures_only_for_the_sources_they_were_taken_on():
    bench = _load_bench()
    text = open(os.path.join(ROOT, bench.COUNTERS_FILE)).read()
    m = re.search(r"Kernel source sha256 `([0-9a-f]{64})`", text)
    assert m, "the counter summary names the kernel source it was measured on"
    got = bench.committed_counters()
    if m.group(1) == bench.kernel_source_sha():
        assert got["traffic_bytes_per_launch"] > 0 and 0 < got["mfma_busy_frac"] < 1
    else:
        assert got == {}  # stale figures are never reported
