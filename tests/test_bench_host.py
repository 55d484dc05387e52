"""Host-side logic of bench.py (no GPU): the algorithmic byte counts behind
roofline.achieved, the source hash that decides whether the committed HBM
traffic figures still describe the kernels, and the one-GPU guard.

The byte counts are pinned to the per-workload figures derived from the
problem statement (rl-triton, Problem: rewards, values with the bootstrap
column, done flags and the outputs, each read or written once): GAE 18 B per
fp32 env-step plus the bootstrap column, and so on.
"""
import hashlib
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from reverse_linear_recurrence_amd.synth import WORKLOADS  # noqa: E402


@pytest.mark.parametrize("name,expected", [
    # r 4 + V 4 + term 1 + trunc 1 + advantages 4 + targets 4 per step, V_T per row
    ("gae_4096x128", 18 * 4096 * 128 + 4 * 4096),
    # r 4 + V 4 + term 1 + G 4 per step (no truncation flags), V_T per row
    ("td_lambda_16384x256", 13 * 16384 * 256 + 4 * 16384),
    # V-trace: r, V, log_rho 12 + term 1 + vs, pg 8 per step, V_T per row;
    # Retrace: r, Q, EQ, log_rho 16 + term 1 + Q_ret 4 per step
    ("offpolicy_2048x1024", 21 * 2048 * 1024 + 4 * 2048 + 21 * 2048 * 1024),
    # bf16 r 2 + V 2 + 2 flags + fp32 outputs 8 per step, V_T per row
    ("gae_bf16_256x16384", 14 * 256 * 16384 + 2 * 256),
    # x 4 + 2 flags + output 4 per step
    ("eligibility_4096x128", 10 * 4096 * 128),
])
def test_algorithmic_bytes(name, expected):
    w = WORKLOADS[name]
    assert bench.algorithmic_bytes(w, w.num_envs, w.T) == expected


@pytest.mark.parametrize("name", [n for n in WORKLOADS if bench.stream_mixes(WORKLOADS[n])])
def test_stream_ceiling_moves_the_per_step_algorithmic_bytes(name):
    """The streaming-ceiling leg moves, per step, exactly the algorithmic
    bytes of every env-step (all but the per-row bootstrap terms)."""
    w = WORKLOADS[name]
    per_step = sum(4 * nf + 2 * nh + nb + 4 * no for nf, nh, nb, no in bench.stream_mixes(w))
    per_row = bench.algorithmic_bytes(w, w.num_envs, 0)
    assert per_step * w.num_envs * w.T == bench.algorithmic_bytes(w, w.num_envs, w.T) - per_row


def test_stream_ceiling_has_a_mix_for_every_scan_workload():
    for name, w in WORKLOADS.items():
        assert (bench.stream_mixes(w) is None) == w.algo.endswith("_probs"), name


def test_window_bytes_add_the_carry_vectors():
    w = WORKLOADS["gae_4096x128"]
    plain = bench.algorithmic_bytes(w, w.num_envs, w.T)
    assert bench.algorithmic_bytes(w, w.num_envs, w.T, window=True) == plain + 16 * w.num_envs


def test_code_text_ignores_comments_and_layout():
    a = "int f(int x) {  // doubles\n  return 2 * x; /* twice */\n}\n"
    b = "int f(int x) {\n    return 2 * x;\n}  // edited comment\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
    assert "doubles" not in bench.code_text(a) and "twice" not in bench.code_text(a)


def test_kernel_source_hash_covers_every_listed_file():
    for family, files in bench.KERNEL_SOURCES.items():
        h = hashlib.sha256()
        for f in files:
            with open(os.path.join(bench._CSRC, f), encoding="utf-8") as fh:
                h.update(bench.code_text(fh.read()).encode())
        assert bench.kernel_source_hash(family) == h.hexdigest()[:16]


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_host_threads_is_bounded_by_affinity_and_one_gpu_share():
    n = bench.host_threads()
    assert 1 <= n <= 16
    assert n <= len(os.sched_getaffinity(0))


def test_cpu_model_is_text_or_absent():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)


def test_traffic_keys_name_the_entry_point_and_split_form():
    assert bench.traffic_key("gae_4096x128") == "gae_4096x128"
    assert bench.traffic_key("gae_4096x128", window=True) == "gae_4096x128/window"
    assert bench.traffic_key("gae_4096x128", materialized=True) == "gae_4096x128/materialized"
    w = "gae_bf16_16x262144"
    assert bench.traffic_key(w, split_form="chained") == w + "/chained"
    assert bench.traffic_key(w, split_form="three-launch") == w + "/three-launch"
    assert bench.traffic_key(w, split_form="unsplit") == w
    # every committed entry is keyed by a workload and a form bench.py produces
    forms = {bench.traffic_key(n, win, mat, s) for n in WORKLOADS for win in (False, True)
             for mat in (False, True) for s in (None, "chained", "three-launch")}
    with open(bench.TRAFFIC_FILE) as f:
        committed = json.load(f)
    assert committed and set(committed) <= forms
