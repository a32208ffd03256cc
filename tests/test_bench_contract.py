"""bench.py's contract on the host: one GPU only (--gpus N > 1, or a
multi-rank launch, exits with status 2 and says so before touching a GPU),
and the committed traffic summary is tied to the kernel sources it was
measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench(["--gpus", "2", "--steps", "1"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_a_multi_rank_launch_is_refused():
    r = run_bench(["--steps", "1"], {"WORLD_SIZE": "2", "RANK": "0"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_names_existing_sources():
    with open(os.path.join(ROOT, "profiles", "w8a8_decode_matvec_traffic.json")) as f:
        rec = json.load(f)
    assert rec["sources"] and all(os.path.exists(os.path.join(ROOT, s)) for s in rec["sources"])
    assert len(rec["source_sha256"]) == 64 and rec["traffic_bytes_per_launch"] > 0
    assert all("rocprofv3 --pmc" in c for c in rec["commands"])
