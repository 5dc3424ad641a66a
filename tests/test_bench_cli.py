"""bench.py's command line on the CPU: more than one GPU is refused with a
message and exit status 2, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ, **(env_extra or {}))
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=env,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_launcher_world_size_is_refused():
    r = _run([], {"WORLD_SIZE": "8"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_forward_source_hash_files_exist():
    # stored HBM counters are keyed by a hash of these files; each must exist
    sys.path.insert(0, ROOT)
    import bench
    from exact_attention_fa2_amd import build
    for name in bench.FWD_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "exact_attention_fa2_amd", name)), name
    assert len(bench.kernel_source_hash()) == 16
    # per-file compiler options name existing sources
    for name in build.EXTRA:
        assert os.path.exists(os.path.join(build.CSRC, name)), name
