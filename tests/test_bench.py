"""Host-side behaviour of bench.py (no GPU)."""
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_kernel_code_sha_does_not_depend_on_the_checkout_path(tmp_path):
    """roofline.traffic is matched to the device code by this hash; a copy
    of the tree at another path (another machine's checkout) must give the same
    value."""
    for d in ("paged_kv_cache_155_amd", "include"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copy(os.path.join(ROOT, "bench.py"), tmp_path / "bench.py")
    code = "import bench; print(bench.kernel_code_sha())"
    here = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    there = subprocess.run([sys.executable, "-c", code], cwd=tmp_path, capture_output=True,
                           text=True)
    assert here.returncode == 0 and there.returncode == 0, here.stderr + there.stderr
    assert here.stdout.strip() == there.stdout.strip()


def test_committed_traffic_matches_current_code():
    """Every counter entry in profiles/traffic.json was taken on the current
    device code (else bench.py would report roofline.traffic as null)."""
    import json
    sys.path.insert(0, ROOT)
    import bench
    entries = {k: v for k, v in json.load(open(bench.TRAFFIC_JSON)).items()
               if not k.startswith("_")}
    assert entries
    sha = bench.kernel_code_sha()
    stale = [k for k, v in entries.items() if v.get("kernel_code_sha") != sha]
    assert not stale, f"counters taken on other code: {stale}"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
