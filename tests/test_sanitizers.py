"""The CPU suite under AddressSanitizer and UndefinedBehaviorSanitizer: the host code of the
library (argument validation, tile selection, the tile-table parser) and the oracle are built
with -fsanitize=address,undefined and the rest of this suite runs against them in a child
process that preloads the sanitizer runtime. Any sanitizer report fails the test (reports go
to a log file, since the sanitizers stop the child at the first one)."""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(HERE)


def test_cpu_suite_under_asan_and_ubsan(tmp_path):
    from block_scaled_w8a8_amd import build
    import oracle
    lib = build.build_sanitized()
    orc = oracle.build_sanitized()
    runtime = build.sanitizer_runtime()
    log = str(tmp_path / "sanitizer")
    env = dict(os.environ)
    env["LD_PRELOAD"] = runtime + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = f"detect_leaks=0:log_path={log}"
    env["UBSAN_OPTIONS"] = f"print_stacktrace=1:log_path={log}"
    env["BFQ_LIBRARY"] = lib
    env["BFQ_TILE_TABLE"] = build.TABLE_PATH      # the library is not beside the package
    env["ORACLE_LIBRARY"] = orc
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p",
                        "no:cacheprovider", "--ignore", os.path.join(HERE, "test_sanitizers.py"),
                        HERE], cwd=REPO, env=env, capture_output=True, text=True, timeout=1200)
    reports = "".join(open(f).read() for f in glob.glob(log + "*"))
    assert not reports, reports[:4000]
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert " passed" in r.stdout
