"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU needed):
  * the C ABI's argument validation and workspace-size queries: every product source
    compiled as the library is (device code unchanged) with the sanitizers on its host code,
    linked with tests/sanitize/api_checks.cpp, which calls every entry point with bad,
    extreme and empty arguments;
  * the C oracle with tests/sanitize/oracle_checks.c, which runs every oracle function on
    small seeded inputs.
Both programs abort on the first sanitizer report (-fno-sanitize-recover)."""
import os
import subprocess

import pytest

from scale_search_weights_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN_HOST = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
SAN_OPTIONS = {"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0:exitcode=41",
               "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1:exitcode=42"}


def _run(cmd, sanitized=False, threads=None):
    env = None
    if sanitized:
        env = dict(os.environ, **SAN_OPTIONS)
        if threads:
            env["OMP_NUM_THREADS"] = str(threads)
    r = subprocess.run(cmd, capture_output=True, text=True, env=env)
    if r.returncode != 0:
        pytest.fail(f"{os.path.basename(cmd[0])}: exit {r.returncode}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}",
                    pytrace=False)
    return r


def test_c_abi_host_code_under_sanitizers(tmp_path):
    objs = []
    # the library's own flags (device code as built), plus the sanitizers on the host side
    common = [*hip_build.FLAGS, *SAN_HOST, "-Xarch_host", "-g", "-Xarch_host", "-fno-omit-frame-pointer"]
    procs = []
    for src in hip_build.SOURCES:
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        procs.append(subprocess.Popen([hip_build.HIPCC, *common, "-c", os.path.join(hip_build.CSRC, src),
                                       "-o", obj], stdout=subprocess.PIPE, stderr=subprocess.PIPE))
        objs.append(obj)
    drv = str(tmp_path / "api_checks.o")
    procs.append(subprocess.Popen([hip_build.HIPCC, *common, "-c", os.path.join(HERE, "api_checks.cpp"), "-o", drv],
                                  stdout=subprocess.PIPE, stderr=subprocess.PIPE))
    for p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, err.decode()[-3000:]
    exe = str(tmp_path / "api_checks")
    _run([hip_build.HIPCC, *SAN_HOST, drv, *objs, "-o", exe])
    r = _run([exe], sanitized=True)
    assert "api checks passed" in r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off", "-std=c11",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          os.path.join(ROOT, "oracle", "nvfp4_oracle.c"), os.path.join(HERE, "oracle_checks.c"),
          "-o", exe, "-lm"])
    r = _run([exe], sanitized=True, threads=4)
    assert "oracle checks passed" in r.stdout
