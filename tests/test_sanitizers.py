"""CPU builds under AddressSanitizer and UndefinedBehaviorSanitizer of the C
oracle (oracle/oracle.c), the GPU library's host code (kvq_host.cpp, with
stub HIP calls and kernel launchers that touch every plane's extent) and
the library's group codec (kvq_codec.h, host build).  Each driver
(tests/san_*_main.*) runs its code through the whole API on small inputs;
the pass is exit status 0, its "ok" line and no sanitizer report."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "quantized_decode_attention_keys_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fno-sanitize-recover=all", "-static-libasan",
       "-fsanitize=address,undefined,float-cast-overflow"]
HIP_HOST = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include"]

CASES = {
    "oracle": (["gcc", "-std=c99"], [os.path.join(TESTS, "san_oracle_main.c"),
                                      os.path.join(ROOT, "oracle", "oracle.c"), "-lm"]),
    "host": (["g++", "-std=c++17"] + HIP_HOST + ["-I", os.path.join(ROOT, "include"), "-I", CSRC],
             [os.path.join(TESTS, "san_host_main.cpp"), os.path.join(CSRC, "kvq_host.cpp")]),
    "codec": (["g++", "-std=c++17"] + HIP_HOST + ["-I", CSRC],
              [os.path.join(TESTS, "san_codec_main.cpp")]),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_sanitized_build_runs_clean(name, tmp_path):
    head, srcs = CASES[name]
    exe = str(tmp_path / f"san_{name}")
    subprocess.check_call(head + SAN + srcs[:1] + srcs[1:] + ["-o", exe],
                          stderr=subprocess.DEVNULL)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("KVQ_SYNC", None)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    report = r.stderr[-3000:]
    assert r.returncode == 0, report
    assert r.stdout.startswith("ok"), r.stdout + report
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, report
