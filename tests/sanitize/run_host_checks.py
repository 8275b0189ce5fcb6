"""Host-only sanitizer run of the oracle and of the C ABI's validation.

Builds, with the host compilers (never hipcc) and -fsanitize=address,undefined:
  * the fp64 oracle (oracle/attn_oracle.c, gcc, OpenMP);
  * the C ABI's argument checks (exact_io_aware_40_amd/csrc/attn_api.cpp,
    g++) linked with link-only launcher stand-ins (launch_stubs.cpp),
then runs the oracle's pins and the ABI validation tests against those
builds.  It must be started with the sanitizer runtimes preloaded
(tests/test_sanitizers.py does that); it exits with pytest's status.
"""
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def build(out_dir):
    oracle_lib = os.path.join(out_dir, "liboracle_san.so")
    subprocess.run(["gcc", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra"] + SAN
                   + ["-o", oracle_lib, os.path.join(ROOT, "oracle", "attn_oracle.c"), "-lm"], check=True)
    api_lib = os.path.join(out_dir, "libattn_api_san.so")
    csrc = os.path.join(ROOT, "exact_io_aware_40_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-fPIC", "-shared", "-Wall", "-D__HIP_PLATFORM_AMD__",
                    "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", csrc] + SAN
                   + ["-o", api_lib, os.path.join(csrc, "attn_api.cpp"), os.path.join(HERE, "launch_stubs.cpp")],
                   check=True)
    return oracle_lib, api_lib


def main():
    with tempfile.TemporaryDirectory() as d:
        oracle_lib, api_lib = build(d)
        sys.path.insert(0, ROOT)
        import oracle
        import exact_io_aware_40_amd as attn
        oracle._LIB_PATH = oracle_lib
        attn._LIB_PATH = api_lib
        import pytest
        tests = [os.path.join(ROOT, "tests", f) for f in
                 ("test_oracle.py", "test_oracle_fp8.py", "test_abi_cpu.py")]
        rc = pytest.main(["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider"] + tests)
        print(f"[sanitizer run] oracle {oracle._lib is not None and oracle._LIB_PATH == oracle_lib}, "
              f"api {attn._lib is not None and attn._LIB_PATH == api_lib}", flush=True)
    return int(rc)


if __name__ == "__main__":
    sys.exit(main())
