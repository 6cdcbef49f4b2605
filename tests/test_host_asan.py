"""The library's host code under AddressSanitizer (CPU only, nothing is launched).

Every library source is compiled with AddressSanitizer on its host side (device code as
in the normal build) and linked with tests/asan/abi_driver.cpp into one executable. The
driver calls every C entry point on paths that end before any launch, and checks each
status and error message. A heap or stack error in the argument checks, the error
strings or the table and descriptor handling stops the run with a sanitizer report.
The driver also enumerates the grouped GEMMs' tile order inside an expert (compiled for
the host) and checks that it maps every expert shape one to one onto its tiles.
The build sits in grouped_expert_gemm_amd/_build_asan/; it is redone when a source,
header or the driver is newer than the executable (about 40 s on 8 cores)."""
import glob
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "grouped_expert_gemm_amd", "_build_asan")
DRIVER = os.path.join(ROOT, "tests", "asan", "abi_driver.cpp")
EXE = os.path.join(OUT, "abi_asan")
# host-side only: each sanitizer flag goes to the host compilation
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-2000:]}\n{r.stderr[-4000:]}"


def _build():
    from grouped_expert_gemm_amd import build as b
    srcs = sorted(glob.glob(os.path.join(b.CSRC, "*.hip")))
    deps = srcs + glob.glob(os.path.join(b.CSRC, "*.h")) + glob.glob(os.path.join(b.INCLUDE, "*.h")) + [DRIVER]
    if os.path.exists(EXE) and all(os.path.getmtime(p) <= os.path.getmtime(EXE) for p in deps):
        return
    os.makedirs(OUT, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(OUT, os.path.basename(src) + ".o")
        _run([b.HIPCC, *b.CFLAGS, *SAN, "-c", src, "-o", obj])
        return obj

    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, srcs))
    drv = os.path.join(OUT, "abi_driver.o")
    _run([b.HIPCC, f"--offload-arch={b.ARCH}", "-x", "hip", "-O1", "-std=c++17", "-I", b.INCLUDE, "-I", b.CSRC, *SAN,
          "-c", DRIVER, "-o", drv])
    _run([b.HIPCC, f"--offload-arch={b.ARCH}", *SAN, "-o", EXE + ".tmp", drv, *objs])
    os.replace(EXE + ".tmp", EXE)


def test_entry_points_under_address_sanitizer():
    _build()
    env = dict(os.environ)
    # the HIP runtime's own allocations outlive main(): leak reports are not this test's subject
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    r = subprocess.run([EXE], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-6000:]
    assert r.returncode == 0, out[-6000:]
    assert "ok: 0 failure(s)" in r.stdout, out[-3000:]


def test_executable_is_instrumented():
    """The check means something only if the sanitizer runtime is in the executable."""
    _build()
    r = subprocess.run(["nm", "-C", EXE], capture_output=True, text=True)
    assert "__asan_init" in r.stdout or "__asan_report_load" in r.stdout
