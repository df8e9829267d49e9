"""The C ABI's host-side argument checks under AddressSanitizer and UndefinedBehaviorSanitizer.

Every source of the library is compiled for the host only (no device code) with both sanitizers
on the host code and aborting on the first report, linked into a shared library of its own with
a stand-in for the HIP runtime that has no device (`tests/sanitize/hip_stub.cpp`: nothing built
here can reach a GPU), and driven by `tests/sanitize/host_validation.cpp`: each entry point with
invalid, extreme (INT_MIN, INT_MAX, sizes at and beyond the documented limits) and valid
arguments, each status compared with the header's.  Valid calls get as far as their launches;
the stand-in checks each launch shape and fails it (OSCAR_ERR_HIP).  CPU only.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "int2_rotated_kv_rotate_amd", "csrc")
DRIVER = os.path.join(ROOT, "tests", "sanitize", "host_validation.cpp")
STUB = os.path.join(ROOT, "tests", "sanitize", "hip_stub.cpp")
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang++"

# host code only: each -fsanitize= applies to the host compilation
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANG)), reason="no ROCm toolchain")
def test_host_validation_under_asan_and_ubsan(tmp_path):
    sys.path.insert(0, ROOT)
    from int2_rotated_kv_rotate_amd.build import SOURCES

    def compile_one(item):
        src, extra = item
        obj = str(tmp_path / src.replace(".hip", ".o"))
        # device-only options (e.g. code-generation flags for gfx950) do not apply here
        host_extra = [f for f in extra if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form")]
        _run([HIPCC, "--offload-host-only", "-O1", "-g", "-fno-omit-frame-pointer", "-fPIC",
              "-std=c++17", *host_extra, *HOST_SANITIZE, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(compile_one, SOURCES.items()))
    # the per-file fat-binary symbols the host objects refer to (never read: the stand-in
    # runtime registers nothing)
    nm = _run(["nm", "-u", *objs]).stdout
    fatbins = sorted({ln.split()[-1] for ln in nm.splitlines() if "__hip_fatbin_" in ln})
    gen = tmp_path / "fatbins.cpp"
    gen.write_text("".join(f'extern "C" const unsigned char {n}[1] = {{0}};\n' for n in fatbins))
    stub_objs = []
    for src in (STUB, str(gen)):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        _run([CLANG, "-c", "-fPIC", "-O1", "-g", "-std=c++17", "-D__HIP_PLATFORM_AMD__",
              "-I/opt/rocm/include", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              src, "-o", obj])
        stub_objs.append(obj)
    lib = str(tmp_path / "liboscar_host_san.so")
    _run([CLANG, "-shared", "-o", lib, *objs, *stub_objs])
    exe = str(tmp_path / "host_validation")
    _run([CLANG, "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g", "-O1",
          "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", DRIVER, "-o", exe,
          f"-L{tmp_path}", "-loscar_host_san", f"-Wl,-rpath,{tmp_path}"])

    env = dict(os.environ)
    env.update(ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    assert " 0 failed" in r.stdout, out[-4000:]
    print(r.stdout.strip())
