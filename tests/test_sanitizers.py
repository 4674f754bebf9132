"""CPU sanitizer tier: the fp64 oracle (gcc) and the C-ABI layer's host code (hipcc, host
side only) rebuilt with AddressSanitizer and UndefinedBehaviorSanitizer, then exercised in
a subprocess with the sanitizer runtime preloaded: every oracle pin, and the ABI layer's
validation paths (shapes, pointers, workspace sizes, the empty calls; nothing reaches a
GPU). Any report aborts the subprocess and fails the test."""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN_ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
           "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"}


def _run(code, preload, tmp_path, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, PYTHONPATH=os.pathsep.join([ROOT, TESTS]),
               **SAN_ENV)
    script = tmp_path / "run.py"
    script.write_text(textwrap.dedent(code))
    r = subprocess.run([sys.executable, str(script)], env=env, capture_output=True, text=True,
                       timeout=timeout, cwd=str(tmp_path))
    assert r.returncode == 0 and "ERROR: AddressSanitizer" not in r.stderr \
        and "runtime error" not in r.stderr, (r.stdout[-3000:], r.stderr[-6000:])
    return r


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(p) or not os.path.exists(p):
        pytest.skip(f"{name} not available")
    return p


def test_oracle_pins_under_asan_ubsan(tmp_path):
    import oracle
    lib = str(tmp_path / "libmsa_oracle_san.so")
    oracle.build(out=lib, extra_flags=["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                                       "-fno-omit-frame-pointer", "-g"])
    r = _run(f"""
        import oracle, oracle_pins
        orc = oracle.Oracle({lib!r})
        for pin in oracle_pins.PINS:
            pin(orc)
            print("ok", pin.__name__, flush=True)
        """, _gcc_runtime("libasan.so"), tmp_path)
    assert r.stdout.count("ok ") >= 19


def _clang_asan_runtime():
    out = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        if not hits:
            pytest.skip("clang AddressSanitizer runtime not available")
        out = hits[0]
    return out


def test_abi_validation_under_asan_ubsan(tmp_path):
    """libmsa.so with msa_api.cpp's host code instrumented (the kernels' objects as built),
    driven through every validation path the CPU ABI tests take."""
    from block_sparse_gqa_msa_amd import build as hb
    objs = [os.path.join(hb.BUILD, s + ".o") for s in hb.SOURCES if s != "msa_api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        hb.build(verbose=False)
    api_obj = str(tmp_path / "msa_api_san.o")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    flags = [f for f in hb.FLAGS if f != "-O3"] + ["-O1", "-g"]
    r = subprocess.run([HIPCC, *flags, *san, "-x", "hip", "-c",
                        os.path.join(hb.CSRC, "msa_api.cpp"), "-o", api_obj],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = str(tmp_path / "libmsa_san.so")
    r = subprocess.run([HIPCC, f"--offload-arch={hb.ARCH}", "-shared", "-fPIC", *san, api_obj, *objs,
                        "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    _run(f"""
        import sys, types, pytest
        from block_sparse_gqa_msa_amd import binding as msa
        lib = msa.load_library({lib!r})
        import test_abi
        names = [n for n in dir(test_abi) if n.startswith("test_") and "missing_library" not in n]
        ran = 0
        for n in names:
            fn = getattr(test_abi, n)
            marks = getattr(fn, "pytestmark", [])
            params = [m for m in marks if m.name == "parametrize"]
            import inspect
            argn = list(inspect.signature(fn).parameters)
            if params:
                pnames = [a.strip() for a in params[0].args[0].split(",")]
                for vals in params[0].args[1]:
                    vals = vals if isinstance(vals, tuple) else (vals,)
                    kw = dict(zip(pnames, vals))
                    if "lib" in argn:
                        kw["lib"] = lib
                    fn(**kw)
                    ran += 1
            else:
                fn(**({{"lib": lib}} if "lib" in argn else {{}}))
                ran += 1
        print("ran", ran, flush=True)
        """, _clang_asan_runtime(), tmp_path)
