"""The checked host build of librtp: its sources compiled with AddressSanitizer,
UndefinedBehaviorSanitizer and the planners' bounds assertions (RTP_HOST_CHECKS),
linked with tests/host_check.cpp into one program that replays C-ABI calls and
runs the head-quad planner (see that file for its input format).

Only the host code is instrumented (each sanitizer flag goes to the host pass);
the device code is compiled without optimisation since it never runs here.
The build is cached under _build/host_check, keyed by the sources and flags.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import long_context_sparse_retrieval_amd as rtp
from long_context_sparse_retrieval_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "host_check")
DRIVER = os.path.join(ROOT, "tests", "host_check.cpp")
EXE = os.path.join(OUT, "host_check")
CLANG = "/opt/rocm/llvm/bin/clang++"

SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g", "-Xarch_host", "-O1", "-Xarch_device", "-O0"]
FLAGS = [f"--offload-arch={B.ARCH}", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{B.INCLUDE}", f"-I{B.CSRC}", "-DRTP_HOST_CHECKS", *SANITIZE]
LINK = ["-fsanitize=address,undefined", "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]

# the sanitizers' runtime options: stop at the first report; the HIP runtime's
# own allocations at exit are not this library's, so leak checking is off
ENV = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def available() -> bool:
    return os.path.exists(B.hipcc()) and os.path.exists(CLANG)


def _key() -> str:
    h = hashlib.sha256(" ".join(FLAGS + LINK).encode())
    paths = sorted(os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC) if f.endswith((".hip", ".h")))
    for p in paths + [os.path.join(B.INCLUDE, "rtp.h"), DRIVER]:
        with open(p, "rb") as fh:
            h.update(os.path.basename(p).encode() + fh.read())
    return h.hexdigest()


def build() -> str:
    """Compile (if the sources changed) and return the program's path."""
    key = _key()
    stamp = os.path.join(OUT, "key")
    if os.path.exists(EXE) and os.path.exists(stamp) and open(stamp).read() == key:
        return EXE
    shutil.rmtree(OUT, ignore_errors=True)
    os.makedirs(OUT)

    def cc(src: str, lang=()) -> str:
        obj = os.path.join(OUT, os.path.basename(src).rsplit(".", 1)[0] + ".o")
        r = subprocess.run([B.hipcc(), *FLAGS, *lang, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode:
            raise RuntimeError(f"checked build failed on {src}:\n{r.stderr[-4000:]}")
        return obj

    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(cc, srcs))
    objs.append(cc(DRIVER, ("-x", "hip")))
    r = subprocess.run([CLANG, *objs, *LINK, "-o", EXE], capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"checked build link failed:\n{r.stderr[-4000:]}")
    with open(stamp, "w") as fh:
        fh.write(key)
    return EXE


def layer_tokens(lay: rtp.Layer) -> str:
    """The layer's C struct, field by field, as the program reads it."""
    c = lay.c()
    out = []
    for name, typ in rtp._CLayer._fields_:
        if name == "head_mode":
            out.append("head_mode=" + ",".join(str(int(m)) for m in lay.head_mode))
        elif typ is ctypes.c_double:
            out.append(f"{name}={float(getattr(c, name))!r}")
        else:
            out.append(f"{name}={int(getattr(c, name))}")
    return " ".join(out)


def call_line(name: str, lay, args) -> str:
    toks = []
    for a in args:
        toks.append("L" if isinstance(a, str) and a == "L" else str(0 if a is None else int(a)))
    return f"call {name} {layer_tokens(lay) if lay is not None else ''} | {' '.join(toks)}"


def run(lines) -> tuple[int, list[str], str]:
    env = dict(os.environ)
    env.update(ENV)
    r = subprocess.run([build()], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                       timeout=600)
    return r.returncode, r.stdout.splitlines(), r.stderr
