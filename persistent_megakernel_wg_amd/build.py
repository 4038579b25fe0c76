"""Build libamk.so (HIP for gfx950 + host C++) in-tree with hipcc."""
import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libamk.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-fPIC", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-Wall",
          "-Wno-unused-function", "-Wno-unused-variable"]
# packed fp32 VALU forms are disabled for all device code
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-munsafe-fp-atomics"]
HOST = ["-x", "c++", "-ffp-contract=off"]

SOURCES = [  # (file, language, extra flags, object name)
    ("api.cpp", "host", [], "api"),
    ("layout.cpp", "host", [], "layout"),
    ("lower.cpp", "host", [], "lower"),
    ("validate.cpp", "host", [], "validate"),
    ("pack.cpp", "host", [], "pack"),
    ("vm.hip", "device", [], "vm"),
] + [  # one object per kernel instance (pipeline depth, weight format)
    ("vm_inst.hip", "device", [f"-DAMK_INST_DEPTH={d}", f"-DAMK_INST_WFMT={w}"], f"vm_d{d}_w{w}")
    for d in (4, 8, 16) for w in (0, 1, 2)
]


def _compile(name, lang, flags_extra, objname, extra):
    src = os.path.join(CSRC, name)
    obj = os.path.join(BUILD_DIR, objname + ".o")
    flags = COMMON + (DEVICE if lang == "device" else HOST) + flags_extra + extra
    cmd = [HIPCC] + flags + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stderr or "").splitlines() if noise not in ln and ln.strip()]
    return obj, "\n".join(msgs)


def build(extra_flags=(), verbose=False, out=None):
    """Compile and link; `out` defaults to the package's libamk.so."""
    out = out or OUT
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags)
    workers = min(16, os.cpu_count() or 4)
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
        futs = {ex.submit(_compile, n, lang, fl, ob, extra): ob for n, lang, fl, ob in SOURCES}
        objs = []
        for f in concurrent.futures.as_completed(futs):
            obj, msg = f.result()
            objs.append(obj)
            if verbose and msg:
                print(f"[{futs[f]}]\n{msg}", file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + sorted(objs)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
