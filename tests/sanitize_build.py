"""CPU sanitizer build: librvq.so with AddressSanitizer and UndefinedBehaviorSanitizer on its HOST code
(argument validation, workspace layouts, record checks, the expert pool's bookkeeping, launchers), and
the oracle and the input generator with both sanitizers.  Device code is compiled as usual and never
instrumented (and nothing here runs on a GPU).  Outputs go to build/sanitize/<source hash>/ and are
reused while the sources are unchanged.  Run under the clang ASan runtime (see runtime_env())."""
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rvq_quantized_moe_amd", "csrc")
sys.path.insert(0, ROOT)
from rvq_quantized_moe_amd import build as _libbuild  # noqa: E402  (the product build's source list)

HIP_SOURCES = [os.path.basename(p) for p in _libbuild.SOURCES if p.endswith(".hip")]
CPP_SOURCES = [os.path.basename(p) for p in _libbuild.SOURCES if p.endswith(".cpp")]
C_LIBS = {"liboracle_san.so": os.path.join(ROOT, "oracle", "rvq_oracle.c"),
          "libsynth_san.so": os.path.join(ROOT, "synth", "synth.c")}
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/llvm/bin/clang"
# the sanitizers apply to the host side of every translation unit only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
COMMON = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-I", os.path.join(ROOT, "include")]


def _hash():
    h = hashlib.sha256()
    files = [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC))] + [os.path.join(ROOT, "include", "rvq.h")]
    files += list(C_LIBS.values()) + [os.path.abspath(__file__)]
    for p in files:
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode() + f.read())
    return h.hexdigest()[:16]


def asan_runtime():
    out = subprocess.check_output([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], text=True).strip()
    if not os.path.exists(out):
        raise FileNotFoundError("clang's AddressSanitizer runtime was not found")
    return out


def runtime_env(outdir):
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan_runtime()
    # the interpreter and the HIP runtime are not instrumented: leak reports would be theirs
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["RVQ_SANITIZED_DIR"] = outdir
    return env


def build():
    outdir = os.path.join(ROOT, "build", "sanitize", _hash())
    lib = os.path.join(outdir, "librvq.so")
    if all(os.path.exists(os.path.join(outdir, n)) for n in ["librvq.so"] + list(C_LIBS)):
        return outdir
    os.makedirs(outdir, exist_ok=True)
    jobs = []
    for f in HIP_SOURCES:
        jobs.append([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                     "-packed-fp32-ops"] + COMMON + HOST_SAN + ["-c", os.path.join(CSRC, f),
                                                                "-o", os.path.join(outdir, f + ".o")])
    for f in CPP_SOURCES:
        jobs.append([HIPCC] + COMMON + HOST_SAN + ["-c", os.path.join(CSRC, f), "-o", os.path.join(outdir, f + ".o")])
    with ThreadPoolExecutor(max_workers=4) as ex:
        for r in ex.map(lambda c: subprocess.run(c, capture_output=True, text=True), jobs):
            if r.returncode != 0:
                raise RuntimeError(r.stderr[-4000:])
    objs = [os.path.join(outdir, f + ".o") for f in HIP_SOURCES + CPP_SOURCES]
    subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + HOST_SAN + ["-o", lib + ".tmp"] + objs)
    os.replace(lib + ".tmp", lib)
    for o in objs:
        os.remove(o)
    for name, src in C_LIBS.items():
        subprocess.check_call([CLANG, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                               "-fno-sanitize-recover=undefined", "-shared", "-fPIC", "-pthread", "-ffp-contract=off",
                               "-o", os.path.join(outdir, name), src, "-lm"])
    return outdir


if __name__ == "__main__":
    print(build())
    sys.exit(0)
