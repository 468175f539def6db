"""Build libkvq.so (HIP, gfx950) in-tree.

``python -m quantized_kv_cache_kvq_amd.build`` compiles every translation
unit under ``csrc/`` with hipcc in parallel and links the shared library next
to this file.  Always recompiles (the build is the check that the sources
compile for gfx950).
"""

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libkvq.so")
OBJ = os.path.join(ROOT, "_build", "obj")

ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    # packed fp32 VALU ops stay off: only scalar/float2 code reaches the ISA
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def source_hash():
    """sha256 (16 hex digits) over the HIP sources and headers the library
    is built from, with comments and whitespace removed: edits to comments
    leave it unchanged.  Compiled into the library (kvq_source_hash) so that
    lib.load() can refuse a library built from other sources."""
    import hashlib
    import re

    def code(path):
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        return " ".join(text.split()).encode()

    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode())
            h.update(code(os.path.join(CSRC, name)))
    h.update(code(os.path.join(ROOT, "include", "kvq.h")))
    return h.hexdigest()[:16]


def hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, defines=()):
    obj = os.path.join(OBJ, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc()] + FLAGS + list(defines) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    return src, obj, r.returncode, err


def build(verbose=True, jobs=None):
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    objs = []
    defs = ['-DKVQ_SOURCE_HASH="%s"' % source_hash()]
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for src, obj, rc, err in ex.map(lambda f: _compile(f, defs), srcs):
            if err.strip() and verbose:
                print(err, file=sys.stderr)
            if rc != 0:
                raise RuntimeError("hipcc failed on %s" % os.path.basename(src))
            objs.append(obj)
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print("built", OUT)
    return OUT


if __name__ == "__main__":
    build()
