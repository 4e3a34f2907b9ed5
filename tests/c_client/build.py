"""Build the C client of libzerostep.so (zero_client.c) with gcc: host code
only, linked against the HIP runtime and the in-tree library, which it finds
beside it in the package directory at run time."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SOURCE = os.path.join(HERE, "zero_client.c")
BINARY = os.path.join(HERE, "zero_client")
PKG = os.path.join(ROOT, "sharded_mixed_precision_step_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_client(verbose: bool = False) -> str:
    """Compile the client (written atomically); the library must be built."""
    gcc = shutil.which("gcc")
    if gcc is None:
        raise RuntimeError("gcc not found")
    fd, tmp = tempfile.mkstemp(prefix=".zero_client.", suffix=".tmp", dir=HERE)
    os.close(fd)
    cmd = [gcc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           SOURCE, "-o", tmp,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-L", PKG, "-lzerostep",
           f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
           "-Wl,-rpath,$ORIGIN/../../sharded_mixed_precision_step_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    try:
        proc = subprocess.run(cmd, capture_output=True, text=True)
        if proc.returncode != 0:
            raise RuntimeError(f"gcc failed ({proc.returncode}):\n{proc.stdout}\n{proc.stderr}")
        os.chmod(tmp, 0o755)
        os.replace(tmp, BINARY)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return BINARY
