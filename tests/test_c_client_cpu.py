"""The C client on the host: it builds against the public header with
-Wall -Wextra -Werror, and refuses malformed input files with status 2
before it makes any HIP call (so these run without a GPU)."""
import os
import struct
import subprocess

import pytest

from c_client.build import BINARY, build_client


@pytest.fixture(scope="module")
def client():
    if not os.path.exists(BINARY):
        build_client()
    return BINARY


def _run(client, tmp_path, data: bytes):
    src = tmp_path / "in.bin"
    src.write_bytes(data)
    return subprocess.run([client, str(src), str(tmp_path / "out.bin")], capture_output=True,
                          text=True, timeout=60)


def test_usage(client):
    proc = subprocess.run([client], capture_output=True, text=True, timeout=60)
    assert proc.returncode == 2 and "usage" in proc.stderr


def test_missing_file(client, tmp_path):
    proc = subprocess.run([client, str(tmp_path / "none.bin"), str(tmp_path / "o.bin")],
                          capture_output=True, text=True, timeout=60)
    assert proc.returncode == 2 and "cannot read" in proc.stderr


@pytest.mark.parametrize("data,why", [
    (b"", "bad header"),
    (struct.pack("<11q", 0x1234, 4, 1, 0, 256, 1, 1, 1, 1, 0, 0), "bad header"),
    (struct.pack("<11q", 0x5A43, 0, 1, 0, 256, 1, 1, 1, 1, 0, 0), "bad sizes"),     # N = 0
    (struct.pack("<11q", 0x5A43, 65, 1, 0, 256, 1, 1, 1, 1, 0, 0), "bad sizes"),    # N > 64
    (struct.pack("<11q", 0x5A43, 4, 1, 4, 256, 1, 1, 1, 1, 0, 0), "bad sizes"),     # rank = N
    (struct.pack("<11q", 0x5A43, 4, 1, 0, 0, 1, 1, 1, 1, 0, 0), "bad sizes"),       # align 0
    (struct.pack("<11q", 0x5A43, 4, 2, 0, 256, 1, 1, 1, 1, 0, 0) + struct.pack("<q", 5),
     "bad sizes"),                                                                 # cut short
], ids=["empty", "magic", "no_replicas", "too_many_replicas", "rank_out_of_range",
        "align_zero", "truncated"])
def test_refuses_malformed_input(client, tmp_path, data, why):
    proc = _run(client, tmp_path, data)
    assert proc.returncode == 2 and why in proc.stderr, proc.stderr
