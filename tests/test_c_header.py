"""The public header compiles as strict C99 and as C++, and a C program
linked against libfd.so calls the host-only entry points (no GPU needed)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "decode_attention_06_amd", "lib")

PROGRAM = r"""
#include "fd.h"
#include "fd_testing.h"
#include <stdio.h>

int main(void) {
    size_t ws = 0;
    fd_status st;
    fd_dtype dt = FD_BF16;
    fd_piece_layout lay = FD_PIECES_INTERLEAVED;
    printf("version %d\n", (int)fd_version());
    printf("status %s %s\n", fd_status_string(FD_OK), fd_status_string(FD_ERR_WORKSPACE));
    printf("plan %d\n", (int)fd_plan_splits(1, 16, 2, 128, 65536, dt, 256));
    printf("tile %d\n", (int)fd_piece_tile_rows(16, 2, 128, dt));
    st = fd_decode_attn_workspace_size(1, 16, 2, 128, 65536, dt, 128, &ws);
    printf("ws %d %lu\n", (int)st, (unsigned long)ws);
    st = fd_decode_attn(NULL, NULL, NULL, NULL, 1, 16, 2, 128, 65536, dt, 0, NULL, FD_BF16, NULL, 0.0f, NULL, 0, NULL);
    printf("null %s %d\n", fd_status_string(st), fd_last_error_message()[0] != '\0');
    printf("layout %d max %d\n", (int)lay, FD_MAX_SPLITS);
    st = fd_testing_decode_attn(NULL, NULL, NULL, NULL, NULL, NULL, 1, 16, 2, 128, 512, dt, 4, NULL, FD_F32, NULL,
                                0.0f, NULL, 0, NULL, 7);
    printf("testing %s\n", fd_status_string(st));
    st = fd_decode_attn_noalloc(NULL, NULL, NULL, NULL, 1, 16, 2, 128, 512, dt, 4, NULL, FD_F32, NULL, 0.0f, NULL);
    printf("noalloc %s %u\n", fd_status_string(st), (unsigned)FD_NOALLOC_MAX_WORKSPACE);
    return 0;
}
"""


@pytest.mark.parametrize("compiler,flags", [("gcc", ["-x", "c", "-std=c99", "-pedantic"]),
                                            ("g++", ["-x", "c++", "-std=c++17"])])
def test_header_compiles_and_links(tmp_path, compiler, flags):
    if not shutil.which(compiler):
        pytest.skip(f"{compiler} not found")
    if not os.path.exists(os.path.join(LIBDIR, "libfd.so")):
        pytest.fail("libfd.so is not built")
    src = tmp_path / "use_fd.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "use_fd"
    cmd = [compiler] + flags + ["-Wall", "-Wextra", "-Werror", "-I", INCLUDE, str(src), "-x", "none",
                                "-L", LIBDIR, "-lfd", "-Wl,-rpath," + LIBDIR, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    lines = dict(line.split(" ", 1) for line in r.stdout.strip().splitlines())
    assert lines["status"] == "FD_OK FD_ERR_WORKSPACE"
    assert 128 <= int(lines["plan"]) <= 512
    assert lines["tile"] == "128"
    st, ws = lines["ws"].split()
    assert st == "0" and int(ws) >= 16 * 128 * 129 * 4
    assert lines["null"] == "FD_ERR_INVALID_ARG 1"
    assert lines["layout"] == "1 max 4096"
    assert lines["testing"] == "FD_ERR_INVALID_ARG"
    assert lines["noalloc"] == "FD_ERR_INVALID_ARG 16777216"
