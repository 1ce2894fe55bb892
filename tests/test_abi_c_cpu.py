"""The boundary is a C ABI: a C99 program that includes only
include/vc_attention.h (plus the HIP runtime API header it names) compiles
warning-free with gcc, links against libvcattn.so, and gets the documented
buffer sizes and error behaviour from host-only calls (no GPU needed)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "bit_attention_video_smooth_amd")

PROGRAM = r"""
#include <stdio.h>
#include "vc_attention.h"

int main(void) {
    /* a bad shape: rejected with VC_ERR_INVALID and a message */
    vc_shape bad = {1, 1, 0, 64};
    size_t sz[9];
    if (vc_prepared_sizes(&bad, sz) != VC_ERR_INVALID || vc_last_error()[0] == '\0') return 1;
    /* a good shape: the documented byte sizes (nb = ceil(L/128), Lp = 128 nb) */
    vc_shape s = {2, 3, 300, 128};
    if (vc_prepared_sizes(&s, sz) != VC_OK) return 2;
    const size_t BH = 6, nb = 3, Lp = 384, d = 128;
    const size_t want[9] = {BH * Lp * d, BH * Lp * d, BH * nb * d * 128, BH * nb * 4, BH * nb * 4,
                            BH * nb * d * 4, BH * nb * d * 4, BH * 300 * 4, BH * 8};
    for (int i = 0; i < 9; i++)
        if (sz[i] != want[i]) { printf("size %d: %zu != %zu\n", i, sz[i], want[i]); return 3; }
    vsmooth_params p = {128, 0, 8, 1, 0, 0, 42};
    size_t ws = 0;
    if (vsmooth_workspace_bytes(&s, &p, &ws) != VC_OK || ws == 0) return 4;
    p.block = 64;  /* only 128-token blocks */
    if (vsmooth_workspace_bytes(&s, &p, &ws) != VC_ERR_UNSUPPORTED) return 5;
    printf("ok version %d\n", vc_version());
    return 0;
}
"""


def test_header_is_c_and_library_links(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(os.path.join(PKG, "libvcattn.so")):
        pytest.fail("needs gcc and the built libvcattn.so")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    src = tmp_path / "abi.c"
    src.write_text(PROGRAM)
    exe = tmp_path / "abi"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), str(src),
           "-L", PKG, "-lvcattn", "-Wl,-rpath," + PKG, "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.startswith("ok version")
