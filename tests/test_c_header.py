"""The C ABI from C: include/muon_rocm.h compiles as strict C99, and a C program linked
against libmuon_rocm.so calls the host-only entry points (no GPU needed): the version,
status strings, default hyperparameters, and the three workspace planners, including
their error codes.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

from matrix_orthogonalising_optimizer_02_amd import build as BUILD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "muon_rocm.h"

int main(void) {
    muon_hparams hp;
    adamw_hparams ahp;
    size_t bytes = 0;
    int64_t rows[2] = {5120, 30720}, cols[2] = {5120, 5120};
    muon_shard sh[1];
    int fails = 0;
    if (muon_abi_version() != MUON_ABI_VERSION) fails++;
    if (strcmp(muon_status_str(MUON_OK), "ok") != 0) fails++;
    muon_default_hparams(&hp);
    if (hp.ns_steps != 5 || hp.period_k != 3 || hp.scale_mode != MUON_SCALE_MAX_DIM) fails++;
    if (hp.ns_a < 3.44f || hp.ns_a > 3.45f || hp.gamma < 0.149f || hp.gamma > 0.151f) fails++;
    adamw_default_hparams(&ahp);
    if (ahp.beta2 < 0.998f || ahp.beta2 > 0.9991f) fails++;
    if (muon_workspace_bytes(rows, cols, 2, &bytes) != MUON_OK || bytes == 0) fails++;
    if (svd_entropy_workspace_bytes(rows, cols, 2, &bytes) != MUON_OK || bytes < (size_t)2 * 5120 * 5120 * 8) fails++;
    sh[0].rows = 3840; sh[0].cols = 5120; sh[0].full_rows = 30720;
    sh[0].w = NULL; sh[0].m = NULL; sh[0].g = NULL;
    if (rownorm_shard_workspace_bytes(sh, 1, &bytes) != MUON_OK || bytes == 0) fails++;
    sh[0].full_rows = 4000; /* not tall: rejected */
    if (rownorm_shard_workspace_bytes(sh, 1, &bytes) != MUON_ERR_INVALID_ARG) fails++;
    if (strlen(muon_last_error()) == 0) fails++;
    if (muon_workspace_bytes(rows, cols, -1, &bytes) != MUON_ERR_INVALID_ARG) fails++;
    printf("c abi checks: %d failures\n", fails);
    return fails;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_header_is_c99_and_host_calls_work_from_c():
    if not os.path.exists(BUILD.LIB_PATH):
        BUILD.build()
    tmp = tempfile.mkdtemp(prefix="muon_c_abi_")
    try:
        src = os.path.join(tmp, "abi.c")
        exe = os.path.join(tmp, "abi")
        with open(src, "w") as fh:
            fh.write(C_PROGRAM)
        libdir = os.path.dirname(BUILD.LIB_PATH)
        cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{ROOT}/include", src,
               f"-L{libdir}", "-lmuon_rocm", f"-Wl,-rpath,{libdir}", "-Wl,-rpath-link,/opt/rocm/lib", "-o", exe]
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        assert res.returncode == 0, res.stdout
        env = dict(os.environ)
        env["LD_LIBRARY_PATH"] = "/opt/rocm/lib:" + env.get("LD_LIBRARY_PATH", "")
        run = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=env,
                             timeout=120)
        assert run.returncode == 0 and "0 failures" in run.stdout, run.stdout
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
