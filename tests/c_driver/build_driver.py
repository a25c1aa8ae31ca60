"""Build tests/c_driver/muon_c_driver (host code only) against libmuon_rocm.so."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "muon_c_driver")
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def build_driver() -> str:
    from matrix_orthogonalising_optimizer_02_amd import build as B

    libdir = os.path.dirname(B.LIB_PATH)
    # compiled as HIP (host code only) so that hipcc supplies the HIP runtime headers
    cmd = [B.hipcc(), "-x", "hip", f"--offload-arch={B.ARCH}", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-O2", "-Wall", "-Werror", f"-I{ROOT}/include",
           os.path.join(HERE, "muon_c_driver.c"), f"-L{libdir}", "-lmuon_rocm", f"-Wl,-rpath,{libdir}",
           "-o", EXE + ".tmp"]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("driver build failed:\n" + " ".join(cmd) + "\n" + res.stdout)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build_driver())
