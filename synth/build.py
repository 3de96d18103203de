"""Build the host (gcc) and device (hipcc, gfx950) fillers of the generator."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["-O3", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose=False):
    host_out = os.path.join(HERE, "libsynth_host.so")
    dev_out = os.path.join(HERE, "libsynth_dev.so")
    cmds = [
        ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", os.path.join(HERE, "synth_host.c"),
         "-o", host_out + ".tmp"],
        ["hipcc", *HIP_FLAGS, "-shared", "-fPIC", os.path.join(HERE, "synth_dev.hip"), "-o", dev_out + ".tmp"],
    ]
    for cmd, out in zip(cmds, (host_out, dev_out)):
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
        os.replace(out + ".tmp", out)
        if verbose:
            print("built", out)
    return host_out, dev_out


def build_host_only():
    host_out = os.path.join(HERE, "libsynth_host.so")
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", os.path.join(HERE, "synth_host.c"),
           "-o", host_out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(r.stderr)
    os.replace(host_out + ".tmp", host_out)
    return host_out


if __name__ == "__main__":
    build(verbose=True)
