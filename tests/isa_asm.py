"""The library's device code compiled to gfx950 assembly (hipcc -S) for the
ISA tests.  The compile takes minutes, so the test session starts it in the
background once collection ends (conftest.py) and runs the ISA tests last;
the tests then wait for it.  Run alone, the tests start it themselves."""
import atexit
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
from ordered_merge_sorted_amd import build  # noqa: E402

JOB = None  # (process, output path) of the compile in flight or done


def available() -> bool:
    return shutil.which(build.hipcc()) is not None


def start():
    """Starts the compile (once) and returns its (process, output path)."""
    global JOB
    if JOB is None:
        out_dir = tempfile.mkdtemp(prefix="omerge_isa_")
        out = os.path.join(out_dir, "omerge.s")
        flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
        proc = subprocess.Popen([build.hipcc(), *flags, "--cuda-device-only", "-S", "-x", "hip",
                                 *build.SOURCES, "-o", out], stdout=subprocess.DEVNULL,
                                stderr=subprocess.DEVNULL)

        def cleanup():
            if proc.poll() is None:
                proc.kill()
                proc.wait()
            shutil.rmtree(out_dir, ignore_errors=True)

        atexit.register(cleanup)
        JOB = (proc, out)
    return JOB


def assembly() -> str:
    """Waits for the compile and returns the assembly text."""
    proc, out = start()
    rc = proc.wait()
    if rc != 0:
        raise RuntimeError("hipcc -S of the library failed (exit %d)" % rc)
    with open(out) as f:
        return f.read()
