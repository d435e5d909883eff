import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for p in (ROOT, os.path.dirname(os.path.abspath(__file__))):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


def _is_isa(item):
    return item.fspath.basename == "test_isa.py"


def pytest_collection_modifyitems(config, items):
    """The ISA tests run last (before the no-alloc GPU tests, which end a GPU
    run): their device-assembly compile runs in the background meanwhile."""
    isa = [it for it in items if _is_isa(it)]
    if isa:
        rest = [it for it in items if not _is_isa(it)]
        last = [it for it in rest if it.fspath.basename.startswith("test_zz")]
        first = [it for it in rest if not it.fspath.basename.startswith("test_zz")]
        items[:] = first + isa + last


def pytest_collection_finish(session):
    if any(_is_isa(it) for it in session.items):
        import isa_asm
        if isa_asm.available():
            isa_asm.start()
