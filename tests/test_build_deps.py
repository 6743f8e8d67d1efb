"""The build's dependency list: every header the HIP sources include makes a
library built before its last edit stale, so that a test run rebuilds it
(CPU only; no compiler is run)."""
import os

from combine_moe_get_dispatch_amd import build_lib


def _included_headers():
    """Headers named by an #include "..." line of the HIP sources and headers."""
    names = set()
    for d in build_lib.sources() + build_lib.headers():
        for line in open(d):
            line = line.strip()
            if line.startswith("#include \""):
                names.add(os.path.normpath(os.path.join(os.path.dirname(d), line.split('"')[1])))
    return names


def test_every_included_header_is_a_dependency():
    deps = set(os.path.normpath(h) for h in build_lib.headers())
    missing = _included_headers() - deps
    assert not missing, f"headers missing from the build's dependency list: {sorted(missing)}"
    for name in ("element_codecs.h", "small_batch.h", "device_common.h", "launch.h"):
        assert os.path.join(build_lib.CSRC, name) in build_lib.headers()


def test_a_newer_header_makes_the_library_stale(tmp_path):
    lib = tmp_path / "lib.so"
    lib.write_bytes(b"")
    deps = build_lib.sources() + build_lib.headers()
    newest = max(os.path.getmtime(d) for d in deps)
    os.utime(lib, (newest + 10, newest + 10))
    assert not build_lib.is_stale(str(lib))
    assert build_lib.is_stale(str(tmp_path / "absent.so"))
    for h in build_lib.headers():
        st = os.stat(h)
        try:
            os.utime(h, (st.st_atime, newest + 20))
            assert build_lib.is_stale(str(lib)), h
        finally:
            os.utime(h, (st.st_atime, st.st_mtime))
    assert not build_lib.is_stale(str(lib))
