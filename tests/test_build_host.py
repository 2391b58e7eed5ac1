"""The build records what it was built from, and the entry points rebuild a
library whose sources have changed since, rather than run it (CPU only)."""
import os
import shutil

import pytest

import __graft_entry__
from deterministic_fixed_order_amd import _build


@pytest.fixture
def copied_sources(tmp_path, monkeypatch):
    """The build's inputs copied into tmp_path, with _build pointed at them."""
    names = {}
    for attr in ("KERNELS", "INTERNAL_HEADER", "EXPORTS_MAP", "HEADER"):
        src = getattr(_build, attr)
        dst = tmp_path / os.path.basename(src)
        shutil.copy(src, dst)
        monkeypatch.setattr(_build, attr, str(dst))
        names[attr] = dst
    hosts = []
    for src in _build.HOST_SOURCES:
        dst = tmp_path / os.path.basename(src)
        shutil.copy(src, dst)
        hosts.append(str(dst))
    monkeypatch.setattr(_build, "HOST_SOURCES", hosts)
    monkeypatch.setattr(_build, "SOURCES", [str(names["KERNELS"])] + hosts)
    return tmp_path


def test_digest_follows_every_input(copied_sources):
    base = _build.source_digest()
    assert base == _build.source_digest()
    for name in ("fold_kernels.hip", "plan.cpp", "detfold.cpp", "internal.h", "exports.map", "detfold.h"):
        path = copied_sources / name
        text = path.read_bytes()
        path.write_bytes(text + b"\n")
        assert _build.source_digest() != base, name
        path.write_bytes(text)
        assert _build.source_digest() == base, name


def test_digest_follows_the_flags(copied_sources, monkeypatch):
    base = _build.source_digest()
    monkeypatch.setattr(_build, "device_flags", lambda: ["-fno-gpu-flush-denormals-to-zero"])
    assert _build.source_digest() != base


def test_is_current_needs_library_and_matching_digest(copied_sources):
    lib = str(copied_sources / "libdetfold.so")
    assert not _build.is_current(lib)                     # nothing built
    open(lib, "wb").close()
    assert not _build.is_current(lib)                     # no digest recorded
    with open(lib + ".sha256", "w") as f:
        f.write(_build.source_digest() + "\n")
    assert _build.is_current(lib)
    kernels = copied_sources / "fold_kernels.hip"
    kernels.write_bytes(kernels.read_bytes() + b"// edited\n")
    assert not _build.is_current(lib)                     # a source changed since
    os.remove(lib)
    with open(lib + ".sha256", "w") as f:
        f.write(_build.source_digest() + "\n")
    assert not _build.is_current(lib)                     # digest without a library


def test_ensure_built_rebuilds_only_when_stale(monkeypatch):
    calls = []
    monkeypatch.setattr(__graft_entry__, "build", lambda: calls.append(1))
    monkeypatch.setattr(_build, "is_current", lambda lib=_build.LIB: True)
    __graft_entry__.ensure_built()
    assert calls == []
    monkeypatch.setattr(_build, "is_current", lambda lib=_build.LIB: False)
    __graft_entry__.ensure_built()
    assert calls == [1]


def test_ensure_built_leaves_a_current_library():
    __graft_entry__.ensure_built()
    assert _build.is_current()
