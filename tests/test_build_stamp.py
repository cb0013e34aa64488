"""The build records a hash of its sources beside the library, and the suite
rebuilds when that hash no longer matches (a stale library is never tested)."""

import importlib.util
import os
import shutil

from conftest import ROOT

_spec = importlib.util.spec_from_file_location(
    "_moe_build_t", os.path.join(ROOT, "mixture_experts_expert_amd", "build.py"))
build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(build)


def test_current_library_is_not_stale():
    # conftest rebuilt it if needed before any test ran
    assert not build.is_stale()


def test_hash_follows_every_source_and_header(tmp_path, monkeypatch):
    csrc, inc = tmp_path / "csrc", tmp_path / "include"
    shutil.copytree(build.CSRC, csrc)
    shutil.copytree(build.INCLUDE, inc)
    monkeypatch.setattr(build, "CSRC", str(csrc))
    monkeypatch.setattr(build, "INCLUDE", str(inc))
    h0 = build.source_hash()
    assert h0 == build.source_hash()
    for path in (csrc / "combine.hip", csrc / "gemm_common.h", inc / "moe_native.h"):
        old = path.read_bytes()
        path.write_bytes(old + b"\n")
        assert build.source_hash() != h0, path.name
        path.write_bytes(old)
    assert build.source_hash() == h0


def test_missing_stamp_reads_as_stale(tmp_path, monkeypatch):
    monkeypatch.setattr(build, "STAMP", str(tmp_path / "absent.srchash"))
    assert build.is_stale()
    stamp = tmp_path / "old.srchash"
    stamp.write_text("0000000000000000\n")
    monkeypatch.setattr(build, "STAMP", str(stamp))
    assert build.is_stale()
