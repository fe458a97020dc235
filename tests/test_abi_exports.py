"""The native libraries load on a machine without a GPU and export every
function their public headers declare (no compute calls here)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "speculative_verify_attention_amd")


def declared(header):
    text = open(os.path.join(ROOT, "include", header)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, re.M)
    return sorted(set(names))


def exported(lib_path):
    import subprocess

    out = subprocess.run(["nm", "-D", "--defined-only", lib_path], stdout=subprocess.PIPE, text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if " T " in line}


@pytest.mark.parametrize("lib,headers", [("libsvattn.so", ["svattn.h", "svdraft.h"]),
                                         ("libsvattn_core.so", ["svcore.h", "svdraft.h"])])
def test_exports(lib, headers):
    path = os.path.join(PKG, lib)
    if not os.path.exists(path):
        pytest.skip(f"{lib} not built (python -m speculative_verify_attention_amd.build)")
    ctypes.CDLL(path)  # loads without a device
    have = exported(path)
    for h in headers:
        names = declared(h)
        assert len(names) >= 8
        missing = [n for n in names if n not in have]
        assert not missing, f"{lib} lacks {missing}"


def test_header_declares_the_boundary():
    names = declared("svattn.h")
    for n in ["kv_create", "kv_append", "kv_rollback", "kv_encode", "spec_verify_attn", "kv_destroy",
              "kv_workspace_bytes", "kv_pool_bytes"]:
        assert n in names
