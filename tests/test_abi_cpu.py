"""Host-only checks of the C ABI library: it loads and exports what include/hspz.h declares.

No compute call is made (no GPU here); parity lives in the gpu-marked tests.
"""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hspz.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hspz_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_symbol_list():
    import ungapped_drop_hsp_amd as h
    assert _declared() == sorted(h.ABI_SYMBOLS)


def test_library_exports_every_declared_symbol():
    import ungapped_drop_hsp_amd as h
    out = subprocess.run(["nm", "-D", "--defined-only", h.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [s for s in _declared() if s not in exported]
    assert not missing, missing
    # nothing but the ABI is exported as a function
    extra = sorted(s for s in exported if s.startswith("hspz") and s not in _declared())
    assert not extra, extra
    lib = h.lib()
    for s in _declared():
        assert getattr(lib, s) is not None


def test_library_is_built_for_gfx950():
    import ungapped_drop_hsp_amd as h
    blob = open(h.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


def test_create_rejects_bad_parameters_without_gpu():
    # parameter validation happens before any device call
    import ungapped_drop_hsp_amd as h
    from workloads import HOXD70
    for kw in (dict(seed_pattern="0111"), dict(seed_pattern="1" * 15),
               dict(seed_pattern="11x1"), dict(hsp_threshold=0), dict(hsp_threshold=2**30 + 1),
               dict(xdrop=-1),
               dict(expand_mode=3), dict(chunk_walk=2), dict(gate_mode=6),
               dict(gate_mode=-1), dict(entropy_mode=2), dict(ref_buckets=257),
               dict(ref_buckets=-1), dict(materialize_mode=3), dict(materialize_mode=-1),
               dict(gate_mode=2, xdrop=600)):  # 7 * max score > X: no exact window gate
        args = dict(seed_pattern="1110100110010101111", sub=HOXD70, n_score=-100, xdrop=910,
                    hsp_threshold=3000)
        args.update(kw)
        with pytest.raises(h.HspzError) as ei:
            h.Engine(**args)
        assert ei.value.code == -1
        # rejected by the parameter checks, not for want of a device
        assert "device" not in str(ei.value), (kw, str(ei.value))


def test_import_fails_loudly_without_library(tmp_path):
    # a copy of the package without libhspz.so must refuse to import
    import shutil
    pkg = os.path.join(ROOT, "ungapped_drop_hsp_amd")
    dst = tmp_path / "ungapped_drop_hsp_amd"
    shutil.copytree(pkg, dst, ignore=shutil.ignore_patterns("*.so", "csrc", "__pycache__"))
    r = subprocess.run(["python", "-c", "import ungapped_drop_hsp_amd"], cwd=tmp_path,
                       capture_output=True, text=True)
    assert r.returncode != 0 and "not built" in r.stderr
