"""Checks on our own gfx950 assembly (CPU only: hipcc cross-compiles).

The fold's bits rest on every add being a plain binary32 add under
round-to-nearest-even with subnormals kept, and its bandwidth on the streaming
cache policy.  This rebuilds the library with -save-temps and reads the
gfx950 assembly it produced:

* no fused or packed float arithmetic anywhere (v_fma*/v_fmac*/v_mad*/v_mac*,
  v_fmaak/v_fmamk, mixed-precision forms, packed FP32);
* every kernel descriptor keeps f32 denormals (.amdhsa_float_denorm_mode_32 3);
* no writes through the scalar data cache;
* the LDS row kernels load with the nt and lds bits and store with nt, and
  the fused round writes whole lines through with sc0 sc1;
* the default kernels spill nothing to scratch.
"""
import glob
import os
import re

import pytest

FUSED = re.compile(r"^\s*(v_fma\w*|v_fmac\w*|v_mad_f\w*|v_mad_mix\w*|v_mac\w*|v_fmaak\w*|v_fmamk\w*"
                   r"|v_pk_fma\w*|v_pk_add_f32|v_pk_mul_f32|v_dot\w*)\b", re.M)
SCALAR_WRITE = re.compile(r"^\s*(s_store\w*|s_buffer_store\w*|s_atomic\w*|s_buffer_atomic\w*"
                          r"|s_dcache_wb\w*|s_dcache_discard\w*|s_scratch_store\w*)\b", re.M)


@pytest.fixture(scope="module")
def isa(tmp_path_factory):
    from deterministic_fixed_order_amd import _build
    out = str(tmp_path_factory.mktemp("isa"))
    _build.save_temps(out)  # a failed build fails every test here, never skips it
    files = sorted(glob.glob(os.path.join(out, "*gfx950*.s")))
    assert files, "no gfx950 assembly produced"
    return "\n".join(open(f).read() for f in files)


def _kernels(text):
    """(demangled-ish name, metadata block) for every kernel."""
    meta = text[text.index("amdhsa.kernels:"):]
    return [(m.group(1), m.group(0)) for m in
            re.finditer(r"- \.agpr_count:.*?\.name:\s+(\S+).*?\.wavefront_size:\s+\d+", meta, re.S)]


def test_no_fused_or_packed_float_arithmetic(isa):
    hits = FUSED.findall(isa)
    assert not hits, "fused/packed float instructions: %s" % sorted(set(hits))


def test_f32_denormals_kept_in_every_kernel(isa):
    modes = re.findall(r"\.amdhsa_float_denorm_mode_32\s+(\d+)", isa)
    assert modes and set(modes) == {"3"}


def test_no_scalar_cache_writes(isa):
    assert not SCALAR_WRITE.findall(isa)


def test_row_kernels_stream_through_lds(isa):
    loads = re.findall(r"^\s*buffer_load_dwordx4\s+.*\blds\b.*$", isa, re.M)
    assert loads and all(" nt" in l for l in loads)
    stores = re.findall(r"^\s*buffer_store_dwordx4\s.*$", isa, re.M)
    assert any(l.rstrip().endswith(" nt") for l in stores)
    assert any("sc0 sc1" in l for l in stores)


def test_default_kernels_do_not_spill(isa):
    ks = _kernels(isa)
    assert ks
    for name, block in ks:
        default = "k_fold_rows" in name or re.search(r"k_fold_vectorILi\d+ELi1E", name) \
            or "k_copy_out" in name
        if default:
            priv = int(re.search(r"\.private_segment_fixed_size:\s+(\d+)", block).group(1))
            assert priv == 0, "%s spills %d bytes" % (name, priv)
