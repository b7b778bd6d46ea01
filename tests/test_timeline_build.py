"""The timeline build is a separate library: the same entry points plus
pkv_timeline_read, while the product library exports no timeline reader.
CPU only (nothing is called on a device)."""
import ctypes

import pytest

import paged_gqa_decode_pkv_amd as pkv
from paged_gqa_decode_pkv_amd import build as pkv_build


def test_product_library_has_no_timeline_reader():
    lib = ctypes.CDLL(pkv.LIB_PATH)
    assert not hasattr(lib, "pkv_timeline_read")
    assert hasattr(lib, "pkv_decode")


@pytest.mark.slow
def test_timeline_build_exports_the_reader_and_every_entry_point():
    path = pkv_build.build(timeline=True)
    assert path == pkv_build.TIMELINE_LIB
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "pkv_timeline_read")
    for name in pkv.ABI_SYMBOLS:
        assert hasattr(lib, name), name
    lib.pkv_abi_version.restype = ctypes.c_int
    assert lib.pkv_abi_version() == pkv.PKV_ABI_VERSION
