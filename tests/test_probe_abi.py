"""CPU checks of libepdc_probe.so (include/epdc_probe.h), the HBM rate
probes the benchmark uses: the library loads, exports every function the
header declares, and rejects bad arguments before any GPU work."""
import ctypes

import pytest

from combine_routing_histogram_amd import build as hip_build
from combine_routing_histogram_amd import probe


@pytest.fixture(scope="module")
def lib():
    if hip_build.is_stale():
        hip_build.build()
    return probe.lib()


def test_exports_every_declared_function(lib):
    names = probe.header_entry_points()
    assert names == sorted(probe._SIGNATURES)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/epdc_probe.h but not exported"


@pytest.mark.parametrize("call,msg", [
    (lambda l: l.epdc_probe_read(None, 1024, 1, 4096, None), "src is NULL"),
    (lambda l: l.epdc_probe_read(4104, 1024, 1, 4096, None), "16-byte aligned"),
    (lambda l: l.epdc_probe_read(4096, 1000, 1, 8192, None), "multiple of 16"),
    (lambda l: l.epdc_probe_read(4096, 1024, 1, None, None), "flag"),
    (lambda l: l.epdc_probe_write(4096, 0, 0, None), "multiple of 16"),
    (lambda l: l.epdc_probe_write(4100, 1024, 0, None), "16-byte aligned"),
    (lambda l: l.epdc_probe_copy(4096, 4096 + 512, 1024, None), "overlap"),
    (lambda l: l.epdc_probe_copy(4096, None, 1024, None), "dst is NULL"),
])
def test_bad_arguments_are_rejected(lib, call, msg):
    assert call(lib) == -1  # EPDC_ERR_INVALID_ARGS
    assert msg in lib.epdc_probe_last_error().decode()
