"""Host logic of the benchmark (no GPU): the read probe's launch sizes and regions stay inside its buffer,
are whole chunks, rotate over at least two regions, and together exceed the 256 MB Infinity Cache wherever
the region count allows."""
import pytest

import bench

TOTAL = bench.ReadProbe.TOTAL
CHUNK = 16384


@pytest.mark.parametrize("nbytes", [0, 1, CHUNK - 1, CHUNK, 132096, 134742016, 272025600, 692736000,
                                    2147745792, 4 << 30, 7 << 30, 1 << 40])
def test_probe_regions_fit_the_buffer(nbytes):
    n, m = bench.probe_regions(nbytes, TOTAL, CHUNK)
    assert n % CHUNK == 0 and CHUNK <= n <= TOTAL // 2
    assert n <= max(CHUNK, nbytes)
    assert 2 <= m <= 64 and m * n <= TOTAL
    if n >= 12 << 20:  # 64 regions of 12 MB already span 768 MB
        assert m * n >= 768 << 20
    if nbytes >= CHUNK and nbytes <= TOTAL // 2:
        assert nbytes - n < CHUNK  # rounded down to the chunk only
