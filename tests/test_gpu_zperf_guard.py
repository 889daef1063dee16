"""Coarse performance guards: the 4K chunk forward and the decode step must
stay within about 1.6x of their measured times on MI355X (0.25 ms per step
and 86 us per step). They catch code changes that silently serialise a
kernel (a run-time branch around stores that makes the compiler wait for
every load, say), which the parity tests cannot see."""
import pytest

pytestmark = pytest.mark.gpu


def test_chunk_forward_4k_step_time():
    import bench
    c, _, x, S0 = bench.chunk_inputs("chunk_4k")
    r = bench.bench_chunk(20, 20, c, x, S0)
    print(f"[perf] 4K chunk forward {r['region_ms']:.4f} ms/step (intra {r['intra_ms']:.4f}, scan {r['scan_ms']:.4f})")
    assert r["region_ms"] < 0.40


def test_decode_step_time():
    import bench
    d = bench.bench_decode(256, steps=256)
    print(f"[perf] decode 256 x 16 heads {d['region_ms'] * 1e3:.1f} us/step")
    assert d["region_ms"] < 0.14
