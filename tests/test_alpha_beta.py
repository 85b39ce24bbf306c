"""The alpha-beta model the bench reports with, against the worked numbers
the pages print."""
import pytest

import bench


def test_handbook_exercise_1gb():
    """Handbook "集合通信原语", section 练习: 8 ranks, 1 GB, 450 GB/s, 5 us:
    bandwidth term 3.9 ms, latency term 0.07 ms, total about 3.96 ms."""
    lat, bw, total = bench.alpha_beta_time(8, 1e9, 5e-6, 450e9)
    assert lat == pytest.approx(0.07e-3)
    assert round(bw * 1e3, 1) == 3.9
    assert round(total * 1e3, 2) == 3.96


def test_handbook_exercise_1mb():
    """Same exercise at 1 MB: bandwidth 3.9 us against latency 70 us."""
    lat, bw, _ = bench.alpha_beta_time(8, 1e6, 5e-6, 450e9)
    assert round(bw * 1e6, 1) == 3.9
    assert lat == pytest.approx(70e-6)
    assert lat / bw == pytest.approx(18, abs=0.1)  # "nearly 20 times"


def test_geek_doc_7b_example():
    """geek-doc page, section 四: N=8, M=14 GB, alpha about 10 us, 400 GB/s:
    latency term about 0.14 ms, bandwidth term 24.5 GB / 400 GB/s about 61 ms,
    bandwidth more than 99% of the total."""
    lat, bw, total = bench.alpha_beta_time(8, 14e9, 10e-6, 400e9)
    assert lat == pytest.approx(0.14e-3)
    assert 2 * 7 / 8 * 14e9 == pytest.approx(24.5e9)
    assert round(bw * 1e3) == 61
    assert bw / total > 0.99


def test_fit_line_recovers_a_line():
    a, b = bench.fit_line([1.0, 2.0, 3.0, 10.0], [5.0 + 2 * x for x in (1.0, 2.0, 3.0, 10.0)])
    assert a == pytest.approx(5.0) and b == pytest.approx(2.0)
