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


def test_two_regime_fit_recovers_alpha_and_beta():
    """Calls follow T = L*alpha + moved/beta where the model holds (small
    calls; calls larger than the last-level cache) and run twice as fast in
    between, as cache-resident calls do: the fit still returns alpha and
    beta, where one line through every size would not."""
    n, launches, alpha, beta = 8, 14, 3e-6, 5e12
    pts = []
    for k in range(10, 29):
        s = 1 << k
        moved = 5 * (n - 1) * s
        cached = s > bench.SWEEP_LATENCY_MAX and n * s <= bench.LLC_BYTES
        pts.append((s, moved, launches * alpha + moved / (2 * beta if cached else beta)))
    a, b = bench.alpha_beta_fit(pts, launches, n)
    assert a == pytest.approx(alpha) and b == pytest.approx(beta)
    a1, b1 = bench.fit_line([p[1] for p in pts], [p[2] for p in pts])
    assert abs(a1 / launches - alpha) > 0.1 * alpha or abs(1 / b1 - beta) > 0.1 * beta
