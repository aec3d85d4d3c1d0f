"""The weight-byte accounting reproduces the figures the pages print."""
import pytest

import goldens
from skinny_bit_block_amd import accounting as acc


def test_pages_figures():
    rows = goldens.accounting()
    assert len(rows) == 11
    for kind, v in rows:
        if kind == "floor":
            ms = v["bytes"] / (v["bw_gbs"] * 1e9) * 1e3
            assert abs(ms - v["ms"]) <= v["tol_ms"]
            continue
        wb = acc.weight_bytes(int(v["N"]), int(v["K"]))
        sec = v["ms"] * 1e-3
        # the page prints times to 3 decimals (+-0.0005 ms) and results to 1 decimal
        rel = 0.0005 / v["ms"]
        if kind == "pct":
            got = acc.pct_of(wb, sec, 273e9)
            assert abs(got - v["pct"]) <= got * rel + 0.05, v
        else:
            got = acc.gbs(wb, sec)
            assert abs(got - v["gbs"]) <= got * rel + 0.05, v


def test_weight_bytes_is_4p5_bits():
    assert acc.weight_bytes(2048, 2048) == 2359296
    assert acc.weight_bytes(34816, 5120) == 100270080
    assert acc.weight_bytes(5120, 17408) == 50135040
    assert acc.weight_bytes(151936, 5120) == 437575680
    assert acc.weight_bytes(7, 512) * 16 == 7 * 512 * 9
    with pytest.raises(ValueError):
        acc.weight_bytes(3, 300)


def test_full_pass():
    shapes = acc.full_pass_shapes()
    assert len(shapes) == 513
    assert acc.full_pass_weight_bytes() == 15725813760
    # floor at 8.0 TB/s
    assert abs(acc.floor_seconds(acc.full_pass_weight_bytes()) - 1.9657e-3) < 1e-6


def test_roofline_guard():
    wb = acc.weight_bytes(34816, 5120)
    floor = wb / 8.0e12
    acc.check_roofline(wb, floor * 1.01)
    with pytest.raises(acc.RooflineViolation):
        acc.check_roofline(wb, floor * 0.99)
    # the pages' own case: 57 ms for 15.8 GB at 273 GB/s is "faster than physics"
    with pytest.raises(acc.RooflineViolation):
        acc.check_roofline(15.8e9, 57e-3, peak_bytes_per_s=273e9)
    acc.check_counter_bytes(0.99 * wb, wb)
    with pytest.raises(acc.RooflineViolation):
        acc.check_counter_bytes(0.5 * wb, wb)
