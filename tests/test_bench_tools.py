"""CPU checks of the bench's profile tooling: the per-call kernel times that
`bench.py --trace-summary` derives from a rocprofv3 kernel-trace database
(a `kernels` view of name, start and end in ns), on a synthetic trace whose
timed region and durations are known."""
import os
import sqlite3
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _trace(path, steps, dec_us, exp_us, gemm_us):
    db = sqlite3.connect(path)
    db.execute("create table kernels (name text, start integer, end integer)")
    t = 0

    def add(name, us):
        nonlocal t
        db.execute("insert into kernels values (?, ?, ?)", (name, t, t + int(us * 1000)))
        t += int(us * 1000) + 500

    # a warm-up dispatch and the hold before the timed region (to be skipped)
    add("void aq::(anonymous namespace)::decode_kernel<128>(DArgs)", 99.0)
    add("at::cuda::(anonymous namespace)::spin_kernel(long)", 1000.0)
    for _ in range(steps):           # decode segments of all steps ...
        for k in range(12):
            add("void aq::(anonymous namespace)::quant_act_kernel<1024, 1>(float const*)", 3.0)
            add("void aq::(anonymous namespace)::decode_kernel<128>(DArgs)", dec_us[k])
    for _ in range(steps):           # ... then the prefill segments
        for p in range(4):
            add("void aq::(anonymous namespace)::quant_act_kernel<256, 3>(float const*)", 5.0)
        for p in range(4):
            add("void aq::(anonymous namespace)::expand_kernel<128>(PackedView)", exp_us[p])
            add("void aq::(anonymous namespace)::prefill_dense_kernel<128, 4, 2, 3, false, false, false>(DenseArgs)",
                gemm_us[p])
    db.commit()
    db.close()


def test_trace_summary_timed_region(tmp_path):
    pytest.importorskip("numpy")
    import bench
    dec = [4.0 + k for k in range(12)]
    exp_, gemm = [7.0, 6.0, 17.0, 10.0], [50.0, 40.0, 150.0, 90.0]
    db = str(tmp_path / "t.db")
    _trace(db, 3, dec, exp_, gemm)
    out = bench.trace_summary(db)
    assert "Timed region: 3 steps." in out
    # decode calls by position: M = 1, 4, 16, then projection, in issue order
    assert "| qkv 5120x3072 M=1 | 4.00 |" in out
    assert "| down 3072x8192 M=16 | 15.00 |" in out
    assert f"Decode mean per call: {sum(dec) / 12:.2f} µs." in out
    # prefill: expansion and GEMM per projection; the fraction is 2MNK / time / 5 POPS
    assert "| o 2560x4096 | 6.00 | `prefill_dense_kernel<128, 4, 2, 3, false, false, false>` | 40.00 |" in out
    ops = 2 * 2048 * 2560 * 4096
    assert f"| {ops / 40.0 / 1e6 / 5000:.3f} |" in out
    assert f"Prefill mean per call (expansion + GEMM): {(sum(exp_) + sum(gemm)) / 4:.2f} µs." in out
