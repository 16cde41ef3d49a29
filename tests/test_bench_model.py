"""The benchmark's byte models and step classes (CPU): the per-launch
algorithmic bytes of each variant average to the documented bytes per point
per step, and the committed counter summary is found by the traffic lookup
when it was taken on the current kernel source."""
import json
import os

import pytest

import bench

N = 1024 * 1024 * 128


@pytest.mark.parametrize("variant,per_point", [("interleaved", 82), ("interleaved_no_q", 72), ("f32", 41),
                                               ("mixed", 74)])
def test_steady_state_bytes(variant, per_point):
    # four steady-state steps (three that defer the x update, one that
    # applies four) of both passes
    f = bench.BYTES_BY_VARIANT[variant][0]
    tot = sum(f(kern, k) for kern in ("fused_prec", "fused_spmv") for k in (5, 6, 7, 8))
    assert tot == 4 * per_point
    assert bench.BYTES_BY_VARIANT[variant][1] == per_point


def test_step_classes_and_timed_launches():
    assert bench.step_class("interleaved", "fused_spmv", 0) == "first"
    assert bench.step_class("interleaved", "fused_spmv", 3) == "nox"
    assert bench.step_class("interleaved", "fused_spmv", 4) == "x4"
    assert bench.step_class("interleaved", "fused_spmv", 6) == "nox"
    assert bench.step_class("interleaved", "fused_prec", 4) == "rest"
    # a solve of K steps times K+1 preconditioner passes and K stencil passes
    assert len(list(bench.timed_steps("fused_prec", [10, 7]))) == 19
    assert len(list(bench.timed_steps("fused_spmv", [10, 7]))) == 17
    tot, cnt = bench.pass_bytes("interleaved", "fused_spmv", [5], 1)
    assert (tot, cnt) == (24 + 40 + 40 + 40 + 80, 5)


def test_mg_cycle_bytes():
    pts = [N // 4 ** l for l in range(11)]          # 1024^2 x 128 down to one column
    per = bench.mg_cycle_bytes(pts, 1) / N
    assert 114.0 < per < 115.5
    # level 0 alone: 32 + 24 + 32 per point and 16 per coarse point
    assert bench.mg_cycle_bytes([N, N // 4], 1) == 88 * N + 16 * (N // 4) + 16 * (N // 4)
    tot, cnt = bench.mg_pass_bytes(pts, [2])
    assert cnt == 3 and tot == bench.mg_cycle_bytes(pts, 0) + 2 * bench.mg_cycle_bytes(pts, 1)


def test_kernel_digest_ignores_comments_only(tmp_path):
    src = open(bench.KERNEL_SOURCE, encoding="utf-8").read()
    p1, p2, p3 = tmp_path / "a.hpp", tmp_path / "b.hpp", tmp_path / "c.hpp"
    p1.write_text(src)
    p2.write_text("// a new comment\n" + src.replace("{", "{ /* note */", 1) + "\n\n")
    p3.write_text(src.replace("kWave = 64", "kWave = 32", 1))
    assert bench.kernel_source_digest(str(p1)) == bench.kernel_source_digest(str(p2))
    assert bench.kernel_source_digest(str(p1)) != bench.kernel_source_digest(str(p3))


def test_traffic_record_matches_source_or_is_ignored():
    rec = json.load(open(bench.TRAFFIC_FILE))
    t = bench.measured_traffic("fused_spmv", "varying-1024x1024x128", "interleaved", [927])
    if rec.get("code_digest") == bench.kernel_source_digest():
        assert t is not None and 6.5e9 < t < 8.5e9
    else:
        assert t is None
    assert bench.measured_traffic("fused_spmv", "other-workload", "interleaved", [927]) is None


def test_standard_bytes():
    # K steps: 104 B per point per step, plus 32 before the loop (z = M^-1 r0,
    # p = z), minus the column solve and p update of step K (launched after
    # the stop test, they return at once)
    for K in (1, 5, 40):
        tot = sum(bench.standard_bytes(kind, [K], 1) for kind in ("apply_A", "precond", "vector"))
        assert tot == 104 * K + 32 - 16 - 24


def test_mg_cycle_bytes_with_coarse_sweeps():
    pts = [N // 4 ** l for l in range(5)]            # 1024^2 down to 64^2 columns
    base = bench.mg_cycle_bytes(pts, 1)              # coarsest treated as one exact solve
    assert bench.mg_cycle_bytes(pts, 1, coarse_sweeps=64) - base == 24 * 63 * pts[-1]
    assert bench.mg_cycle_bytes(pts, 1, coarse_sweeps=64, two_pass_sweeps=True) - base == 48 * 63 * pts[-1]
    # Chebyshev steps: the first like a damped sweep, every later one also
    # reads z_{k-1}
    assert bench.mg_cycle_bytes(pts, 1, coarse_sweeps=16, chebyshev=True) - base == (24 + 32 * 14) * pts[-1]
    assert bench.mg_cycle_bytes(pts, 1, coarse_sweeps=16, two_pass_sweeps=True, chebyshev=True) - base == \
        (48 + 56 * 14) * pts[-1]
    assert bench.mg_cycle_bytes(pts, 1, coarse_sweeps=1, chebyshev=True) == bench.mg_cycle_bytes(pts, 1, coarse_sweeps=1)


def test_sampled_profiling_steps():
    """With a profiling period P the library times the solve loops' passes at
    the steps k with k mod P < 4: four consecutive steps, so the stencil
    pass's two forms as often as in a whole solve, in every P; the byte
    accounting counts the same launches."""
    assert bench.PROFILE_WINDOW == 4
    ks = list(bench.timed_steps("fused_prec", [18], period=8))
    assert ks == [0, 1, 2, 3, 8, 9, 10, 11, 16, 17, 18]
    ks = list(bench.timed_steps("fused_spmv", [18, 7], period=8))
    assert ks == [0, 1, 2, 3, 8, 9, 10, 11, 16, 17] + [0, 1, 2, 3]
    assert list(bench.timed_steps("fused_prec", [10], period=1)) == list(range(11))
    n = 1 << 20
    totp, cntp = bench.pass_bytes("interleaved", "fused_spmv", [927], n, period=16)
    tot1, cnt1 = bench.pass_bytes("interleaved", "fused_spmv", [927], n)
    assert cntp == len([k for k in range(927) if k % 16 < 4])
    # one step in four of the sample applies the x updates, as in the whole
    # solve, so its mean is the whole solve's
    assert abs(totp / cntp - tot1 / cnt1) <= 0.01 * tot1 / cnt1
    pts = [8, 4, 2]
    t, c = bench.mg_pass_bytes(pts, [9], period=8)
    assert c == len([k for k in range(10) if k % 8 < 4])
