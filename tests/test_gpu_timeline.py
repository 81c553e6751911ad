"""GPU tests of the stamped launch (qmv_affine_timeline, a measurement aid; 4-bit
group-64 and 2-bit group-128 codes):
its output equals the product launch's bit for bit, it keeps the product's
launch shape and residency, and every wavefront of the grid writes ordered
stamps from a plausible place on the chip.  Cases: the 12B- and 27B-class
projection shapes at one and thirteen vectors (whole K and K windows), a
ragged shape with rows past N, and every rows-per-wavefront choice."""
import pytest
import torch

import gpu_util as U
from inputs import gen

pytestmark = pytest.mark.gpu

CASES = [
    # workload or (N, K), M, rows per wavefront (0 = the library's choice)
    ("up_4b_15360x3840", 1, 0),
    ("up_4b_15360x3840", 13, 0),
    ("down_4b_3840x15360", 1, 0),
    ("down_4b_3840x15360", 13, 0),   # K windows
    ("up_4b_17408x5120", 2, 0),
    ("down_4b_5120x17408", 1, 0),     # three rows per wavefront
    ((1000, 1984), 3, 0),             # 31 groups per row, rows past N in the last block
    ((777, 2240), 5, 1),
    ((777, 2240), 5, 2),
    ((777, 2240), 5, 3),
    ((777, 2240), 5, 4),
    ("up_2b_15360x3840", 1, 0),
    ("up_2b_15360x3840", 13, 0),
    ((513, 2176, 2), 3, 1),           # 2-bit, 17 groups of 128, one row per wavefront
]


def _problem(spec):
    if isinstance(spec, str):
        return gen.make_problem(spec)
    N, K, bits = spec if len(spec) == 3 else (*spec, 4)
    return gen.make_problem(N=N, K=K, bits=bits, gs=64 if bits == 4 else 128, sb="bf16",
                            x_dtype="bf16", seed=N + K)


@pytest.mark.parametrize("spec,M,R", CASES)
def test_timeline_matches_the_product_launch(spec, M, R):
    p = _problem(spec)
    label = f"{spec} M={M} R={R}"
    U.say(label)
    w, s, b, x = U.to_dev(p)
    xm = x[:M].contiguous()
    y = U.q.affine(w, s, b, xm, bits=p.bits, group_size=p.gs, out_dtype=torch.float32, rows_per_wave=R)
    yt, stamps, info = U.q.timeline(w, s, b, xm, bits=p.bits, group_size=p.gs, rows_per_wave=R,
                                    out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int32), yt.view(torch.int32)), label

    kinf = U.q.kernel_info(M, p.N, p.K, p.bits, p.gs, rows_per_wave=R)
    assert info["grid"] == kinf["grid"] and info["wg_size"] == kinf["wg_size"], (info, kinf)
    assert info["waves"] == kinf["grid"] * kinf["wg_size"] // 64
    # the stamps change nothing of the launch's residency
    assert info["blocks_per_cu"] == info["product_blocks_per_cu"] > 0, info
    assert info["clock_khz"] > 0

    a = stamps.cpu()
    t = a[:, :3]
    assert bool((t[:, 0] > 0).all()), f"{label}: a wavefront wrote no stamps"
    assert bool((t[:, 1:] >= t[:, :-1]).all()), f"{label}: stamps out of order"
    span_ms = float(t[:, 2].max() - t[:, 0].min()) / info["clock_khz"]
    assert 0 < span_ms < 100, f"{label}: launch spans {span_ms} ms"
    xcc = a[:, 3] >> 32
    assert bool((xcc >= 0).all() and (xcc < 8).all()), f"{label}: XCC ids {xcc.unique()}"
    cus = torch.unique(xcc * 256 + ((a[:, 3] >> 8) & 0xFF)).numel()
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert 1 <= cus <= n_cu, (cus, n_cu)


def test_timeline_query_only():
    # no stamps buffer: the call fills the launch's fields and launches nothing
    p = gen.make_problem(N=300, K=1152, bits=4, gs=64, sb="bf16", x_dtype="bf16", seed=7)
    w, s, b, x = U.to_dev(p)
    y = torch.full((2, p.N), 7.0, dtype=torch.float32, device=U.DEV)
    info = U.q.TimelineInfo()
    st = U.q.timeline_ptr(w.data_ptr(), s.data_ptr(), b.data_ptr(), x.data_ptr(), y.data_ptr(),
                          2, p.N, p.K, 4, 64, U.q.DT_F32, 0, None, 0, info)
    torch.cuda.synchronize()
    assert st == 0 and info.waves > 0
    assert bool((y == 7.0).all())
    # too small a stamps buffer is refused before the launch
    stamps = torch.zeros(info.waves * U.q.STAMPS - 1, dtype=torch.int64, device=U.DEV)
    st = U.q.timeline_ptr(w.data_ptr(), s.data_ptr(), b.data_ptr(), x.data_ptr(), y.data_ptr(),
                          2, p.N, p.K, 4, 64, U.q.DT_F32, 0, stamps.data_ptr(), stamps.numel(), info)
    torch.cuda.synchronize()
    assert st == 4 and bool((y == 7.0).all())
