"""GPU checks of the measurement probes: they run, leave the sink alone, and
take time that grows with their work (a probe whose loads or MFMAs were
optimized away would not)."""
import pytest
import torch

from tests.helpers import say

pytestmark = pytest.mark.gpu


def _q8():
    import q8_quantized_matmul_amd as q8
    return q8


def _time_us(fn, reps=5):
    fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1000.0 / reps


def test_probe_read_runs_and_scales():
    q8 = _q8()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    small = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    big = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
    t_small = _time_us(lambda: q8.q8_0_probe_read(small, sink))
    t_big = _time_us(lambda: q8.q8_0_probe_read(big, sink))
    say(f"[probe] read 1 MiB {t_small:.1f} us, 512 MiB {t_big:.1f} us "
        f"({(512 << 20) / t_big / 1e3:.0f} GB/s)")
    assert int(sink.item()) == 0
    assert t_big > 4 * t_small
    # A ragged size (not a multiple of the per-workgroup chunk) stays in bounds.
    q8.q8_0_probe_read(big[: (3 << 20) + 48], sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_probe_mfma_runs_and_scales():
    q8 = _q8()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    t1 = _time_us(lambda: q8.q8_0_probe_mfma_i8(100, sink))
    t8 = _time_us(lambda: q8.q8_0_probe_mfma_i8(800, sink))
    tops = q8.PROBE_MFMA_OPS_PER_ITER * 800 / (t8 * 1e-6) / 1e12
    say(f"[probe] mfma 100 rounds {t1:.1f} us, 800 rounds {t8:.1f} us ({tops:.0f} TOPS)")
    assert int(sink.item()) == 0
    assert t8 > 4 * t1


@pytest.mark.parametrize("mix", [0, 1, 2])
def test_probe_mfma_mix_runs_and_scales(mix):
    q8 = _q8()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    t1 = _time_us(lambda: q8.q8_0_probe_mfma_mix(100, mix, sink))
    t8 = _time_us(lambda: q8.q8_0_probe_mfma_mix(800, mix, sink))
    tops = q8.PROBE_MFMA_OPS_PER_ITER * 800 / (t8 * 1e-6) / 1e12
    say(f"[probe] mix {mix}: 100 rounds {t1:.1f} us, 800 rounds {t8:.1f} us ({tops:.0f} TOPS of int8 work)")
    assert int(sink.item()) == 0
    assert t8 > 4 * t1



def test_probe_launch_runs():
    """The empty launch leaves the sink alone and costs far less than a
    launch that streams memory (it is the fixed part of every launch)."""
    q8 = _q8()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    big = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    t_empty = _time_us(lambda: q8.q8_0_probe_launch(1024, sink), reps=50)
    t_read = _time_us(lambda: q8.q8_0_probe_read(big, sink), reps=20)
    say(f"[probe] empty launch {t_empty:.2f} us, 64 MiB read {t_read:.1f} us")
    assert int(sink.item()) == 0
    assert t_empty < t_read
