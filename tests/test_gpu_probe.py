"""The benchmark's measurement probes (libq8probe.so) run to completion: the
read probe over a buffer for every offered load depth (it writes nothing for
these buffers), the int8 matrix-core and exact-fold probes, and the grid-barrier probe, whose
rounds all complete on every workgroup (no timeout flagged) and whose
consecutive calls continue from the epochs the previous call left."""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from int8_weight_streaming_amd import probe as q8probe
    q8probe.load()
    return q8probe


@pytest.mark.parametrize("lpt", [4, 8, 12, 16])
def test_read_probe_runs(probe, lpt):
    log(f"read probe lpt={lpt}")
    buf = torch.arange(1 << 22, dtype=torch.int32, device=DEV)        # 16 MiB
    s = probe.sink(DEV)
    probe.read(buf, lpt, s)
    probe.read(buf[: (1 << 22) - 20], lpt, s)                         # ragged last span
    torch.cuda.synchronize()
    assert int(s.abs().sum().item()) == 0


def test_mfma_probe_runs(probe):
    s = probe.sink(DEV)
    ops = probe.mfma_i8(16, 100, s)
    torch.cuda.synchronize()
    assert ops == 16 * 4 * 100 * 8 * 65536
    assert int(s.abs().sum().item()) == 0


def test_fold_probe_runs(probe):
    s = probe.sink(DEV)
    ops = probe.fold(16, 100, s)
    torch.cuda.synchronize()
    assert ops == 16 * 4 * 100 * 4 * 65536
    assert int(s.abs().sum().item()) == 0


def test_barrier_probe_completes(probe):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    flags = probe.barrier_flags(DEV)
    for g in sorted({1, 64, min(256, cus), cus}):
        log(f"barrier probe workgroups={g}")
        flags.zero_()
        probe.barrier(flags, g, 50)
        probe.barrier(flags, g, 25)
        probe.barrier(flags, g, 0)
        torch.cuda.synchronize()
        f = flags.cpu().numpy()
        assert f[-1] == 0, f"barrier timed out with {g} workgroups"
        for r in range(8):
            assert np.all(f[r * 1024: r * 1024 + g] == 75), (g, r)
