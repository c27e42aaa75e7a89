"""The placement check (pa_placement_check) on the device: it runs, reports
the device's compute units, and its fractions are fractions.  The fractions
themselves depend on the hardware's dispatcher and on other work sharing the
device, so they are reported by the benchmark, not asserted here."""
import pytest
import torch

pytestmark = pytest.mark.gpu


def test_placement_check_runs():
    from paged_kv_cache_pool_amd import binding as B
    r = B.placement_check()
    print(r, flush=True)
    assert r["compute_units"] == torch.cuda.get_device_properties(0).multi_processor_count
    assert 1 <= r["xcds"] <= 16
    for k in ("one_wave_alone", "two_wave_paired", "xcd_round_robin"):
        assert 0.0 <= r[k] <= 1.0, (k, r[k])
