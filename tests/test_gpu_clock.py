"""The clock probe (a measurement aid next to the attention calls): every
workgroup reports engine cycles and 100 MHz real-time ticks over its spin,
the ticks cover the requested spin, and the implied clock lies within the
MI355X's engine-clock range (at most 2.4 GHz, plus margin for rounding)."""
import pytest

gpu = pytest.mark.gpu


@gpu
def test_clock_probe_reports_a_plausible_clock():
    import torch
    import packed_sequence_attention_amd as bd
    dev = torch.device("cuda:0")
    out = torch.full((2 * 32,), -1, dtype=torch.int64, device=dev)
    bd.clock_probe(out, ticks=2000)
    torch.cuda.synchronize()
    c = out.view(-1, 2).cpu()
    assert bool((c[:, 1] >= 2000).all()) and bool((c[:, 1] < 2000 + 100000).all())
    mhz = c[:, 0].double() / c[:, 1].double() * 100.0
    assert bool((mhz > 50).all()) and bool((mhz < 2600).all()), mhz.tolist()
