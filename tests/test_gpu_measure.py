"""The measurement entry points (qmoe_stream_read, qmoe_wave_latency) run and
report sane values; they feed the bench line's ceiling and latency sections."""
import pytest
import torch

from decode_moe_mul_amd import qmoe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,bpc", [(1 << 16, 4), ((1 << 23) + 148, 2), ((1 << 23) + 148, 16)])
def test_stream_read_runs_and_writes_at_most_the_sink(n, bpc):
    """Sizes below one step per block (all of it read grid-stride) and with
    whole per-block chunks plus a remainder."""
    buf = torch.arange(n, dtype=torch.int32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    qmoe.stream_read(buf, bpc, sink)
    torch.cuda.synchronize()
    assert (sink[1:] == 0).all()


def test_wave_latency_values_are_sane():
    lat = qmoe.wave_latency()
    print(lat)
    assert 500 <= lat["shader_clock_mhz"] <= 5000
    assert 1 <= lat["valu_dependent_cycles"] <= lat["dpp_wave_max_cycles"]
    assert 1 <= lat["ballot_round_trip_cycles"] < 10000
    # ten rounds of at least a wave max each, plus the sort
    assert lat["wave_topk_512_k10_cycles"] >= 10 * lat["dpp_wave_max_cycles"]
    assert 1 <= lat["lane_sort_8_cycles"] < lat["wave_topk_512_k10_cycles"]
