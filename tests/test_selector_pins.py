"""Pins of the oracle's alpha-beta model against the tables printed on the
pages (CPU only).  See tests/golden/tuning_tables.json for the citations."""
import json
import os

import pytest

from oracle import select as S

with open(os.path.join(os.path.dirname(__file__), "golden", "tuning_tables.json")) as f:
    G = json.load(f)


def _model(m):
    c = G["constants"]
    return S.RingModel(bw_per_channel=m["bw_per_channel"], ll_max_bw=m["ll_max_bw"],
                       ll128_per_channel_max_bw=m["ll128_per_channel_max_bw"],
                       eff=tuple(c["eff_model"]), base_lat=tuple(c["base_lat"]),
                       hw_lat=tuple(c["hw_lat_nvlink"]))


def test_a100_ring_row():
    g = G["a100"]
    m = _model(g)
    for proto in ("Simple", "LL128"):
        lat, bw = g["printed"][proto]
        assert S.ring_latency(m, g["nranks"], proto) == pytest.approx(lat, abs=0.05)
        assert S.ring_alg_bw(m, g["nranks"], g["nchannels"], proto) == pytest.approx(bw, abs=0.05)
    # LL: the bandwidth matches the page; the latency printed there (22.4) does
    # not follow from the page's own constants (6.6 + 14 x 0.6 = 15.0).
    assert S.ring_alg_bw(m, g["nranks"], g["nchannels"], "LL") == pytest.approx(g["printed"]["LL"][1], abs=0.05)
    assert S.ring_latency(m, g["nranks"], "LL") == pytest.approx(g["ll_latency_from_constants"], abs=1e-9)


def test_h100_machine_one():
    g = G["h100"]
    m = _model(g)
    for proto, bw in g["printed_bw"].items():
        assert S.ring_alg_bw(m, g["nranks"], g["nchannels"], proto) == pytest.approx(bw, abs=0.5)
    for proto in ("Simple", "LL128"):
        assert S.ring_latency(m, g["nranks"], proto) == pytest.approx(g["printed_lat"][proto], abs=0.05)


def test_machine_two_crossover():
    g = G["machine_two"]
    m = _model(g)
    bws = {p: S.ring_alg_bw(m, g["nranks"], g["nchannels"], p) for p in ("Simple", "LL128")}
    for p, bw in g["printed_bw"].items():
        assert bws[p] == pytest.approx(bw, abs=0.5)
    lat_s = S.ring_latency(m, g["nranks"], "Simple")
    lat_l = S.ring_latency(m, g["nranks"], "LL128")
    # with the page's rounded bandwidths the crossover is the printed 4.3 MB
    s_rounded = S.crossover_bytes(lat_l, g["printed_bw"]["LL128"], lat_s, g["printed_bw"]["Simple"])
    assert s_rounded / 1e6 == pytest.approx(g["printed_crossover_mb"], abs=0.05)
    # the model's own choice flips there too
    s_exact = S.crossover_bytes(lat_l, bws["LL128"], lat_s, bws["Simple"])
    assert 4.1e6 < s_exact < 4.4e6
    sel_small, _ = S.select(m, g["nranks"], g["nchannels"], int(s_exact * 0.9), enabled=("LL128", "Simple"))
    sel_big, _ = S.select(m, g["nranks"], g["nchannels"], int(s_exact * 1.1), enabled=("LL128", "Simple"))
    assert (sel_small, sel_big) == ("LL128", "Simple")


def test_ll_vs_nvls_crossover_formula():
    g = G["nvls_crossover"]
    s = S.crossover_bytes(g["ll_lat"], g["ll_bw"], g["nvls_lat"], g["nvls_bw"])
    assert s / 1e3 == pytest.approx(g["printed_kb"], rel=0.02)


def test_channel_shrink_rule():
    g = G["channel_rule"]
    m = S.RingModel(bw_per_channel=1, ll_max_bw=1, ll128_per_channel_max_bw=1,
                    threads=(512, 640, g["threads"]), thread_threshold=(8, 8, g["threshold"]),
                    max_channels=64, max_pairs=1 << 20)
    for nbytes, nch in g["cases"]:
        assert S.auto_channels(m, 8, "Simple", nbytes) == nch


def test_selection_is_argmin_with_simple_winning_ties():
    m = _model(G["a100"])
    n, nch = 8, 24
    for nbytes in [8, 1 << 10, 1 << 16, 1 << 20, 1 << 24, 1 << 30]:
        best, times = S.select(m, n, nch, nbytes)
        assert times[S.PROTOS.index(best)] == min(times)
    # identical models for all three protocols: the tie goes to Simple
    flat = S.RingModel(bw_per_channel=10, ll_max_bw=1e9, ll128_per_channel_max_bw=1e9,
                       eff=(1.0, 1.0, 1.0), base_lat=(5, 5, 5), hw_lat=(1, 1, 1))
    assert S.select(flat, 8, 4, 12345)[0] == "Simple"
    flat2 = S.RingModel(bw_per_channel=10, ll_max_bw=1e9, ll128_per_channel_max_bw=1e9,
                        eff=(1.0, 1.0, 0.5), base_lat=(5, 5, 5), hw_lat=(1, 1, 1))
    assert S.select(flat2, 8, 4, 12345)[0] == "LL128"
    with pytest.raises(ValueError):
        S.select(m, n, nch, 100, enabled=())
