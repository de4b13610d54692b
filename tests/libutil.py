"""Shared helpers of the library tests: build-on-demand and model fixtures."""
import json
import os

import ring_allreduce_reduce_amd as ra
from oracle import select as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def lib():
    if not os.path.exists(ra.LIB_PATH):
        from ring_allreduce_reduce_amd import _build
        _build.build()
    return ra.load()


def golden_model_dict():
    with open(os.path.join(GOLDEN, "mi355x_model.json")) as f:
        return {k: v for k, v in json.load(f).items() if not k.startswith("_")}


def oracle_model(d=None) -> S.RingModel:
    d = d or golden_model_dict()
    return S.RingModel(bw_per_channel=d["bw_per_channel"], ll_max_bw=d["ll_max_bw"],
                       ll128_per_channel_max_bw=d["ll128_per_channel_max_bw"], eff=tuple(d["eff"]),
                       base_lat=tuple(d["base_lat_us"]), hw_lat=tuple(d["hw_lat_us"]),
                       max_channels=d["max_channels"], max_pairs=d["max_pairs"],
                       threads=tuple(d["threads"]), thread_threshold=tuple(d["thread_threshold"]),
                       default_chunk_bytes=tuple(d["default_chunk_bytes"]))


def lib_model(d) -> "ra.ringar_model_t":
    return ra.model_from_dict(d)


def oracle_tree_model(d, nranks) -> S.TreeModel:
    """The library's Tree rows as the oracle's model: every virtual rank one
    vertex (n_nodes = n, one rank per node), the per-level latency as the
    inter-node step."""
    return S.TreeModel(bw_per_channel=d["bw_per_channel"], per_channel_max_bw=d["tree_per_channel_max_bw"],
                       ll_max_bw=d["ll_max_bw"], per_channel_max_ll128_bw=d["tree_ll128_per_channel_max_bw"],
                       allreduce_eff=d["tree_allreduce_eff"], ll_divisor=d["tree_ll_divisor"],
                       n_nodes=nranks, ranks_per_node=1, base_lat=tuple(d["tree_base_lat_us"]),
                       intra_lat=(0.0, 0.0, 0.0), inter_lat=tuple(d["tree_hw_lat_us"]),
                       correction=bool(d["tree_correction"]), ll128_factor=d["tree_ll128_factor"])
