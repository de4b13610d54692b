"""The kernels' 16-bit arithmetic against the oracle on every finite value:
each fp16 / bf16 bit pattern x0 (NaN and infinity excluded) meets a partner
x1 chosen so that the fp32 result of one hop lands exactly halfway between
two neighbouring 16-bit values (x1 = +-half a unit in the last place of
x0, both tie directions), just past halfway, in the subnormal range (x0 and
x1 both subnormal), or beyond the largest finite value.  With two ranks
every element is one hop, op(received, local), rounded once to nearest even,
so this pins the rounding (ties to even, subnormals kept, overflow to
infinity) of whatever instruction the kernel uses for it, under every op
and all three protocols.
"""
import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_reduce_amd as ra
from ring_allreduce_reduce_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")

# exponent bits, mantissa bits, exponent bias of the two formats
FMT = {"float16": (5, 10, 15), "bfloat16": (8, 7, 127)}


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _finite_patterns(dtype):
    ebits, mbits, _ = FMT[dtype]
    p = np.arange(1 << 16, dtype=np.uint32)
    exp = (p >> mbits) & ((1 << ebits) - 1)
    return p[exp != (1 << ebits) - 1].astype(np.uint16)


def _half_ulp_bits(dtype, x):
    """Bit pattern of +half a unit in the last place of each |x| (a power of
    two, or the smallest subnormal where half an ulp is below it)."""
    ebits, mbits, bias = FMT[dtype]
    exp = (x.astype(np.int32) >> mbits) & ((1 << ebits) - 1)
    e = np.maximum(exp, 1)                # subnormals share the ulp of exponent 1
    h = e - mbits - 1                     # biased exponent of half an ulp
    out = np.where(h >= 1, (h << mbits), 1 << np.clip(h + mbits - 1, 0, mbits - 1))
    return out.astype(np.uint16)


def _partners(dtype, x, rng):
    ebits, mbits, _ = FMT[dtype]
    half = _half_ulp_bits(dtype, x)
    sign = np.uint16(0x8000)
    cases = [
        half,                                      # exact tie, same sign as a positive x0
        half | sign,                               # exact tie the other way
        (half + 1).astype(np.uint16),              # just past halfway
        (rng.integers(0, 1 << mbits, x.size) | (rng.integers(0, 2, x.size) << 15)).astype(np.uint16),  # subnormal
        (((1 << ebits) - 2) << mbits | ((1 << mbits) - 1)) * np.ones(x.size, np.uint16),  # largest finite
    ]
    return cases


@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
@pytest.mark.parametrize("proto", ["Simple", "LL", "LL128"])
def test_one_hop_rounding_on_every_finite_value(dtype, proto):
    rng = np.random.default_rng(7)
    x = _finite_patterns(dtype)
    for k, partner in enumerate(_partners(dtype, x, rng)):
        for op in ("sum", "prod", "min", "max", "avg"):
            xs = [x.copy(), partner.copy()]
            if k == 3:
                # subnormal with subnormal: sums and differences stay subnormal or near
                xs[0] = (x & np.uint16(0x8000 | ((1 << FMT[dtype][1]) - 1))).astype(np.uint16)
            xs = [a.view(W.STORAGE[dtype]) for a in xs]     # bit patterns as the storage type
            print(f"case rounding {dtype} {proto} partner {k} {op}", flush=True)
            sends = [W.to_torch(a, dtype, DEV) for a in xs]
            recvs = [torch.zeros_like(s) for s in sends]
            ra.allreduce(sends, recvs, op=op, nchannels=4, proto=proto)
            torch.cuda.synchronize()
            code = ra.ringar_get_async_error(torch.cuda.current_stream().cuda_stream)
            assert code == 0, ra.ringar_result_string(code)
            plan = ra.ringar_plan(x.size, dtype, 2, 4, proto)
            want = oracle.ring_allreduce(xs, dtype, op, plan.nchannels, plan.chunk_elems)
            for r in range(2):
                got = W.from_torch(recvs[r], dtype)
                bad = np.flatnonzero(got.view(np.uint16) != want[r].view(np.uint16))
                assert bad.size == 0, (dtype, proto, k, op, r, bad[:4], xs[0][bad[:4]], xs[1][bad[:4]],
                                       got.view(np.uint16)[bad[:4]], want[r].view(np.uint16)[bad[:4]])
