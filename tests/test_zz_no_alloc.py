"""pa_decode_noalloc (the static-scratch variant of pa_decode for callers that cannot allocate)
against pa_decode through the C ABI: two calls in a row on one GPU's scratch, the second with a
smaller batch, each bitwise equal to pa_decode with its own workspace and within the stated
tolerance of the fp64 oracle; then a shared-prefix planning call and a reusing call."""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_31_amd as pa
import workloads
from gpu_util import Dev, assert_close, host_bits, oracle_after_append
from workloads.generate import Spec

pytestmark = pytest.mark.gpu


def _noalloc(dev, shared=0):
    """pa_decode_noalloc through the C ABI, on the current stream."""
    wl = dev.wl

    def p(t):
        return None if t is None else ctypes.c_void_p(t.data_ptr())
    desc = pa.decode_desc(dev.q, dev.k_cache, dev.tables, wl.max_context_len,
                          wl.spec.partition_tokens, shared)
    out = torch.empty_like(dev.q)
    st = pa.lib().pa_decode_noalloc(ctypes.byref(desc), p(dev.q), p(dev.k_cache), p(dev.v_cache),
                                    p(dev.k_scale), p(dev.v_scale), p(dev.tables), p(dev.lens),
                                    ctypes.c_float(float(wl.scale)), p(out),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == pa.PA_OK, pa.status_string(st)
    torch.cuda.synchronize()
    return host_bits(out)


def test_noalloc_equals_pa_decode_on_two_calls_the_second_smaller():
    specs = [
        Spec("noalloc_a", 24, 32, 4, 128, "bf16", "bf16", ("uniform", 1, 3000),
             pool=("times", 2), seed=301),
        Spec("noalloc_b", 5, 16, 2, 64, "bf16", "fp8_e4m3", ("list", (700, 1, 33, 129, 2)),
             pool=("times", 2), seed=302),
    ]
    for spec in specs:
        wl = workloads.make(spec)
        dev = Dev(wl)
        dev.append()
        torch.cuda.synchronize()
        got = _noalloc(dev)
        want = dev.decode()                       # pa_decode with the binding's workspace
        assert np.array_equal(got, want), spec.name
        ref, _, _ = oracle_after_append(wl)
        # the smaller batch holds a 1-token context of an fp8 cache (counted rounding-limited)
        assert_close(got, ref, spec.q_dtype, f"noalloc {spec.name}",
                     relief=spec.kv_dtype == "fp8_e4m3")


def test_noalloc_with_shared_prefixes_plans_and_reuses():
    spec = Spec("noalloc_share", 12, 16, 2, 128, "bf16", "bf16", ("lognormal", 100.0, 1.0, 3000),
                prefix=(4, 256), pool=("times", 2), seed=303)
    wl = workloads.make(spec)
    dev = Dev(wl)
    dev.append()
    torch.cuda.synchronize()
    planned = _noalloc(dev, shared=1)
    reused = _noalloc(dev, shared=2)
    assert np.array_equal(planned, reused)
    assert np.array_equal(planned, dev.decode(shared_prefixes=True))
    ref, _, _ = oracle_after_append(wl)
    assert_close(planned, ref, "bf16", "noalloc shared prefixes")
