"""pa_kv_append on the GPU: the whole pool after the append equals the oracle's scatter, bit for
bit; padding slots and slots outside the pool leave everything untouched."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import Dev, host_bits
from workloads.generate import Spec

pytestmark = pytest.mark.gpu


def _check_pool(dev, k_ref, v_ref):
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(dev.k_cache), k_ref)
    assert np.array_equal(host_bits(dev.v_cache), v_ref)


@pytest.mark.parametrize("kv_dtype,q_dtype,D", [("bf16", "bf16", 64), ("f16", "f16", 128),
                                                 ("fp8_e4m3", "bf16", 128), ("bf16", "bf16", 128)])
def test_append_matches_oracle_scatter(kv_dtype, q_dtype, D):
    spec = Spec("app", 6, 8, 4, D, q_dtype, kv_dtype, ("list", (1, 16, 17, 32, 33, 300)),
                pool=("times", 3), seed=21)
    wl = workloads.make(spec)
    dev = Dev(wl)
    dev.append()
    k_ref, v_ref = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, wl.slot_mapping)
    _check_pool(dev, k_ref, v_ref)


def test_append_skips_padding_and_out_of_pool_slots():
    wl = workloads.make(Spec("app2", 4, 4, 2, 64, "bf16", "bf16", ("list", (5, 20, 40, 3)),
                             pool=("times", 2), seed=22))
    slots = wl.slot_mapping.copy()
    slots[1] = -1
    slots[3] = wl.num_blocks * 16 + 7        # outside the pool: skipped by the kernel
    dev = Dev(wl)
    dev.slots = torch.from_numpy(slots).cuda()
    dev.append()
    valid = slots.copy()
    valid[3] = -1
    k_ref, v_ref = oracle.kv_append(wl.k_cache, wl.v_cache, wl.k_new, wl.v_new, valid)
    _check_pool(dev, k_ref, v_ref)
