"""Whole steps captured into a HIP graph and replayed (pa_graph_*, StepGraph).

A decode step of a model runs the attention of every layer; each call is a launch with its own
fixed cost (design.babushkai.com "GPU推論の内部構造": per-launch overhead of decode steps and graphs
as the remedy).  These tests capture steps of several layers, replay them several times with
eager work in between, and check every replay bitwise against the same calls run eagerly, and the
caches against the oracle's append."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_31_amd as pa
import workloads
from gpu_util import assert_close, dev_bits, host_bits
from workloads.generate import Spec

pytestmark = pytest.mark.gpu


class Layer:
    """One attention layer's cache, query rows and new K/V, on the device."""

    def __init__(self, spec, seed):
        self.wl = wl = workloads.make(spec, seed=seed)
        s = spec
        self.q = dev_bits(wl.q, s.q_dtype)
        self.k = dev_bits(wl.k_cache, s.kv_dtype)
        self.v = dev_bits(wl.v_cache, s.kv_dtype)
        self.k_new = dev_bits(wl.k_new, s.kv_dtype)
        self.v_new = dev_bits(wl.v_new, s.kv_dtype)
        self.tables = torch.from_numpy(wl.block_tables).cuda()
        self.lens = torch.from_numpy(wl.context_lens).cuda()
        self.ks = None if wl.k_scale is None else torch.from_numpy(wl.k_scale).cuda()
        self.vs = None if wl.v_scale is None else torch.from_numpy(wl.v_scale).cuda()
        self.out = torch.empty_like(self.q)

    def call(self, stream, shared=False):
        wl = self.wl
        return pa.DecodeCall(self.q, self.k, self.v, self.tables, self.lens, float(wl.scale),
                             self.out, k_scale=self.ks, v_scale=self.vs,
                             max_context_len=wl.max_context_len, shared_prefixes=shared,
                             k_new=self.k_new, v_new=self.v_new, stream=stream,
                             workspace=pa.new_workspace(
                                 pa.pa_decode_workspace_size(pa.decode_desc(
                                     self.q, self.k, self.tables, wl.max_context_len, 0, shared)),
                                 self.q.device))


SPECS = [
    Spec("g_mha", 6, 8, 8, 128, "f16", "f16", ("list", (1, 17, 300, 2048, 33, 900)), seed=1),
    Spec("g_gqa", 5, 16, 2, 128, "bf16", "bf16", ("list", (64, 5, 1500, 700, 16)), seed=2),
    Spec("g_fp8", 3, 8, 2, 64, "bf16", "fp8_e4m3", ("list", (1000, 2, 4097)), seed=3),
    Spec("g_share", 8, 8, 2, 128, "bf16", "bf16", ("uniform", 20, 600), prefix=(4, 256), seed=4),
]


def test_multi_layer_step_replays_bitwise():
    stream = torch.cuda.Stream()
    layers = [Layer(SPECS[i % len(SPECS)], seed=200 + i) for i in range(6)]
    with torch.cuda.stream(stream):
        calls = [ly.call(stream, shared=ly.wl.spec.prefix is not None) for ly in layers]
        for c in calls:                                  # eager: warm-up and reference
            c()
    stream.synchronize()
    ref_out = [host_bits(ly.out) for ly in layers]
    ref_k = [host_bits(ly.k) for ly in layers]
    for ly, o in zip(layers, ref_out):                   # the eager step itself is right
        k, v = oracle.kv_append(ly.wl.k_cache, ly.wl.v_cache, ly.wl.k_new, ly.wl.v_new,
                                ly.wl.slot_mapping)
        assert np.array_equal(host_bits(ly.k), k) and np.array_equal(host_bits(ly.v), v)
        s = ly.wl.spec
        ref = oracle.decode(ly.wl.q, k, v, ly.wl.block_tables, ly.wl.context_lens, ly.wl.scale,
                            s.q_dtype, s.kv_dtype, ly.wl.k_scale, ly.wl.v_scale)
        # the layers hold contexts of 1, 2 and 5 tokens (counted rounding-limited relief)
        assert_close(o, ref, s.q_dtype, f"eager {s.name}", relief=True)

    graph = pa.StepGraph(calls, stream)
    for rep in range(3):
        with torch.cuda.stream(stream):
            for ly in layers:                            # eager work between replays
                ly.out.zero_()
        graph()
        stream.synchronize()
        for i, ly in enumerate(layers):
            assert np.array_equal(host_bits(ly.out), ref_out[i]), f"replay {rep} layer {i}"
            assert np.array_equal(host_bits(ly.k), ref_k[i]), f"replay {rep} layer {i} cache"


def test_replay_reads_buffers_updated_in_place():
    """A later step runs by writing new queries and new-token rows into the same buffers."""
    stream = torch.cuda.Stream()
    layers = [Layer(SPECS[1], seed=210 + i) for i in range(3)]
    with torch.cuda.stream(stream):
        calls = [ly.call(stream) for ly in layers]
        for c in calls:
            c()
    stream.synchronize()
    graph = pa.StepGraph(calls, stream)
    g = torch.Generator(device="cuda").manual_seed(7)
    for rep in range(3):
        with torch.cuda.stream(stream):
            for ly in layers:
                ly.q.copy_(torch.randn(ly.q.shape, generator=g, device="cuda").to(ly.q.dtype))
                ly.v_new.copy_(torch.randn(ly.v_new.shape, generator=g, device="cuda")
                               .to(ly.v_new.dtype))
        graph()
        stream.synchronize()
        got = [host_bits(ly.out) for ly in layers]
        with torch.cuda.stream(stream):
            for c in calls:                              # the same step eagerly
                c()
        stream.synchronize()
        for i, ly in enumerate(layers):
            assert np.array_equal(got[i], host_bits(ly.out)), f"replay {rep} layer {i}"


def test_graph_of_mixed_entry_points():
    """Quantising append, multi-query attention (two kernels with its key partitions) and a plain
    append in one captured step."""
    stream = torch.cuda.Stream()
    rng = np.random.default_rng(220)
    spec = Spec("g_mix", 4, 8, 2, 128, "bf16", "fp8_e4m3", ("list", (40, 300, 1000, 7)), seed=5)
    wl = workloads.make(spec, poison=False)
    kc, vc = dev_bits(wl.k_cache, "fp8_e4m3"), dev_bits(wl.v_cache, "fp8_e4m3")
    ks, vs = torch.from_numpy(wl.k_scale).cuda(), torch.from_numpy(wl.v_scale).cuda()
    T = np.minimum(wl.context_lens, 3)
    qs = np.concatenate([[0], np.cumsum(T)]).astype(np.int32)
    N = int(qs[-1])
    slots = []
    for b in range(spec.batch):
        pos = wl.context_lens[b] - T[b] + np.arange(T[b])
        slots.extend(wl.block_tables[b, pos // 16].astype(np.int64) * 16 + pos % 16)
    slots = torch.tensor(slots, dtype=torch.int64, device="cuda")
    k16 = torch.from_numpy(rng.standard_normal((N, 2, 128)).astype(np.float32)).cuda().bfloat16()
    v16 = torch.from_numpy(rng.standard_normal((N, 2, 128)).astype(np.float32)).cuda().bfloat16()
    q = dev_bits(workloads.storage_bits(rng.standard_normal((N, 8, 128)), "bf16"), "bf16")
    out = torch.empty_like(q)
    qs_d = torch.from_numpy(qs).cuda()
    tables, lens = torch.from_numpy(wl.block_tables).cuda(), torch.from_numpy(wl.context_lens).cuda()

    class Quant:
        def __call__(self):
            pa.pa_kv_append_quant(k16, v16, slots, kc, vc, ks, vs, first_token_scale=True,
                                  stream=stream)

    multi = pa.MultiCall(q, qs_d, kc, vc, tables, lens, float(wl.scale), out, 3, k_scale=ks,
                         v_scale=vs, partition_tokens=64, stream=stream)
    calls = [Quant(), multi]
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    stream.synchronize()
    ref = [host_bits(t) for t in (out, kc, vc)] + [ks.cpu().numpy(), vs.cpu().numpy()]
    graph = pa.StepGraph(calls, stream)
    for rep in range(3):
        with torch.cuda.stream(stream):
            out.zero_()
        graph()
        stream.synchronize()
        got = [host_bits(t) for t in (out, kc, vc)] + [ks.cpu().numpy(), vs.cpu().numpy()]
        for name, g_, r_ in zip(("out", "k", "v", "k_scale", "v_scale"), got, ref):
            assert np.array_equal(g_, r_), f"replay {rep}: {name}"
