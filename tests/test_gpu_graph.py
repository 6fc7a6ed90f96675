"""The decode step under HIP graph capture.

The calls of one decode step -- store the step's token and rotate the
queries (4-bit cache: one launch), decode, merge -- are captured in one
graph on torch's capture stream and replayed.  Every replay, each after eager work and a
synchronization, must reproduce the eager step's outputs bit for bit: the
library's kernels write every output element themselves and record no
memset, so a captured step is safe to replay.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from helpers import MlaCase, Q4Case, TqCase

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    assert torch.cuda.is_available(), "no GPU"
    import fp8_quantized_kv_amd as m
    return m


def _replays_match(step, outputs, replays=3):
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(replays):
        for t in outputs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, e in zip(outputs, ref):
            assert torch.equal(t, e), f"replay {r} differs from the eager step"
        step()  # eager work between replays
        torch.cuda.synchronize()
        for t, e in zip(outputs, ref):
            assert torch.equal(t, e), f"eager step after replay {r} differs"


def _last_slots(case):
    ps = case.w.page_size
    rows = [wl.slots_for(case.lay.page_table[b], np.array([T - 1]), ps) for b, T in enumerate(case.lens)]
    return torch.cat(rows).to("cuda")


@pytest.mark.parametrize("split_keys", [512, 2048])
def test_q4_step_replays_in_a_graph(kvq, split_keys):
    """Store + rotate + decode + merge over a ragged batch; 512-key splits run
    the wave-pair kernel, 2048-key splits the single-wave one."""
    w = wl.shrink(wl.RAGGED, prefill_chunk=0)
    lens = [3000, 700, 4500]
    case = Q4Case(w, lens, build_oracle=False)
    B, Hq, D = len(lens), w.n_q_heads, w.head_dim
    gen = torch.Generator(device="cuda").manual_seed(11)
    k_new = torch.randn((B, w.n_kv_heads, D), generator=gen, device="cuda").to(torch.bfloat16)
    v_new = torch.randn((B, w.n_kv_heads, D), generator=gen, device="cuda").to(torch.bfloat16)
    slots = _last_slots(case)
    acc_shape, mz_shape = kvq.partial_shapes(case.cache, B, Hq, case.max_seq_len, split_keys)
    f32 = dict(dtype=torch.float32, device="cuda")
    bufs = {"q_rot": torch.empty((B, Hq, D), **f32), "part_acc": torch.empty(acc_shape, **f32),
            "part_m": torch.empty(mz_shape, **f32), "part_z": torch.empty(mz_shape, **f32),
            "out": torch.empty((B, Hq, D), **f32), "lse": torch.empty((B, Hq), **f32)}

    def step():  # the store and the rotation in one launch
        kvq.decode_step(case.cache, case.q, case.page_table, case.seq_lens, case.max_seq_len, w.sm_scale,
                        split_keys, bufs, new_kv=(k_new, v_new, slots))

    _replays_match(step, [bufs["out"], bufs["lse"]])


def test_fp8_step_replays_in_a_graph(kvq):
    """Store + decode + merge over the fp8 latent cache, 40 heads, two sequences."""
    w = wl.shrink(wl.MLA_262K, n_layers=1, seq_len=0, n_heads=40)
    lens = [2500, 900]
    case = MlaCase(w, lens, build_oracle=False)
    B, H = len(lens), w.n_heads
    gen = torch.Generator(device="cuda").manual_seed(12)
    x_new = torch.randn((B, w.head_dim), generator=gen, device="cuda")
    slots = _last_slots(case)
    acc_shape, mz_shape = kvq.partial_shapes(case.cache, B, H, case.max_seq_len, 1024)
    f32 = dict(dtype=torch.float32, device="cuda")
    bufs = {"part_acc": torch.empty(acc_shape, **f32), "part_m": torch.empty(mz_shape, **f32),
            "part_z": torch.empty(mz_shape, **f32), "out": torch.empty((B, H, w.kv_lora), **f32),
            "lse": torch.empty((B, H), **f32)}

    def step():
        kvq.decode_step(case.cache, case.q, case.page_table, case.seq_lens, case.max_seq_len, w.sm_scale, 1024,
                        bufs, new_kv=(x_new, None, slots))

    _replays_match(step, [bufs["out"], bufs["lse"]])


def test_tq4_step_replays_in_a_graph(kvq):
    """Store + query rotation + decode (matrix cores) + merge and inverse
    rotation over the TQ4 latent cache, 40 heads, two sequences."""
    w = wl.shrink(wl.MLA_TQ4_262K, n_layers=1, seq_len=0, n_heads=40)
    lens = [2500, 900]
    case = TqCase(w, lens, build_oracle=False)
    B, H = len(lens), w.n_heads
    gen = torch.Generator(device="cuda").manual_seed(13)
    x_new = torch.randn((B, w.head_dim), generator=gen, device="cuda")
    slots = _last_slots(case)
    acc_shape, mz_shape = kvq.partial_shapes(case.cache, B, H, case.max_seq_len, 512)
    f32 = dict(dtype=torch.float32, device="cuda")
    bufs = {"q_rot": torch.empty((B, H, w.head_dim), **f32), "part_acc": torch.empty(acc_shape, **f32),
            "part_m": torch.empty(mz_shape, **f32), "part_z": torch.empty(mz_shape, **f32),
            "out": torch.empty((B, H, w.kv_lora), **f32), "lse": torch.empty((B, H), **f32)}

    def step():
        kvq.decode_step(case.cache, case.q, case.page_table, case.seq_lens, case.max_seq_len, w.sm_scale, 512,
                        bufs, new_kv=(x_new, None, slots))

    _replays_match(step, [bufs["out"], bufs["lse"]])


def test_drafted_rows_replay_in_a_graph(kvq):
    """Rotate + kvq_decode_attn_rows + merge for four drafted rows of one
    sequence (the row layout's 1-D grid) under capture."""
    w = wl.GQA_32K
    case = Q4Case(w, [3000], build_oracle=False)
    R, Hq, D = 4, w.n_q_heads, w.head_dim
    lens = torch.tensor([2997, 2998, 2999, 3000], dtype=torch.int32, device="cuda")
    q = wl.q4_query(wl.shrink(w, batch=R), 1, "cuda")
    row = case.page_table[0].contiguous()
    acc_shape, mz_shape = kvq.partial_shapes(case.cache, R, Hq, 3000, 2048)
    f32 = dict(dtype=torch.float32, device="cuda")
    q_rot = torch.empty((R, Hq, D), **f32)
    pa, pm, pz = torch.empty(acc_shape, **f32), torch.empty(mz_shape, **f32), torch.empty(mz_shape, **f32)
    out, lse = torch.empty((R, Hq, D), **f32), torch.empty((R, Hq), **f32)

    def step():
        kvq.kvq_rotate_q(q, out=q_rot)
        kvq.kvq_decode_attn_rows(case.cache, q_rot, row, lens, 3000, w.sm_scale, 2048, pa, pm, pz)
        kvq.kvq_merge(case.cache, pa, pm, pz, lens, 3000, 2048, out=out, lse=lse)

    _replays_match(step, [out, lse])
