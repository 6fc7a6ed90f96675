"""kvq_attend (decode + merge in one call, the partials in a caller workspace)
against the two separate calls, bit for bit, for every cache format and both
4-bit matrix-core kernels, through the C ABI."""
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


def _say(*a):
    print(*a, flush=True)


def _two_calls(kvq, case, q, split):
    pa, pm, pz = kvq.kvq_decode_attn(case.cache, q, case.page_table, case.seq_lens, case.max_seq_len,
                                     case.w.sm_scale, split)
    return kvq.kvq_merge(case.cache, pa, pm, pz, case.seq_lens, case.max_seq_len, split)


def _one_call(kvq, case, q, split, fill, ws=None):
    need = kvq.kvq_attend_workspace_bytes(case.cache, q.shape[0], q.shape[1], case.max_seq_len, split)
    if ws is None:
        ws = torch.full((need,), fill, dtype=torch.uint8, device="cuda")  # stale contents must not matter
    out = kvq.kvq_attend(case.cache, q, case.page_table, case.seq_lens, case.max_seq_len, case.w.sm_scale, split,
                         workspace=ws[:need])
    torch.cuda.synchronize()
    return out


# (bits, split): the wave-pair kernel (4-bit, split <= 1024), the single-wave
# kernel with 4 waves (split 2048; 8- and 6-bit)
@pytest.mark.parametrize("bits,split", [(4, 512), (4, 2048), (8, 512), (6, 1024)])
def test_attend_equals_decode_then_merge_h32(kvq, bits, split):
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=3, seq_len=0, bits=bits)
    case = Q4Case(w, [3000, 0, 5000], build_oracle=False)
    q_rot = kvq.kvq_rotate_q(case.q)
    _say(f"attend bits={bits} split={split}")
    o2, l2 = _two_calls(kvq, case, q_rot, split)
    o1, l1 = _one_call(kvq, case, q_rot, split, 0xFF)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("split", [512, 4096])
def test_attend_equals_decode_then_merge_d128(kvq, split):
    """head_dim 128 (the single-wave kernel: 8 waves at split 512, 4 at 4096),
    groups of 4 heads, one sequence longer than the rest and one empty."""
    w = wl.shrink(wl.TINY, batch=4, seq_len=0)
    case = Q4Case(w, [9000, 1, 0, 4097], build_oracle=False)
    q_rot = kvq.kvq_rotate_q(case.q)
    _say(f"attend d128 split={split}")
    o2, l2 = _two_calls(kvq, case, q_rot, split)
    o1, l1 = _one_call(kvq, case, q_rot, split, 0x00)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_attend_reuses_its_workspace(kvq):
    """One workspace through calls of different sizes (batch, lengths, split,
    kernel): each call gives the two-call bits, whatever the last one left."""
    ws = torch.full((64 << 20,), 0xFF, dtype=torch.uint8, device="cuda")
    for i, (lens, split) in enumerate([([20000, 7000], 512), ([33000], 2048), ([5, 3000, 12000, 1], 512),
                                        ([20000, 7000], 1024), ([65536, 100, 40000], 2048)]):
        w = wl.shrink(wl.GQA_32K, n_layers=1, batch=len(lens), seq_len=0)
        case = Q4Case(w, lens, layer=i, build_oracle=False)
        q_rot = kvq.kvq_rotate_q(case.q)
        _say(f"attend reuse {i}: lens={lens} split={split}")
        o2, l2 = _two_calls(kvq, case, q_rot, split)
        o1, l1 = _one_call(kvq, case, q_rot, split, None, ws=ws)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("split", [256, 2048])
def test_attend_equals_decode_then_merge_latent(kvq, split):
    w = wl.shrink(wl.MLA_262K, n_heads=64, seq_len=0)
    case = MlaCase(w, [2500, 700], build_oracle=False)
    _say(f"attend fp8 split={split}")
    o2, l2 = _two_calls(kvq, case, case.q, split)
    o1, l1 = _one_call(kvq, case, case.q, split, 0x7F)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    t = TqCase(w, [2500, 700], build_oracle=False, n_heads=32)
    q_rot = kvq.kvq_tq_rotate_q(t.q)
    _say(f"attend tq4 split={split}")
    o2, l2 = _two_calls(kvq, t, q_rot, split)
    o1, l1 = _one_call(kvq, t, q_rot, split, 0xFF)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
