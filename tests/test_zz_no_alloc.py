"""kvq_attend_noalloc (the partials in the library's static per-GPU scratch,
nothing allocated) against kvq_attend (the same work on a caller workspace),
through the C ABI: the same bits on two calls in a row, the second with a
smaller input (fewer sequences, shorter contexts, fewer splits), so the
scratch's stale contents from the first call meet the second; and a request
beyond the scratch is refused before any launch."""
import ctypes

import pytest
import torch

import workloads as wl
from helpers import MlaCase, Q4Case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    assert torch.cuda.is_available(), "no GPU"
    import fp8_quantized_kv_amd as m
    return m


def _say(*a):
    print(*a, flush=True)


def _noalloc_raw(kvq, case, q, split, out, lse):
    """kvq_attend_noalloc through ctypes, raw pointers and torch's current stream."""
    P = ctypes.c_void_p
    B, Hq, _ = q.shape
    rc = kvq.lib.kvq_attend_noalloc(ctypes.byref(case.cache.desc), P(q.data_ptr()), Hq, P(case.page_table.data_ptr()),
                                    int(case.page_table.shape[1]), P(case.seq_lens.data_ptr()), B,
                                    int(case.max_seq_len), ctypes.c_float(case.w.sm_scale), split, P(out.data_ptr()),
                                    P(lse.data_ptr()), P(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, kvq.lib.kvq_status_string(rc)


def _check_case(kvq, case, q, split):
    B, Hq, _ = q.shape
    out = torch.full((B, Hq, case.cache.dv), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    _noalloc_raw(kvq, case, q, split, out, lse)
    ref_o, ref_l = kvq.kvq_attend(case.cache, q, case.page_table, case.seq_lens, case.max_seq_len, case.w.sm_scale,
                                  split)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)


def test_noalloc_q4_two_calls_second_smaller(kvq):
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=3, seq_len=0)
    big = Q4Case(w, [9000, 20000, 4100], build_oracle=False)
    _say("noalloc q4: 3 sequences up to 20000 positions, split 2048")
    _check_case(kvq, big, kvq.kvq_rotate_q(big.q), 2048)
    small = Q4Case(wl.shrink(w, batch=2), [700, 1500], layer=1, build_oracle=False)
    _say("noalloc q4: 2 sequences up to 1500 positions, split 512")
    _check_case(kvq, small, kvq.kvq_rotate_q(small.q), 512)


def test_noalloc_fp8_two_calls_second_smaller(kvq):
    w = wl.shrink(wl.MLA_262K, n_heads=128, seq_len=0)
    big = MlaCase(w, [8000, 3000], build_oracle=False)
    _say("noalloc fp8: 2 sequences up to 8000 positions, split 256")
    _check_case(kvq, big, big.q, 256)
    small = MlaCase(wl.shrink(w, n_heads=16), [900], layer=1, build_oracle=False)
    _say("noalloc fp8: 1 sequence of 900 positions, split 512")
    _check_case(kvq, small, small.q, 512)


def test_noalloc_rejects_beyond_scratch(kvq):
    """Partials of 128 heads x 1024 splits x 512 channels (256 MiB) exceed the 64 MiB scratch."""
    w = wl.shrink(wl.MLA_262K, n_heads=128, seq_len=0)
    case = MlaCase(w, [40], build_oracle=False)
    need = kvq.kvq_attend_workspace_bytes(case.cache, 1, 128, 262144, 256)
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p
    out = torch.empty((1, 128, 512), dtype=torch.float32, device="cuda")
    pt = torch.zeros((1, 262144 // 16), dtype=torch.int32, device="cuda")
    rc = kvq.lib.kvq_attend_noalloc(ctypes.byref(case.cache.desc), P(case.q.data_ptr()), 128, P(pt.data_ptr()),
                                    262144 // 16, P(case.seq_lens.data_ptr()), 1, 262144,
                                    ctypes.c_float(w.sm_scale), 256, P(out.data_ptr()), None,
                                    P(torch.cuda.current_stream().cuda_stream))
    assert rc == -4 and b"static scratch" in kvq.lib.kvq_status_string(rc)
