"""Drafted rows (TensorFold issue "qwen27 CUDA: an opt-in 4-bit attention
cache", "What it is": decode rounds attend shared 512-key chunks plus each
row's tail with an in-order merge, and drafted output must equal the output
of the rows decoded one at a time): kvq_decode_attn_rows against the oracle,
and bit for bit against kvq_decode_attn over a batch repeating the page-table
row and against each row decoded alone."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import TOL, Q4Case, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvq():
    assert torch.cuda.is_available(), "no GPU"
    import fp8_quantized_kv_amd as m
    return m


def _say(*a):
    print(*a, flush=True)


def _rows_vs_batch_vs_serial(kvq, case, q, lens, split):
    """Partials and merged output of the three ways; returns the rows' (out, lse)."""
    w = case.w
    R = len(lens)
    T = max(lens)
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    q_rot = kvq.kvq_rotate_q(q)
    row = case.page_table[0].contiguous()
    pr = kvq.kvq_decode_attn_rows(case.cache, q_rot, row, sl, T, w.sm_scale, split)
    pb = kvq.kvq_decode_attn(case.cache, q_rot, row.expand(R, -1).contiguous(), sl, T, w.sm_scale, split)
    torch.cuda.synchronize()
    for a, b in zip(pr, pb):
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.cpu().numpy().view(np.uint32))
    o, l = kvq.kvq_merge(case.cache, *pr, sl, T, split)
    o, l = o.cpu().numpy(), l.cpu().numpy()
    for r in range(R):
        p1 = kvq.kvq_decode_attn(case.cache, q_rot[r:r + 1].contiguous(), row[None].contiguous(), sl[r:r + 1].contiguous(),
                                 T, w.sm_scale, split)
        o1, l1 = kvq.kvq_merge(case.cache, *p1, sl[r:r + 1].contiguous(), T, split)
        assert np.array_equal(o1.cpu().numpy()[0].view(np.uint32), o[r].view(np.uint32))
        assert np.array_equal(l1.cpu().numpy()[0].view(np.uint32), l[r].view(np.uint32))
    return o, l


@pytest.mark.parametrize("wname,split", [("gqa_q4_32k", 512), ("gqa_q4_32k", 2048), ("gqa_q8_32k", 512),
                                         ("gqa_q6_32k", 1024), ("tiny_q4_d128_t1024", 512),
                                         ("tiny_q4_d128_t1024", 2048)])
def test_rows_match_oracle_batch_and_serial(kvq, wname, split):
    """Six consecutive drafted rows (lengths T0 .. T0 + 5 over one stored
    sequence), then ragged rows (0, 1, a chunk boundary, a tail): oracle
    parity within tolerance, partials equal to the repeated-row batch bit for
    bit, merged rows equal to each row decoded alone.  head_dim 256 (wave-pair
    kernel at 512-key 4-bit splits, single-wave kernel otherwise) and 128
    (eight-wave workgroups at 512 keys, four at 2048)."""
    w = wl.WORKLOADS[wname]
    T_full = 3005
    case = Q4Case(w, [T_full])
    for lens in ([3000 + r for r in range(6)], [0, 1, 512, 2049, 3005]):
        _say(f"rows {wname} split={split} lens={lens}")
        q = wl.q4_query(wl.shrink(w, batch=len(lens)), 1, "cuda")
        o, l = _rows_vs_batch_vs_serial(kvq, case, q, lens, split)
        pt = np.repeat(case.lay.page_table.numpy()[:1], len(lens), axis=0)
        ro, rl = oracle.q4_attention(case.k_ref, case.v_ref, q.cpu().numpy(), pt, np.array(lens, np.int32),
                                     w.sm_scale)
        err = rel_err(o, ro)
        _say(f"  max_rel_err={err.max():.2e}")
        assert err.max() < TOL
        fin = np.isfinite(rl)
        assert np.array_equal(fin, np.isfinite(l))
        assert np.max(np.abs(l[fin] - rl[fin])) < 1e-3 * max(1.0, np.abs(rl[fin]).max())


def test_rows_full_size_bit_identical(kvq):
    """Four drafted rows at the full 262144-position context, split 2048 (the
    headline decode's launch): partials equal the repeated-row batch and each
    merged row equals that row decoded alone, bit for bit; sampled heads of
    the last row against the oracle."""
    w = wl.GQA_262K
    case = Q4Case(w, [w.seq_len])
    lens = [w.seq_len - 3 + r for r in range(4)]
    _say(f"rows full size lens={lens}")
    q = wl.q4_query(wl.shrink(w, batch=4), 1, "cuda")
    o, l = _rows_vs_batch_vs_serial(kvq, case, q, lens, w.split_keys)
    ro, rl = oracle.q4_attention(case.k_ref, case.v_ref, q[3:4].cpu().numpy(), case.lay.page_table.numpy()[:1],
                                 np.array(lens[3:], np.int32), w.sm_scale)
    err = rel_err(o[3:4], ro)
    _say(f"  last row max_rel_err={err.max():.2e}")
    assert err.max() < TOL


def test_rows_argument_checks(kvq):
    """More than 64 rows and the latent formats are refused."""
    w = wl.GQA_32K
    case = Q4Case(w, [600], build_oracle=False)
    q = torch.zeros((65, w.n_q_heads, w.head_dim), device="cuda")
    sl = torch.full((65,), 600, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        kvq.kvq_decode_attn_rows(case.cache, q, case.page_table[0].contiguous(), sl, 600, w.sm_scale, 512)
