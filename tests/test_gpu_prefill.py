"""kvq_prefill_attn -- a prompt chunk's query rows over their sequence's 4-bit
cache, as split partials, then kvq_merge with the rows' lengths -- against the
oracle's chunk attention (fp64 over the dequantized cache), through the C ABI:
chunks in the middle and at the start of a sequence, several split sizes
(several tiles, partial tiles, ragged row groups), head_dim 128 and 256,
groups of 1 to 8 query heads, and rows with arbitrary (also zero) lengths."""
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


def _gpu_chunk(kvq, case, q, row_lens, split):
    q_rot = kvq.kvq_rotate_q(q)
    pt = case.page_table[0].contiguous()
    rl = torch.tensor(list(row_lens), dtype=torch.int32, device="cuda")
    T = case.max_seq_len
    pa, pm, pz = kvq.kvq_prefill_attn(case.cache, q_rot, pt, rl, T, case.w.sm_scale, split)
    o, lse = kvq.kvq_merge(case.cache, pa, pm, pz, rl, T, split)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def _check(case, q, row_lens, o, lse):
    ro, rl = oracle.q4_chunk_attention(case.k_ref, case.v_ref, q.cpu().numpy(), case.lay.page_table[0].numpy(),
                                       np.asarray(row_lens, np.int32), case.w.sm_scale)
    err = rel_err(o, ro)
    _say(f"  max_rel_err={err.max():.2e}")
    assert np.all(np.isfinite(o)) and err.max() < TOL
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - rl[fin]), initial=0) < 1e-3 * max(1.0, np.abs(rl[fin]).max(initial=0))
    for r, n in enumerate(row_lens):
        if n == 0:
            assert np.all(o[r] == 0) and np.all(np.isneginf(lse[r]))


@pytest.mark.parametrize("D,Hq,Hkv,P,C,split", [
    (256, 24, 4, 3000, 100, 1024),   # a chunk after 3000 positions
    (256, 24, 4, 0, 300, 128),       # a chunk from position 0 (a whole prompt)
    (256, 8, 1, 700, 37, 2048),      # groups of 8 heads, a ragged last row group
    (256, 4, 4, 1234, 17, 96),       # one head per KV head, splits of 3 tiles
    (128, 16, 2, 500, 45, 512),      # head_dim 128
])
def test_prefill_matches_oracle(kvq, D, Hq, Hkv, P, C, split):
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=1, seq_len=0, head_dim=D, n_q_heads=Hq, n_kv_heads=Hkv,
                  sm_scale=float(1.0 / np.sqrt(D)))
    case = Q4Case(w, [P + C])
    q = wl.q4_chunk_queries(w, 0, C, "cuda")
    lens = [P + 1 + r for r in range(C)]
    _say(f"prefill D={D} Hq={Hq} Hkv={Hkv} P={P} C={C} split={split}")
    o, lse = _gpu_chunk(kvq, case, q, lens, split)
    _check(case, q, lens, o, lse)


def test_prefill_arbitrary_row_lengths(kvq):
    """Rows of any lengths in any order (drafted rows, rows of length 0, rows
    shorter than their neighbours), over a shuffled page table."""
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=1, seq_len=0, shuffle_pages=True)
    T = 4100
    case = Q4Case(w, [T])
    lens = [T, 1, 0, 4099, 33, 2048, 2049, 0, 4100, 15, 16, 17, 3000]
    q = wl.q4_chunk_queries(w, 0, len(lens), "cuda", seed_key=3)
    _say("prefill arbitrary lengths")
    for split in (512, 4096):
        o, lse = _gpu_chunk(kvq, case, q, lens, split)
        _check(case, q, lens, o, lse)


def test_prefill_deterministic(kvq):
    w = wl.shrink(wl.GQA_32K, n_layers=1, batch=1, seq_len=0)
    case = Q4Case(w, [2600], build_oracle=False)
    q = wl.q4_chunk_queries(w, 0, 64, "cuda")
    lens = [2537 + r for r in range(64)]
    a = _gpu_chunk(kvq, case, q, lens, 1024)
    b = _gpu_chunk(kvq, case, q, lens, 1024)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
