"""Seeded synthetic inputs for the sub-byte KV cache workloads.

This module only draws random numbers and lays out page tables; it holds
none of the method's arithmetic (no rotation, quantization or attention).
Both sides of every comparison -- the GPU library and the CPU oracle -- take
their inputs from here, so a test feeds the exact same tensors to both.

The shapes follow the pages' workloads: 4 KV heads x head_dim 256 with
144-byte 4-bit rows and 16 attention layers (TensorFold issue "qwen27 CUDA:
an opt-in 4-bit attention cache", section "What it is"); a 512 + 64 fp8
latent with 128 absorbed heads (colibri pull request "KV cache quantization:
fp8 (KV8) + 4-bit TurboQuant (KV_TQ)", KV8 commit).  Real models and text
are not available, so K/V rows are N(0,1) with heavy-tailed (Student-t,
nu = 3) or outlier channels -- the kurtotic statistics that motivate the
rotation (FreeToken pull request "feat(kvcache): add reliable quantized KV
cache", test-fix commit, kurtotic round trips).

Every tensor is drawn from a torch.Generator seeded from (workload seed,
layer, 4096-token block), so a position's values do not depend on how many
positions are generated at once: a test at a shorter context sees exactly
the first rows of the full workload.
"""
from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import torch

BLOCK_TOKENS = 4096


@dataclass(frozen=True)
class Q4Workload:
    """A decode workload over the 4-bit Hadamard-32 cache."""
    name: str
    seed: int
    n_layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int = 0                 # fixed context (0 when lens are drawn)
    len_range: Tuple[int, int] = (0, 0)  # inclusive uniform range for ragged batches
    page_size: int = 16
    kv_dtype: torch.dtype = torch.bfloat16
    q_std: float = 1.0
    sm_scale: float = 1.0
    outlier_channels: int = 0        # channels scaled by outlier_scale
    outlier_scale: float = 20.0
    heavy_channels: int = 0          # channels drawn Student-t(3)
    shuffle_pages: bool = False
    plant_at: Optional[int] = None   # position whose K equals the group's first query
    prefill_chunk: int = 0           # extra tokens stored per step (not attended)
    split_keys: int = 2048
    bits: int = 4                    # code width of the block format (4, 6 or 8)
    chunk_rows: int = 0              # a prompt chunk: the last chunk_rows positions, each a query row

    @property
    def row_bytes(self):
        return {4: 16, 6: 24, 8: 32}[self.bits] * (self.head_dim // 32) + 2 * (self.head_dim // 32)

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads


@dataclass(frozen=True)
class MlaWorkload:
    """A decode workload over the fp8 e4m3 latent cache (absorbed attention)."""
    name: str
    seed: int
    n_layers: int
    batch: int
    n_heads: int
    kv_lora: int
    rope_dim: int
    seq_len: int
    page_size: int = 16
    heavy_channels: int = 16
    sm_scale: float = 1.0
    split_keys: int = 1024

    @property
    def head_dim(self):
        return self.kv_lora + self.rope_dim


# The five workloads.  sm_scale = 1/sqrt(head_dim) except for the tiny case,
# whose query is already drawn N(0,1)/sqrt(128).
TINY = Q4Workload("tiny_q4_d128_t1024", seed=1001, n_layers=1, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=128,
                  seq_len=1024, kv_dtype=torch.float32, q_std=128 ** -0.5, sm_scale=1.0, outlier_channels=4,
                  split_keys=512)
GQA_32K = Q4Workload("gqa_q4_32k", seed=1002, n_layers=16, batch=1, n_q_heads=24, n_kv_heads=4, head_dim=256,
                     seq_len=32768, sm_scale=1 / 16, heavy_channels=16, split_keys=512)
GQA_262K = Q4Workload("gqa_q4_262k", seed=1003, n_layers=16, batch=1, n_q_heads=24, n_kv_heads=4, head_dim=256,
                      seq_len=262144, sm_scale=1 / 16, heavy_channels=16, plant_at=131072, split_keys=2048)
RAGGED = Q4Workload("ragged_q4_b16", seed=1004, n_layers=1, batch=16, n_q_heads=24, n_kv_heads=4, head_dim=256,
                    len_range=(4096, 65536), sm_scale=1 / 16, heavy_channels=16, shuffle_pages=True,
                    prefill_chunk=2048, split_keys=2048)
MLA_262K = MlaWorkload("mla_fp8_262k", seed=1005, n_layers=4, batch=1, n_heads=128, kv_lora=512, rope_dim=64,
                       seq_len=262144, sm_scale=576 ** -0.5, split_keys=2048)

# The 8- and 6-bit block variants on the 32K shape (the same inputs; only the code width differs).
GQA_32K_Q8 = replace(GQA_32K, name="gqa_q8_32k", bits=8)
GQA_32K_Q6 = replace(GQA_32K, name="gqa_q6_32k", bits=6)

# The latent workload's rows at 32K positions, stored with the rotated-int4 + Lloyd-Max codec.
MLA_TQ4_32K = replace(MLA_262K, name="mla_tq4_32k", seq_len=32768, split_keys=256)
MLA_TQ4_262K = replace(MLA_262K, name="mla_tq4_262k")

# A 2048-row prompt chunk after the 32K context (one layer): the chunk's rows are
# positions 32768 .. 34815, stored first, and row r attends [0, 32768 + r];
# one split covers the whole context (34816 = 1088 tiles of 32 keys).
CHUNK_32K = replace(GQA_32K, name="chunk_q4_32k", n_layers=1, seq_len=32768 + 2048, chunk_rows=2048,
                    split_keys=32768 + 2048)

WORKLOADS = {w.name: w for w in (TINY, GQA_32K, GQA_262K, RAGGED, MLA_262K, GQA_32K_Q8, GQA_32K_Q6, MLA_TQ4_32K,
                                              MLA_TQ4_262K, CHUNK_32K)}


def shrink(w, **kw):
    """The same workload with some sizes changed (for tests that must run fast)."""
    return replace(w, **kw)


def _gen(device, *key):
    g = torch.Generator(device=device)
    h = 0
    for k in key:
        h = (h * 1000003 + int(k)) % (2 ** 62)
    g.manual_seed(h)
    return g


def seq_lens(w):
    """Context length of each sequence (int list)."""
    if w.seq_len:
        return [w.seq_len] * w.batch
    lo, hi = w.len_range
    g = _gen("cpu", w.seed, 7)
    return torch.randint(lo, hi + 1, (w.batch,), generator=g).tolist()


@dataclass
class PageLayout:
    page_table: torch.Tensor   # [B][max_pages] int32 (unused entries 0)
    num_pages: int             # pages in the pool (including the prefill chunk's)
    prefill_pages: torch.Tensor  # pages reserved for the prefill chunk (int32)


def page_layout(w, lens=None):
    """Page table for the sequences (pages in order, or a seeded shuffle of the pool)."""
    lens = seq_lens(w) if lens is None else lens
    ps = w.page_size
    need = [-(-T // ps) for T in lens]
    n_pre = -(-getattr(w, "prefill_chunk", 0) // ps)
    total = sum(need) + n_pre
    if getattr(w, "shuffle_pages", False):
        perm = torch.randperm(total, generator=_gen("cpu", w.seed, 11)).to(torch.int32)
    else:
        perm = torch.arange(total, dtype=torch.int32)
    max_pages = max(need) if need else 1
    pt = torch.zeros((len(lens), max(max_pages, 1)), dtype=torch.int32)
    off = 0
    for b, n in enumerate(need):
        pt[b, :n] = perm[off:off + n]
        off += n
    return PageLayout(pt, total, perm[off:off + n_pre].clone())


def _heavy_rows(w, n_tok, channels_sel, g, device, std_rows):
    """[n_tok][H][D] N(0,1) with the selected channels replaced by Student-t(3)."""
    x = torch.randn(std_rows, generator=g, device=device)
    if channels_sel is not None:
        H, k = channels_sel.shape
        z = torch.randn((n_tok, H, k), generator=g, device=device)
        chi2 = torch.randn((n_tok, H, k, 3), generator=g, device=device).pow(2).sum(-1)
        t = z / torch.sqrt(chi2 / 3.0)
        idx = channels_sel.to(device).unsqueeze(0).expand(n_tok, H, k)
        x.scatter_(2, idx, t)
    return x


def q4_channel_choice(w, device="cpu"):
    """Per KV head, the channels that carry outliers or heavy tails ([H_kv][k] int64)."""
    k = w.outlier_channels or w.heavy_channels
    if not k:
        return None
    g = _gen("cpu", w.seed, 13)
    return torch.stack([torch.randperm(w.head_dim, generator=g)[:k] for _ in range(w.n_kv_heads)]).to(device)


def q4_kv_block(w, layer, block, device="cpu", which="kv"):
    """K and V of positions [block*4096, (block+1)*4096) of every sequence slot-range.

    Returns (k, v), each [4096][H_kv][D] in w.kv_dtype.  Sequences share the
    position stream: sequence b position j uses global token index
    sum(lens[:b]) + j (see q4_kv_tokens)."""
    g = _gen(device, w.seed, 101, layer, block)
    sel = q4_channel_choice(w, device)
    shape = (BLOCK_TOKENS, w.n_kv_heads, w.head_dim)
    out = []
    for _ in range(2):
        if w.outlier_channels:
            x = torch.randn(shape, generator=g, device=device)
            idx = sel.unsqueeze(0).expand(BLOCK_TOKENS, -1, -1)
            x.scatter_(2, idx, x.gather(2, idx) * w.outlier_scale)
        else:
            x = _heavy_rows(w, BLOCK_TOKENS, sel if w.heavy_channels else None, g, device, shape)
        out.append(x.to(w.kv_dtype))
    return out[0], out[1]


def q4_kv_tokens(w, layer, start, count, device="cpu"):
    """K and V of global tokens [start, start+count): ([count][H_kv][D], same)."""
    ks, vs = [], []
    b0, b1 = start // BLOCK_TOKENS, (start + count - 1) // BLOCK_TOKENS
    for blk in range(b0, b1 + 1):
        k, v = q4_kv_block(w, layer, blk, device)
        lo = max(start, blk * BLOCK_TOKENS) - blk * BLOCK_TOKENS
        hi = min(start + count, (blk + 1) * BLOCK_TOKENS) - blk * BLOCK_TOKENS
        ks.append(k[lo:hi])
        vs.append(v[lo:hi])
    return torch.cat(ks), torch.cat(vs)


def q4_query(w, layer, device="cpu"):
    """Query [B][H_q][D] float32, N(0, q_std^2), unrotated."""
    g = _gen(device, w.seed, 202, layer)
    return torch.randn((w.batch, w.n_q_heads, w.head_dim), generator=g, device=device) * w.q_std


def plant(w, k_tokens, q, token_offset, b=0):
    """Write the planted key: K at position plant_at of sequence b (in a token
    range starting at token_offset) equals the unrotated query of the first
    query head of each KV head's group.  Returns True if the range held it."""
    if w.plant_at is None:
        return False
    j = w.plant_at - token_offset
    if not 0 <= j < k_tokens.shape[0]:
        return False
    for gkv in range(w.n_kv_heads):
        k_tokens[j, gkv] = q[b, gkv * w.group].to(k_tokens.dtype)
    return True


def q4_chunk_queries(w, layer, n_rows, device="cpu", seed_key=0):
    """Queries of a prompt chunk's rows: [n_rows][H_q][D] f32 ~ N(0,1), as the
    decode query (the chunk's rows are ordinary positions of the sequence)."""
    g = _gen(device, w.seed, 505, layer, seed_key)
    return torch.randn((n_rows, w.n_q_heads, w.head_dim), generator=g, device=device, dtype=torch.float32)


def q4_prefill_chunk(w, layer, device="cpu"):
    """The extra chunk stored each step (ragged workload): ([n][H_kv][D], same)."""
    g = _gen(device, w.seed, 303, layer)
    shape = (w.prefill_chunk, w.n_kv_heads, w.head_dim)
    sel = q4_channel_choice(w, device)
    k = _heavy_rows(w, w.prefill_chunk, sel, g, device, shape).to(w.kv_dtype)
    v = _heavy_rows(w, w.prefill_chunk, sel, g, device, shape).to(w.kv_dtype)
    return k, v


def slots_for(page_table_row, positions, page_size):
    """Slots (int64) of logical positions of one sequence."""
    positions = torch.as_tensor(positions, dtype=torch.int64)
    pages = page_table_row.to(torch.int64)[positions // page_size]
    return pages * page_size + positions % page_size


# ---------------------------------------------------------------- fp8 latent

def mla_channel_choice(w):
    g = _gen("cpu", w.seed, 13)
    return torch.randperm(w.kv_lora, generator=g)[:w.heavy_channels]


def mla_rows_block(w, layer, block, device="cpu"):
    """Latent rows of positions [block*4096, (block+1)*4096): [4096][576] float32."""
    g = _gen(device, w.seed, 101, layer, block)
    x = torch.randn((BLOCK_TOKENS, w.head_dim), generator=g, device=device)
    k = w.heavy_channels
    if k:
        sel = mla_channel_choice(w).to(device)
        z = torch.randn((BLOCK_TOKENS, k), generator=g, device=device)
        chi2 = torch.randn((BLOCK_TOKENS, k, 3), generator=g, device=device).pow(2).sum(-1)
        x[:, sel] = z / torch.sqrt(chi2 / 3.0)
    return x


def mla_rows(w, layer, start, count, device="cpu"):
    xs = []
    b0, b1 = start // BLOCK_TOKENS, (start + count - 1) // BLOCK_TOKENS
    for blk in range(b0, b1 + 1):
        x = mla_rows_block(w, layer, blk, device)
        lo = max(start, blk * BLOCK_TOKENS) - blk * BLOCK_TOKENS
        hi = min(start + count, (blk + 1) * BLOCK_TOKENS) - blk * BLOCK_TOKENS
        xs.append(x[lo:hi])
    return torch.cat(xs)


def mla_query(w, layer, device="cpu"):
    """Absorbed query [B][H][kv_lora + rope] float32 ~ N(0,1)."""
    g = _gen(device, w.seed, 202, layer)
    return torch.randn((w.batch, w.n_heads, w.head_dim), generator=g, device=device)


def dsa_selection(w, lens, n_sel, max_sel=None, seed_key=0):
    """A sparse-attention selection per sequence: n_sel[b] distinct positions
    of [0, lens[b]) in a seeded random order (a top-k list has no order the
    attention depends on), padded with -1 to max_sel entries.  Returns
    (sel int32 [B][max_sel], n_sel int32 [B]) on the CPU."""
    max_sel = max(n_sel) if max_sel is None else max_sel
    sel = torch.full((len(lens), max_sel), -1, dtype=torch.int32)
    for b, (T, n) in enumerate(zip(lens, n_sel)):
        assert n <= T and n <= max_sel
        g = _gen("cpu", w.seed, 404, seed_key, b)
        sel[b, :n] = torch.randperm(T, generator=g)[:n].to(torch.int32)
    return sel, torch.tensor(list(n_sel), dtype=torch.int32)
