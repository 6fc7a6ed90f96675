"""Shared test helpers: build one workload's caches on the GPU (through the
library) and on the host (through the oracle) from the same seeded inputs,
and compare them.  The oracle never sees anything the GPU produced."""
import os

import numpy as np
import torch

import oracle
import workloads as wl

TOL = 2e-3   # max |o_gpu - o_ref| / max |o_ref| per (sequence, head)


# (test, largest relative error) of every rel_err call in the session; the
# conftest prints the worst per test at the end, so the margin below the bar
# is visible in every run, passing or not.
MARGINS = []


def rel_err(o_gpu, o_ref):
    """Per (sequence, head): max abs error over max abs reference value."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    den = np.abs(o_ref).max(axis=-1)
    num = np.abs(o_gpu - o_ref).max(axis=-1)
    err = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    if err.size:
        test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
        MARGINS.append((test, float(err.max())))
    return err


class Q4Case:
    """A 4-bit workload instance: inputs, GPU cache, oracle pools."""

    def __init__(self, w, lens, layer=0, device="cuda", store_chunk=None, build_oracle=True, fill=None,
                 kv_scale=None):
        import fp8_quantized_kv_amd as kvq
        self.w, self.lens, self.layer = w, list(lens), layer
        self.lay = wl.page_layout(w, self.lens)
        fmt = {4: kvq.FMT_Q4_H32, 6: kvq.FMT_Q6_H32, 8: kvq.FMT_Q8_H32}[w.bits]
        self.cache = kvq.Q4Cache(self.lay.num_pages, w.n_kv_heads, w.head_dim, w.page_size, device, fmt=fmt)
        if fill is not None:  # bytes the stores do not overwrite keep this value
            self.cache.k_pool.fill_(fill)
            self.cache.v_pool.fill_(fill)
        self.q = wl.q4_query(wl.shrink(w, batch=len(self.lens)), layer, device)
        self.page_table = self.lay.page_table.to(device)
        self.seq_lens = torch.tensor(self.lens, dtype=torch.int32, device=device)
        self.max_seq_len = max(self.lens) if self.lens else 0
        q_planted = self.q.clone()
        if kv_scale is not None:  # the query grows by the inverse, so the scores keep their spread
            self.q = (self.q / kv_scale).contiguous()
        shape = oracle.q4_pool_shape(self.lay.num_pages, w.n_kv_heads, w.page_size, w.head_dim, w.bits)
        self.k_ref = np.zeros(shape, np.uint8) if build_oracle else None
        self.v_ref = np.zeros(shape, np.uint8) if build_oracle else None
        off = 0
        for b, T in enumerate(self.lens):
            if T == 0:
                continue
            k, v = wl.q4_kv_tokens(w, layer, off, T, device)
            if b == 0:
                wl.plant(w, k, q_planted, 0, b=0)
            if kv_scale is not None:  # a power of two: exact in f32/bf16, scales become binary16 subnormals
                k, v = k * kv_scale, v * kv_scale
            off += T
            slots = wl.slots_for(self.lay.page_table[b], np.arange(T), w.page_size)
            step = store_chunk or T
            for t0 in range(0, T, step):
                kvq.kvq_store(self.cache, k[t0:t0 + step].contiguous(), v[t0:t0 + step].contiguous(),
                              slots[t0:t0 + step].to(device))
            if build_oracle:
                oracle.q4_store(self.k_ref, self.v_ref, k.float().cpu().numpy(), v.float().cpu().numpy(),
                                slots.numpy(), w.page_size)

    def gpu_attention(self, split_keys, want_partials=False):
        import fp8_quantized_kv_amd as kvq
        q_rot = kvq.kvq_rotate_q(self.q)
        pa, pm, pz = kvq.kvq_decode_attn(self.cache, q_rot, self.page_table, self.seq_lens, self.max_seq_len,
                                        self.w.sm_scale, split_keys)
        out, lse = kvq.kvq_merge(self.cache, pa, pm, pz, self.seq_lens, self.max_seq_len, split_keys)
        torch.cuda.synchronize()
        if want_partials:
            return out.cpu().numpy(), lse.cpu().numpy(), (pa.cpu().numpy(), pm.cpu().numpy(), pz.cpu().numpy())
        return out.cpu().numpy(), lse.cpu().numpy()

    def ref_attention(self, chunk=None, return_partials=False, heads=None):
        q = self.q.cpu().numpy()
        return oracle.q4_attention(self.k_ref, self.v_ref, q, self.lay.page_table.numpy(),
                                   np.array(self.lens, np.int32), self.w.sm_scale, chunk=chunk,
                                   return_partials=return_partials)


class MlaCase:
    """An fp8 latent workload instance."""

    def __init__(self, w, lens, layer=0, device="cuda", build_oracle=True, fill=None):
        import fp8_quantized_kv_amd as kvq
        self.w, self.lens = w, list(lens)
        self.lay = wl.page_layout(w, self.lens)
        self.cache = kvq.Fp8Cache(self.lay.num_pages, w.head_dim, w.rope_dim, w.page_size, device)
        if fill is not None:  # bytes the stores do not overwrite keep this value
            self.cache.codes.fill_(fill)
            self.cache.scales.view(torch.uint8).fill_(fill)
        self.q = wl.mla_query(wl.shrink(w, batch=len(self.lens)), layer, device)
        self.page_table = self.lay.page_table.to(device)
        self.seq_lens = torch.tensor(self.lens, dtype=torch.int32, device=device)
        self.max_seq_len = max(self.lens) if self.lens else 0
        n_slots = self.lay.num_pages * w.page_size
        self.codes_ref = np.zeros((n_slots, w.head_dim), np.uint8) if build_oracle else None
        self.scales_ref = np.zeros((n_slots, 2), np.float32) if build_oracle else None
        off = 0
        for b, T in enumerate(self.lens):
            if T == 0:
                continue
            x = wl.mla_rows(w, layer, off, T, device)
            off += T
            slots = wl.slots_for(self.lay.page_table[b], np.arange(T), w.page_size)
            kvq.kvq_store(self.cache, x, None, slots.to(device))
            if build_oracle:
                oracle.fp8_store(self.codes_ref, self.scales_ref, x.cpu().numpy(), slots.numpy(), w.rope_dim)

    def gpu_attention(self, split_keys):
        import fp8_quantized_kv_amd as kvq
        pa, pm, pz = kvq.kvq_decode_attn(self.cache, self.q, self.page_table, self.seq_lens, self.max_seq_len,
                                        self.w.sm_scale, split_keys)
        out, lse = kvq.kvq_merge(self.cache, pa, pm, pz, self.seq_lens, self.max_seq_len, split_keys)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()

    def gpu_attention_sel(self, sel, n_sel, split_keys):
        """Decode over the selected rows, then the merge (sel, n_sel: CPU int32 tensors)."""
        import fp8_quantized_kv_amd as kvq
        sel_d, ns_d = sel.to("cuda"), n_sel.to("cuda")
        pa, pm, pz = kvq.kvq_decode_attn_sel(self.cache, self.q, self.page_table, sel_d, ns_d, self.w.sm_scale,
                                             split_keys)
        out, lse = kvq.kvq_merge(self.cache, pa, pm, pz, ns_d, int(sel.shape[1]), split_keys)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()

    def ref_attention_sel(self, sel, n_sel):
        return oracle.mla_attention_sel(self.codes_ref, self.scales_ref, self.q.cpu().numpy(),
                                        self.lay.page_table.numpy(), sel.numpy(), n_sel.numpy(), self.w.sm_scale,
                                        self.w.rope_dim, self.w.page_size)

    def ref_attention(self, heads=None):
        q = self.q.cpu().numpy()
        if heads is not None:
            q = q[:, heads]
        return oracle.mla_attention(self.codes_ref, self.scales_ref, q, self.lay.page_table.numpy(),
                                    np.array(self.lens, np.int32), self.w.sm_scale, self.w.rope_dim,
                                    self.w.page_size)


class TqCase:
    """A rotated-int4 + Lloyd-Max latent workload instance (the fp8 workload's rows and queries)."""

    def __init__(self, w, lens, layer=0, device="cuda", build_oracle=True, n_heads=None):
        import fp8_quantized_kv_amd as kvq
        self.w, self.lens = w, list(lens)
        self.lay = wl.page_layout(w, self.lens)
        self.cache = kvq.TqCache(self.lay.num_pages, w.page_size, device)
        q = wl.mla_query(wl.shrink(w, batch=len(self.lens)), layer, device)
        self.q = q[:, :n_heads].contiguous() if n_heads else q
        self.page_table = self.lay.page_table.to(device)
        self.seq_lens = torch.tensor(self.lens, dtype=torch.int32, device=device)
        self.max_seq_len = max(self.lens) if self.lens else 0
        n_slots = self.lay.num_pages * w.page_size
        (cs, rs) = oracle.tq_pool_shape(self.lay.num_pages, w.page_size)
        self.codes_ref = np.zeros(cs, np.uint8) if build_oracle else None
        self.radii_ref = np.zeros(rs, np.float32) if build_oracle else None
        off = 0
        for b, T in enumerate(self.lens):
            if T == 0:
                continue
            x = wl.mla_rows(w, layer, off, T, device)
            off += T
            slots = wl.slots_for(self.lay.page_table[b], np.arange(T), w.page_size)
            kvq.kvq_store(self.cache, x, None, slots.to(device))
            if build_oracle:
                oracle.tq_store(self.codes_ref, self.radii_ref, x.float().cpu().numpy(), slots.numpy())

    def gpu_attention(self, split_keys):
        """Rotate the query, decode, merge (+ inverse rotation)."""
        import fp8_quantized_kv_amd as kvq
        q_rot = kvq.kvq_tq_rotate_q(self.q)
        pa, pm, pz = kvq.kvq_decode_attn(self.cache, q_rot, self.page_table, self.seq_lens, self.max_seq_len,
                                        self.w.sm_scale, split_keys)
        out, lse = kvq.kvq_merge(self.cache, pa, pm, pz, self.seq_lens, self.max_seq_len, split_keys)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()

    def ref_attention(self, heads=None):
        q = self.q if heads is None else self.q[:, heads]
        return oracle.tq_attention(self.codes_ref, self.radii_ref, q.cpu().numpy(), self.lay.page_table.numpy(),
                                   np.array(self.lens, np.int32), self.w.sm_scale, self.w.page_size)

