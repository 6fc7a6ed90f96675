#!/usr/bin/env python3
"""Decode-step benchmark for the 4-bit Hadamard-32 KV cache on one MI355X.

One step = one pass of the hot path over every layer of the workload:
kvq_store of the step's new token (K and V), kvq_rotate_q, kvq_decode_attn
(split-K over the paged 4-bit cache), kvq_merge (log-sum-exp merge and the
inverse rotation).  Inputs are synthetic and seeded (module `workloads`) and
resident in HBM before timing starts; 16 layer caches are cycled so the
working set (4.8 GB at 262K) is far above the 256 MB Infinity Cache.

Prints one JSON line: whole-step KV-read throughput (algorithmic bytes:
T x KV heads x (K, V) x 144 B per layer) and microseconds per layer, from
uninstrumented steps; decode + merge alone per layer; the step replayed as
one HIP graph per layer (each replay first checked against the eager step's
outputs, bit for bit; not faster than the eager launches, which already
keep the queue full); a roofline object for the
decode kernel, whose average launch is timed by HIP events on the stream it
runs on around steps of decode launches alone, back to back (region time /
launches; the figure with an event pair around every launch, which adds the
event records' own cost, is reported beside it); side measurements
of the 32K 4-bit, the ragged-batch and the 262K fp8-latent workloads; and
the CPU oracle timed on a bounded sample of the headline workload.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s

# HBM bytes per decode launch of the headline workload from rocprofv3 FETCH_SIZE and WRITE_SIZE
# passes (KiB per dispatch), scaled by what the same counters read for a 256 MiB device copy
# (FETCH_SIZE x 2.0, WRITE_SIZE x 1.0); valid only for the kernel sources they were taken on
# (keyed by the sha256 of the kernel file followed by the device-helper header it includes).
TRAFFIC = {
    "cb49a6e0450434563dceb0d3d89e053cb4eb6254b14d2ed8c71e106d5196a936": {
        "fetch_kib": 147708.5, "write_kib": 3264.0, "fetch_scale": 2.0, "write_scale": 1.0,
        "profile": "profiles/decode_q4_mfma_gqa_q4_262k.md"},
    # the same counters: these sources add the 8- and 6-bit step forms, and the 4-bit
    # instantiations compile to the same instructions as those of the key above
    "ac089d7e295e717113db3d57be593225a95ce96e804d6331cb38e6dce4e76b79": {
        "fetch_kib": 147708.5, "write_kib": 3264.0, "fetch_scale": 2.0, "write_scale": 1.0,
        "profile": "profiles/decode_q4_mfma_gqa_q4_262k.md"},
}
DECODE_SOURCES = (os.path.join("fp8_quantized_kv_amd", "csrc", "decode_q4_mfma.hip"),
                  os.path.join("fp8_quantized_kv_amd", "csrc", "mfma_common.h"))


def decode_traffic():
    """Calibrated HBM bytes per launch if the counters match the current kernel sources, else None."""
    import hashlib
    h = hashlib.sha256()
    try:
        for src in DECODE_SOURCES:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
    except OSError:
        return None
    digest = h.hexdigest()
    t = TRAFFIC.get(digest)
    if t is None:
        return None
    return int(round(t["fetch_kib"] * 1024 * t["fetch_scale"] + t["write_kib"] * 1024 * t["write_scale"]))
METRIC = "KV-read GB/s (% of HBM peak) and µs/layer, 4-bit split-K decode at 32K/262K"


def _log(*a):
    print(*a, file=sys.stderr, flush=True)


class _Bench:
    """Per-layer raw C-ABI calls of one step: a list of (entry point, args)
    per layer, with the index of the decode call (and of other calls to time)."""

    DECODE = None
    DECODE_MERGE = ()  # indices of the decode and merge calls
    EXTRA_TIMED = {}  # name -> call index, timed like the decode
    STEP = None  # indices of the calls one step runs (None: every call)
    EVENT_CALLS = None  # the calls run while one of them is timed by events (None: the step's)

    def step(self, events=None, which=None, stream=None, only=None):
        """Enqueue one step; if events is a list of (start, end) pairs, bracket
        call `which` (default: the decode) of each layer with them, on the
        stream the kernels run on.  `stream` (a raw handle) replaces the
        stream the calls were built with; `only` restricts the step to the
        calls with those indices."""
        L = self.kvq.lib
        which = self.DECODE if which is None else which
        if only is None:
            only = self.STEP
        for layer, calls in enumerate(self.raw):
            rc = 0
            for i, (fn, args) in enumerate(calls):
                if only is not None and i not in only:
                    continue
                if stream is not None:
                    args = args[:-1] + (stream,)
                if events is not None and i == which:
                    events[layer][0].record()
                rc |= getattr(L, fn)(*args)
                if events is not None and i == which:
                    events[layer][1].record()
            if rc:
                raise RuntimeError(f"launch failed in layer {layer}")

    def outputs(self):
        """Copies of the step's outputs (every layer's merged context and lse)."""
        return self.out.clone(), self.lse.clone()


class Q4Bench(_Bench):
    """Every layer's cache, query and buffers for one 4-bit workload, plus the
    raw C-ABI argument tuples of one step (validated once by building them
    through the binding's checks).  Calls per layer: store + rotate (one
    launch, kvq_store_rotate_q), decode, merge; and, where the library has
    it (the Hadamard-32 formats at head_dim 256), kvq_decode_step, the same
    work in two launches with the same bits.  A step runs kvq_decode_step where it
    exists (the three calls are timed too, as us_per_layer_three_launches),
    else the three calls."""

    DECODE = 1
    DECODE_MERGE = (1, 2)

    def __init__(self, w, device="cuda"):
        import numpy as np
        import torch

        import fp8_quantized_kv_amd as kvq
        import workloads as wl
        self.w, self.kvq = w, kvq
        T = w.seq_len
        self.T = T
        lay = wl.page_layout(w, [T])
        self.page_table = lay.page_table.to(device)
        self.seq_lens = torch.tensor([T], dtype=torch.int32, device=device)
        self.caches, self.q, self.k_new, self.v_new = [], [], [], []
        chunk = 32768
        slots_all = wl.slots_for(lay.page_table[0], np.arange(T), w.page_size).to(device)
        fmt = {4: kvq.FMT_Q4_H32, 6: kvq.FMT_Q6_H32, 8: kvq.FMT_Q8_H32}[w.bits]
        for layer in range(w.n_layers):
            c = kvq.Q4Cache(lay.num_pages, w.n_kv_heads, w.head_dim, w.page_size, device, fmt=fmt)
            q = wl.q4_query(w, layer, device)
            for t0 in range(0, T, chunk):
                n = min(chunk, T - t0)
                k, v = wl.q4_kv_tokens(w, layer, t0, n, device)
                wl.plant(w, k, q, t0)
                kvq.kvq_store(c, k, v, slots_all[t0:t0 + n])
                if t0 + n == T:
                    self.k_new.append(k[-1:].clone())
                    self.v_new.append(v[-1:].clone())
            self.caches.append(c)
            self.q.append(q)
        self.slot_new = slots_all[T - 1:T].clone()
        acc_shape, mz_shape = kvq.partial_shapes(self.caches[0], 1, w.n_q_heads, T, w.split_keys)
        f32 = dict(dtype=torch.float32, device=device)
        self.q_rot = torch.empty((1, w.n_q_heads, w.head_dim), **f32)
        self.pa, self.pm, self.pz = torch.empty(acc_shape, **f32), torch.empty(mz_shape, **f32), torch.empty(mz_shape, **f32)
        self.out = torch.empty((w.n_layers, 1, w.n_q_heads, w.head_dim), **f32)
        self.lse = torch.empty((w.n_layers, 1, w.n_q_heads), **f32)
        ws_bytes = kvq.kvq_attend_workspace_bytes(self.caches[0], 1, w.n_q_heads, T, w.split_keys)
        self.ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=device)
        torch.cuda.synchronize()
        # One checked pass through the binding validates every argument once;
        # the step's outputs are then those of kvq_decode_step where it runs.
        self.fused = True
        for layer in range(w.n_layers):
            c = self.caches[layer]
            kvq.kvq_store_rotate_q(c, self.k_new[layer], self.v_new[layer], self.slot_new, self.q[layer],
                                   out=self.q_rot)
            kvq.kvq_decode_attn(c, self.q_rot, self.page_table, self.seq_lens, T, w.sm_scale, w.split_keys,
                                self.pa, self.pm, self.pz)
            kvq.kvq_merge(c, self.pa, self.pm, self.pz, self.seq_lens, T, w.split_keys, out=self.out[layer],
                          lse=self.lse[layer])
            if self.fused:
                try:
                    kvq.kvq_decode_step(c, self.k_new[layer], self.v_new[layer], self.q[layer], self.page_table,
                                        self.seq_lens, T, w.sm_scale, w.split_keys, workspace=self.ws,
                                        out=self.out[layer], lse=self.lse[layer])
                except kvq.KvqError as e:
                    if e.status != kvq.KVQ_ERR_UNSUPPORTED:
                        raise
                    self.fused = False
        torch.cuda.synchronize()
        P = ctypes.c_void_p
        stream = P(torch.cuda.current_stream().cuda_stream)
        self.raw = []
        for layer, c in enumerate(self.caches):
            d = ctypes.byref(c.desc)
            self.raw.append([
                ("kvq_store_rotate_q", (d, P(self.k_new[layer].data_ptr()), P(self.v_new[layer].data_ptr()),
                                        kvq._DTYPES[self.k_new[layer].dtype], P(self.slot_new.data_ptr()), 1,
                                        P(self.q[layer].data_ptr()), 0, P(self.q_rot.data_ptr()), w.n_q_heads,
                                        stream)),
                ("kvq_decode_attn", (d, P(self.q_rot.data_ptr()), w.n_q_heads, P(self.page_table.data_ptr()),
                                     self.page_table.shape[1], P(self.seq_lens.data_ptr()), 1, T,
                                     ctypes.c_float(w.sm_scale), w.split_keys, P(self.pa.data_ptr()),
                                     P(self.pm.data_ptr()), P(self.pz.data_ptr()), stream)),
                ("kvq_merge", (d, P(self.pa.data_ptr()), P(self.pm.data_ptr()), P(self.pz.data_ptr()),
                               P(self.seq_lens.data_ptr()), 1, w.n_q_heads, T, w.split_keys, 1,
                               P(self.out[layer].data_ptr()), P(self.lse[layer].data_ptr()), stream)),
            ])
            if self.fused:
                self.raw[-1].append(
                    ("kvq_decode_step", (d, P(self.k_new[layer].data_ptr()), P(self.v_new[layer].data_ptr()),
                                         kvq._DTYPES[self.k_new[layer].dtype], P(self.q[layer].data_ptr()), 0,
                                         w.n_q_heads, P(self.page_table.data_ptr()), self.page_table.shape[1],
                                         P(self.seq_lens.data_ptr()), 1, T, ctypes.c_float(w.sm_scale),
                                         w.split_keys, P(self.ws.data_ptr()), ctypes.c_size_t(self.ws.numel()),
                                         P(self.out[layer].data_ptr()), P(self.lse[layer].data_ptr()), stream)))
        if self.fused:
            self.STEP = (3,)
            self.THREE_CALLS = self.EVENT_CALLS = (0, 1, 2)

    @property
    def kv_bytes_per_layer(self):
        w = self.w
        return self.T * w.n_kv_heads * 2 * w.row_bytes

    flops_per_layer = None


class MlaBench(_Bench):
    """The fp8 latent workload: every layer's cache and query; step per layer:
    store the step's token, decode (absorbed attention, split-T), merge -- as
    kvq_decode_step (the store inside the decode launch, then the merge), with
    the three calls timed too (us_per_layer_three_launches)."""

    DECODE = 1
    DECODE_MERGE = (1, 2)
    ROTATED = False  # the query is rotated before the decode, the context back in the merge

    def __init__(self, w, device="cuda"):
        import numpy as np
        import torch

        import fp8_quantized_kv_amd as kvq
        import workloads as wl
        self.w, self.kvq = w, kvq
        T = w.seq_len
        self.T = T
        lay = wl.page_layout(w, [T])
        self.page_table = lay.page_table.to(device)
        self.seq_lens = torch.tensor([T], dtype=torch.int32, device=device)
        slots_all = wl.slots_for(lay.page_table[0], np.arange(T), w.page_size).to(device)
        self.caches, self.q, self.x_new = [], [], []
        chunk = 32768
        for layer in range(w.n_layers):
            c = self._new_cache(kvq, lay, w, device)
            for t0 in range(0, T, chunk):
                n = min(chunk, T - t0)
                x = wl.mla_rows(w, layer, t0, n, device)
                kvq.kvq_store(c, x, None, slots_all[t0:t0 + n])
                if t0 + n == T:
                    self.x_new.append(x[-1:].clone())
            self.caches.append(c)
            self.q.append(wl.mla_query(w, layer, device))
        self.slot_new = slots_all[T - 1:T].clone()
        acc_shape, mz_shape = kvq.partial_shapes(self.caches[0], 1, w.n_heads, T, w.split_keys)
        f32 = dict(dtype=torch.float32, device=device)
        self.pa, self.pm, self.pz = torch.empty(acc_shape, **f32), torch.empty(mz_shape, **f32), torch.empty(mz_shape, **f32)
        self.out = torch.empty((w.n_layers, 1, w.n_heads, w.kv_lora), **f32)
        self.lse = torch.empty((w.n_layers, 1, w.n_heads), **f32)
        self.q_rot = torch.empty((1, w.n_heads, w.head_dim), **f32)
        self.fused = not self.ROTATED  # the fp8 rows' step form; the rotated rows have none
        if self.fused:
            ws_bytes = kvq.kvq_attend_workspace_bytes(self.caches[0], 1, w.n_heads, T, w.split_keys)
            self.ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=device)
        torch.cuda.synchronize()
        for layer in range(w.n_layers):
            c = self.caches[layer]
            if self.ROTATED:
                qd = kvq.kvq_store_rotate_q(c, self.x_new[layer], None, self.slot_new, self.q[layer], out=self.q_rot)
            else:
                kvq.kvq_store(c, self.x_new[layer], None, self.slot_new)
                qd = self.q[layer]
            kvq.kvq_decode_attn(c, qd, self.page_table, self.seq_lens, T, w.sm_scale, w.split_keys,
                                self.pa, self.pm, self.pz)
            kvq.kvq_merge(c, self.pa, self.pm, self.pz, self.seq_lens, T, w.split_keys, out=self.out[layer],
                          lse=self.lse[layer])
            if self.fused:
                kvq.kvq_decode_step(c, self.x_new[layer], None, self.q[layer], self.page_table, self.seq_lens, T,
                                    w.sm_scale, w.split_keys, workspace=self.ws, out=self.out[layer],
                                    lse=self.lse[layer])
        torch.cuda.synchronize()
        P = ctypes.c_void_p
        stream = P(torch.cuda.current_stream().cuda_stream)
        self.raw = []
        for layer, c in enumerate(self.caches):
            d = ctypes.byref(c.desc)
            qd = self.q_rot if self.ROTATED else self.q[layer]
            xdt = kvq._DTYPES[self.x_new[layer].dtype]
            first = (("kvq_store_rotate_q", (d, P(self.x_new[layer].data_ptr()), None, xdt, P(self.slot_new.data_ptr()),
                                             1, P(self.q[layer].data_ptr()), kvq.DT_F32, P(self.q_rot.data_ptr()),
                                             w.n_heads, stream))
                     if self.ROTATED else
                     ("kvq_store", (d, P(self.x_new[layer].data_ptr()), None, xdt, P(self.slot_new.data_ptr()), 1,
                                    stream)))
            self.raw.append([first,
                ("kvq_decode_attn", (d, P(qd.data_ptr()), w.n_heads, P(self.page_table.data_ptr()),
                                     self.page_table.shape[1], P(self.seq_lens.data_ptr()), 1, T,
                                     ctypes.c_float(w.sm_scale), w.split_keys, P(self.pa.data_ptr()),
                                     P(self.pm.data_ptr()), P(self.pz.data_ptr()), stream)),
                ("kvq_merge", (d, P(self.pa.data_ptr()), P(self.pm.data_ptr()), P(self.pz.data_ptr()),
                               P(self.seq_lens.data_ptr()), 1, w.n_heads, T, w.split_keys, 1 if self.ROTATED else 0,
                               P(self.out[layer].data_ptr()), P(self.lse[layer].data_ptr()), stream)),
            ])
            if self.fused:
                self.raw[-1].append(
                    ("kvq_decode_step", (d, P(self.x_new[layer].data_ptr()), None, xdt, P(self.q[layer].data_ptr()),
                                         kvq.DT_F32, w.n_heads, P(self.page_table.data_ptr()),
                                         self.page_table.shape[1], P(self.seq_lens.data_ptr()), 1, T,
                                         ctypes.c_float(w.sm_scale), w.split_keys, P(self.ws.data_ptr()),
                                         ctypes.c_size_t(self.ws.numel()), P(self.out[layer].data_ptr()),
                                         P(self.lse[layer].data_ptr()), stream)))
        if self.fused:
            self.STEP = (3,)
            self.THREE_CALLS = self.EVENT_CALLS = (0, 1, 2)

    ROW_BYTES = 576 + 8  # code bytes + two f32 scales per position

    @staticmethod
    def _new_cache(kvq, lay, w, device):
        return kvq.Fp8Cache(lay.num_pages, w.head_dim, w.rope_dim, w.page_size, device)

    @property
    def kv_bytes_per_layer(self):
        return self.T * self.ROW_BYTES

    @property
    def flops_per_layer(self):
        # per position and head: <q, k> over 576 values and the 512-wide value accumulation, 2 flop per MAC
        w = self.w
        return self.T * w.n_heads * 2 * (w.head_dim + w.kv_lora)


class TqBench(MlaBench):
    """The same latent workload stored with the rotated-int4 + Lloyd-Max codec
    (288 code bytes + two f32 radii per position); step per layer: store and
    rotate the query (one launch), decode on matrix cores, merge + inverse
    rotation."""

    ROW_BYTES = 288 + 8
    ROTATED = True

    @staticmethod
    def _new_cache(kvq, lay, w, device):
        return kvq.TqCache(lay.num_pages, w.page_size, device)


class DsaBench(_Bench):
    """Selected rows (DSA gather) over the fp8 latent workload's layer caches:
    `batch` sequences share each layer's context (the same pages), each with
    its own query and its own seeded selection of n_sel distinct positions;
    step per layer: decode over the selection, merge."""

    DECODE = 0
    DECODE_MERGE = (0, 1)

    def __init__(self, mla, n_sel, batch, split_keys=512, device="cuda"):
        import torch

        import workloads as wl
        w, kvq = mla.w, mla.kvq
        self.w, self.kvq, self.n_sel, self.batch = w, kvq, n_sel, batch
        T = mla.T
        H = w.n_heads
        self.page_table = mla.page_table.expand(batch, -1).contiguous()
        self.q, self.sel = [], []
        for layer in range(w.n_layers):
            self.q.append(wl.mla_query(wl.shrink(w, batch=batch), layer, device))
            sel, ns = wl.dsa_selection(w, [T] * batch, [n_sel] * batch, n_sel, seed_key=layer)
            self.sel.append(sel.to(device))
        self.n_sel_t = ns.to(device)
        acc_shape, mz_shape = kvq.partial_shapes(mla.caches[0], batch, H, n_sel, split_keys)
        f32 = dict(dtype=torch.float32, device=device)
        self.pa, self.pm, self.pz = torch.empty(acc_shape, **f32), torch.empty(mz_shape, **f32), torch.empty(mz_shape, **f32)
        self.out = torch.empty((w.n_layers, batch, H, w.kv_lora), **f32)
        self.lse = torch.empty((w.n_layers, batch, H), **f32)
        for layer, c in enumerate(mla.caches):  # one checked pass through the binding
            kvq.kvq_decode_attn_sel(c, self.q[layer], self.page_table, self.sel[layer], self.n_sel_t, w.sm_scale,
                                    split_keys, self.pa, self.pm, self.pz)
            kvq.kvq_merge(c, self.pa, self.pm, self.pz, self.n_sel_t, n_sel, split_keys, out=self.out[layer],
                          lse=self.lse[layer])
        torch.cuda.synchronize()
        P = ctypes.c_void_p
        stream = P(torch.cuda.current_stream().cuda_stream)
        self.raw = []
        for layer, c in enumerate(mla.caches):
            d = ctypes.byref(c.desc)
            self.raw.append([
                ("kvq_decode_attn_sel", (d, P(self.q[layer].data_ptr()), H, P(self.page_table.data_ptr()),
                                         self.page_table.shape[1], P(self.sel[layer].data_ptr()),
                                         P(self.n_sel_t.data_ptr()), batch, n_sel, ctypes.c_float(w.sm_scale),
                                         split_keys, P(self.pa.data_ptr()), P(self.pm.data_ptr()),
                                         P(self.pz.data_ptr()), stream)),
                ("kvq_merge", (d, P(self.pa.data_ptr()), P(self.pm.data_ptr()), P(self.pz.data_ptr()),
                               P(self.n_sel_t.data_ptr()), batch, H, n_sel, split_keys, 0,
                               P(self.out[layer].data_ptr()), P(self.lse[layer].data_ptr()), stream)),
            ])

    @property
    def kv_bytes_per_layer(self):
        return self.batch * self.n_sel * (self.w.head_dim + 8)

    @property
    def flops_per_layer(self):
        w = self.w
        return self.batch * self.n_sel * w.n_heads * 2 * (w.head_dim + w.kv_lora)


class RowsBench(_Bench):
    """R drafted rows of the headline sequence over the 4-bit workload's layer
    caches: row r attends the first T - R + 1 + r positions.  Step per layer:
    rotate the R query rows, decode them, merge.  shared=True decodes them with
    kvq_decode_attn_rows (one page-table row, the rows of a split dispatched
    together on one XCD); shared=False with kvq_decode_attn over a batch of R
    entries repeating that row (the rows' workgroups far apart in the grid).
    Both give the same bits."""

    DECODE = 1
    DECODE_MERGE = (1, 2)

    def __init__(self, q4, n_rows, shared, device="cuda"):
        import torch

        import workloads as wl
        w, kvq = q4.w, q4.kvq
        self.w, self.kvq, self.R, self.shared = w, kvq, n_rows, shared
        T = q4.T
        self.lens = [T - n_rows + 1 + r for r in range(n_rows)]
        self.seq_lens = torch.tensor(self.lens, dtype=torch.int32, device=device)
        pt_row = q4.page_table[0].contiguous()
        self.page_table = pt_row if shared else pt_row.expand(n_rows, -1).contiguous()
        self.q = [wl.q4_query(wl.shrink(w, batch=n_rows), layer, device) for layer in range(w.n_layers)]
        acc_shape, mz_shape = kvq.partial_shapes(q4.caches[0], n_rows, w.n_q_heads, T, w.split_keys)
        f32 = dict(dtype=torch.float32, device=device)
        self.q_rot = torch.empty((n_rows, w.n_q_heads, w.head_dim), **f32)
        self.pa, self.pm, self.pz = torch.empty(acc_shape, **f32), torch.empty(mz_shape, **f32), torch.empty(mz_shape, **f32)
        self.out = torch.empty((w.n_layers, n_rows, w.n_q_heads, w.head_dim), **f32)
        self.lse = torch.empty((w.n_layers, n_rows, w.n_q_heads), **f32)
        dec = kvq.kvq_decode_attn_rows if shared else kvq.kvq_decode_attn
        for layer, c in enumerate(q4.caches):  # one checked pass through the binding
            kvq.kvq_rotate_q(self.q[layer], out=self.q_rot)
            dec(c, self.q_rot, self.page_table, self.seq_lens, T, w.sm_scale, w.split_keys, self.pa, self.pm, self.pz)
            kvq.kvq_merge(c, self.pa, self.pm, self.pz, self.seq_lens, T, w.split_keys, out=self.out[layer],
                          lse=self.lse[layer])
        torch.cuda.synchronize()
        P = ctypes.c_void_p
        stream = P(torch.cuda.current_stream().cuda_stream)
        n_pages = self.page_table.shape[-1]
        self.raw = []
        for layer, c in enumerate(q4.caches):
            d = ctypes.byref(c.desc)
            self.raw.append([
                ("kvq_rotate_q", (P(self.q[layer].data_ptr()), 0, P(self.q_rot.data_ptr()), n_rows * w.n_q_heads,
                                  w.head_dim, stream)),
                ("kvq_decode_attn_rows" if shared else "kvq_decode_attn",
                 (d, P(self.q_rot.data_ptr()), w.n_q_heads, P(self.page_table.data_ptr()), n_pages,
                  P(self.seq_lens.data_ptr()), n_rows, T, ctypes.c_float(w.sm_scale), w.split_keys,
                  P(self.pa.data_ptr()), P(self.pm.data_ptr()), P(self.pz.data_ptr()), stream)),
                ("kvq_merge", (d, P(self.pa.data_ptr()), P(self.pm.data_ptr()), P(self.pz.data_ptr()),
                               P(self.seq_lens.data_ptr()), n_rows, w.n_q_heads, T, w.split_keys, 1,
                               P(self.out[layer].data_ptr()), P(self.lse[layer].data_ptr()), stream)),
            ])

    @property
    def kv_bytes_per_layer(self):
        """Cache bytes the rows attend, counted once (the bytes one row reads)."""
        w = self.w
        return max(self.lens) * w.n_kv_heads * 2 * w.row_bytes

    flops_per_layer = None


class RaggedBench(_Bench):
    """The ragged batch: 16 sequences of seeded lengths over a shuffled paged
    pool (one layer).  Step: the 2048-token prefill chunk of a 17th sequence
    packed into its reserved pages, then kvq_decode_step (each sequence's new
    token stored and the queries rotated inside the decode launch, merge);
    the same with the store and rotation as one launch of their own
    (kvq_store_rotate_q, decode, merge) is timed too."""

    DECODE = 2
    DECODE_MERGE = (2, 3)
    EXTRA_TIMED = {"chunk_store": 0}

    def __init__(self, w, device="cuda"):
        import numpy as np
        import torch

        import fp8_quantized_kv_amd as kvq
        import workloads as wl
        self.w, self.kvq = w, kvq
        lens = wl.seq_lens(w)
        self.lens = lens
        self.T = max(lens)
        lay = wl.page_layout(w, lens)
        self.page_table = lay.page_table.to(device)
        self.seq_lens = torch.tensor(lens, dtype=torch.int32, device=device)
        c = kvq.Q4Cache(lay.num_pages, w.n_kv_heads, w.head_dim, w.page_size, device)
        self.cache = c
        off, k_last, v_last, s_last = 0, [], [], []
        for b, T in enumerate(lens):
            k, v = wl.q4_kv_tokens(w, 0, off, T, device)
            off += T
            slots = wl.slots_for(lay.page_table[b], np.arange(T), w.page_size).to(device)
            kvq.kvq_store(c, k, v, slots)
            k_last.append(k[-1:])
            v_last.append(v[-1:])
            s_last.append(slots[-1:])
        self.k_new, self.v_new, self.slot_new = torch.cat(k_last), torch.cat(v_last), torch.cat(s_last)
        self.k_chunk, self.v_chunk = wl.q4_prefill_chunk(w, 0, device)
        pages = lay.prefill_pages.to(torch.int64)
        j = torch.arange(w.prefill_chunk, dtype=torch.int64)
        self.slot_chunk = (pages[j // w.page_size] * w.page_size + j % w.page_size).to(device)
        self.q = wl.q4_query(w, 0, device)
        acc_shape, mz_shape = kvq.partial_shapes(c, w.batch, w.n_q_heads, self.T, w.split_keys)
        f32 = dict(dtype=torch.float32, device=device)
        self.q_rot = torch.empty_like(self.q)
        self.pa, self.pm, self.pz = torch.empty(acc_shape, **f32), torch.empty(mz_shape, **f32), torch.empty(mz_shape, **f32)
        self.out = torch.empty((w.batch, w.n_q_heads, w.head_dim), **f32)
        self.lse = torch.empty((w.batch, w.n_q_heads), **f32)
        kvq.kvq_store(c, self.k_chunk, self.v_chunk, self.slot_chunk)
        kvq.kvq_store_rotate_q(c, self.k_new, self.v_new, self.slot_new, self.q, out=self.q_rot)
        kvq.kvq_decode_attn(c, self.q_rot, self.page_table, self.seq_lens, self.T, w.sm_scale, w.split_keys,
                            self.pa, self.pm, self.pz)
        kvq.kvq_merge(c, self.pa, self.pm, self.pz, self.seq_lens, self.T, w.split_keys, out=self.out, lse=self.lse)
        ws_bytes = kvq.kvq_attend_workspace_bytes(c, w.batch, w.n_q_heads, self.T, w.split_keys)
        self.ws = torch.empty((ws_bytes,), dtype=torch.uint8, device=device)
        kvq.kvq_decode_step(c, self.k_new, self.v_new, self.q, self.page_table, self.seq_lens, self.T, w.sm_scale,
                            w.split_keys, workspace=self.ws, out=self.out, lse=self.lse)
        torch.cuda.synchronize()
        P = ctypes.c_void_p
        stream = P(torch.cuda.current_stream().cuda_stream)
        d = ctypes.byref(c.desc)
        dt = kvq._DTYPES[self.k_new.dtype]
        B, Hq, D = w.batch, w.n_q_heads, w.head_dim
        self.raw = [[
            ("kvq_store", (d, P(self.k_chunk.data_ptr()), P(self.v_chunk.data_ptr()), dt, P(self.slot_chunk.data_ptr()),
                           w.prefill_chunk, stream)),
            ("kvq_store_rotate_q", (d, P(self.k_new.data_ptr()), P(self.v_new.data_ptr()), dt,
                                    P(self.slot_new.data_ptr()), B, P(self.q.data_ptr()), 0, P(self.q_rot.data_ptr()),
                                    B * Hq, stream)),
            ("kvq_decode_attn", (d, P(self.q_rot.data_ptr()), Hq, P(self.page_table.data_ptr()),
                                 self.page_table.shape[1], P(self.seq_lens.data_ptr()), B, self.T,
                                 ctypes.c_float(w.sm_scale), w.split_keys, P(self.pa.data_ptr()),
                                 P(self.pm.data_ptr()), P(self.pz.data_ptr()), stream)),
            ("kvq_merge", (d, P(self.pa.data_ptr()), P(self.pm.data_ptr()), P(self.pz.data_ptr()),
                           P(self.seq_lens.data_ptr()), B, Hq, self.T, w.split_keys, 1, P(self.out.data_ptr()),
                           P(self.lse.data_ptr()), stream)),
            ("kvq_decode_step", (d, P(self.k_new.data_ptr()), P(self.v_new.data_ptr()), dt, P(self.q.data_ptr()), 0,
                                 Hq, P(self.page_table.data_ptr()), self.page_table.shape[1],
                                 P(self.seq_lens.data_ptr()), B, self.T, ctypes.c_float(w.sm_scale), w.split_keys,
                                 P(self.ws.data_ptr()), ctypes.c_size_t(self.ws.numel()), P(self.out.data_ptr()),
                                 P(self.lse.data_ptr()), stream)),
        ]]
        self.STEP = (0, 4)
        self.THREE_CALLS = self.EVENT_CALLS = (0, 1, 2, 3)

    @property
    def kv_bytes_per_layer(self):
        w = self.w
        return sum(self.lens) * w.n_kv_heads * 2 * w.row_bytes

    flops_per_layer = None


class ChunkBench(_Bench):
    """A prompt chunk (TensorFold "What it is": prompt chunks are packed, then
    attended over the decoded slots): one layer's 32K-position 4-bit cache and
    a chunk of chunk_rows rows after it.  Step: the chunk's K/V stored
    (kvq_store), its queries rotated (kvq_rotate_q), the chunk's attention as
    split partials (kvq_prefill_attn; row r attends [0, P + r]), the merge."""

    DECODE = 2
    DECODE_MERGE = (2, 3)

    def __init__(self, w, device="cuda"):
        import numpy as np
        import torch

        import fp8_quantized_kv_amd as kvq
        import workloads as wl
        self.w, self.kvq = w, kvq
        T, C = w.seq_len, w.chunk_rows
        P = T - C
        self.T, self.P, self.C = T, P, C
        lay = wl.page_layout(w, [T])
        c = kvq.Q4Cache(lay.num_pages, w.n_kv_heads, w.head_dim, w.page_size, device)
        self.cache = c
        slots = wl.slots_for(lay.page_table[0], np.arange(T), w.page_size).to(device)
        for t0 in range(0, T, 32768):
            k, v = wl.q4_kv_tokens(w, 0, t0, min(32768, T - t0), device)
            kvq.kvq_store(c, k, v, slots[t0:t0 + k.shape[0]])
            if t0 + k.shape[0] == T:
                self.k_chunk, self.v_chunk = k[-C:].contiguous(), v[-C:].contiguous()
        self.slot_chunk = slots[P:].contiguous()
        self.q = wl.q4_chunk_queries(w, 0, C, device)
        self.page_row = lay.page_table[0].to(device).contiguous()
        self.row_lens = torch.arange(P + 1, T + 1, dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        acc_shape, mz_shape = kvq.partial_shapes(c, C, w.n_q_heads, T, w.split_keys)
        self.q_rot = torch.empty_like(self.q)
        self.pa, self.pm, self.pz = torch.empty(acc_shape, **f32), torch.empty(mz_shape, **f32), torch.empty(mz_shape, **f32)
        self.out = torch.empty((C, w.n_q_heads, w.head_dim), **f32)
        self.lse = torch.empty((C, w.n_q_heads), **f32)
        # one checked pass through the binding
        kvq.kvq_store(c, self.k_chunk, self.v_chunk, self.slot_chunk)
        kvq.kvq_rotate_q(self.q, out=self.q_rot)
        kvq.kvq_prefill_attn(c, self.q_rot, self.page_row, self.row_lens, T, w.sm_scale, w.split_keys,
                             self.pa, self.pm, self.pz)
        kvq.kvq_merge(c, self.pa, self.pm, self.pz, self.row_lens, T, w.split_keys, out=self.out, lse=self.lse)
        torch.cuda.synchronize()
        P_ = ctypes.c_void_p
        stream = P_(torch.cuda.current_stream().cuda_stream)
        d = ctypes.byref(c.desc)
        Hq, D = w.n_q_heads, w.head_dim
        self.raw = [[
            ("kvq_store", (d, P_(self.k_chunk.data_ptr()), P_(self.v_chunk.data_ptr()), kvq._DTYPES[self.k_chunk.dtype],
                           P_(self.slot_chunk.data_ptr()), C, stream)),
            ("kvq_rotate_q", (P_(self.q.data_ptr()), 0, P_(self.q_rot.data_ptr()), C * Hq, D, stream)),
            ("kvq_prefill_attn", (d, P_(self.q_rot.data_ptr()), Hq, P_(self.page_row.data_ptr()),
                                  self.page_row.shape[0], P_(self.row_lens.data_ptr()), C, T,
                                  ctypes.c_float(w.sm_scale), w.split_keys, P_(self.pa.data_ptr()),
                                  P_(self.pm.data_ptr()), P_(self.pz.data_ptr()), stream)),
            ("kvq_merge", (d, P_(self.pa.data_ptr()), P_(self.pm.data_ptr()), P_(self.pz.data_ptr()),
                           P_(self.row_lens.data_ptr()), C, Hq, T, w.split_keys, 1, P_(self.out.data_ptr()),
                           P_(self.lse.data_ptr()), stream)),
        ]]

    @property
    def kv_bytes_per_layer(self):
        w = self.w
        return self.T * w.n_kv_heads * 2 * w.row_bytes

    @property
    def flops_per_layer(self):
        """Scores and context of every (row, head, attended key): 2 x 2 x D flop each."""
        w = self.w
        keys = self.C * self.P + self.C * (self.C + 1) // 2
        return 4 * w.n_q_heads * w.head_dim * keys


def capture(b, only=None):
    """The step (or the calls `only`) captured as one HIP graph on a side
    stream, after one eager run of it on that stream."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b.step(stream=ctypes.c_void_p(side.cuda_stream), only=only)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.step(stream=ctypes.c_void_p(torch.cuda.current_stream().cuda_stream), only=only)
    torch.cuda.synchronize()
    return g


def check_graph(b, g, replays=3):
    """Every replay of the step's graph, each after an eager step and a
    synchronization, reproduces the eager step's outputs bit for bit."""
    import torch
    b.step()
    torch.cuda.synchronize()
    ref = b.outputs()
    for _ in range(replays):
        b.out.zero_()
        b.lse.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = b.outputs()
        if not (torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])):
            raise RuntimeError("graph replay differs from the eager step")
        b.step()
        torch.cuda.synchronize()


def time_graph(g, steps, warmup):
    """ms per replay of `steps` back-to-back replays after `warmup` replays."""
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(steps):
        g.replay()
    t_end.record()
    torch.cuda.synchronize()
    return t_start.elapsed_time(t_end) / steps, time.perf_counter() - wall0


def time_steps(b, steps, warmup, only=None):
    """ms per step of `steps` uninstrumented steps (of the calls `only`, if
    given) after `warmup` warm-up steps."""
    import torch
    for _ in range(warmup):
        b.step(only=only)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for _ in range(steps):
        b.step(only=only)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return t_start.elapsed_time(t_end) / steps, wall


def time_decode(b, steps, which=None):
    """Average launch of call `which` (default: the decode) in ms: `steps` more
    steps with that launch bracketed by HIP events in every layer.  (Event
    records stall the queue for a few microseconds, so these steps are not
    the ones whose time is reported.)"""
    import torch
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(b.w.n_layers)] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        b.step(ev[s], which, only=b.EVENT_CALLS)
    torch.cuda.synchronize()
    d = [e0.elapsed_time(e1) for row in ev for (e0, e1) in row]
    return sum(d) / len(d)


def settle(b, min_ms=50.0):
    """Untimed steps for at least min_ms of GPU time: a side workload's first
    timing right after its setup ran several percent slow when its warm-up
    was only a few short steps."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done = 0.0
    while done < min_ms:
        e0.record()
        for _ in range(10):
            b.step()
        e1.record()
        torch.cuda.synchronize()
        done += e0.elapsed_time(e1)


def measure(b, steps, warmup, side=False):
    """The eager step; decode + merge alone; the step replayed as one HIP
    graph (each replay first checked against the eager step's outputs); and
    the decode launch (and other calls to time) by events.  Side workloads
    (side=True) first run settle()."""
    import torch
    if side:
        settle(b)
    ms_step, wall = time_steps(b, steps, warmup)
    ms_three = time_steps(b, steps, warmup, only=b.THREE_CALLS)[0] if getattr(b, "THREE_CALLS", None) else None
    ms_dm, _ = time_steps(b, steps, warmup, only=b.DECODE_MERGE)
    g = capture(b)
    check_graph(b, g)
    ms_graph, _ = time_graph(g, steps, warmup)
    del g
    torch.cuda.synchronize()
    L = b.w.n_layers
    # The decode's average launch: steps of decode launches alone, back to back
    # between two events (region time / launches; inter-launch gaps included).
    ms_dec, _ = time_steps(b, steps, warmup, only=(b.DECODE,))
    dec_ms = ms_dec / L
    # The same launches each bracketed by its own event pair (adds the event
    # records' own cost, about 1.5 us per launch).
    dec_ms_bracketed = time_decode(b, steps)
    kvb = b.kv_bytes_per_layer
    r = {"ms_per_step": ms_step, "us_per_layer": ms_step * 1e3 / L, "decode_us": dec_ms * 1e3,
         "decode_us_bracketed": dec_ms_bracketed * 1e3,
         "decode_merge_us_per_layer": ms_dm * 1e3 / L, "graph_us_per_layer": ms_graph * 1e3 / L,
         "step_gbs": kvb * L / (ms_step * 1e-3) / 1e9, "decode_gbs": kvb / (dec_ms * 1e-3) / 1e9, "wall_s": wall}
    if ms_three is not None:
        r["us_per_layer_three_launches"] = ms_three * 1e3 / L
    if b.flops_per_layer:
        r["decode_tflops"] = b.flops_per_layer / (dec_ms * 1e-3) / 1e12
    for name, idx in b.EXTRA_TIMED.items():
        r[name + "_us"] = time_decode(b, steps, idx) * 1e3
    return r


def read_ceiling(gib=2, batches=3, per_batch=5):
    """HBM read rate of kvq_stream_read over a buffer well above the last-level
    cache, with the non-temporal hint and with the default cache policy
    (median over `batches` event-timed runs of `per_batch` back-to-back
    launches, GB/s)."""
    import torch

    import fp8_quantized_kv_amd as kvq
    buf = torch.ones((gib << 30,), dtype=torch.uint8, device="cuda")
    res = torch.zeros((1,), dtype=torch.int32, device="cuda")
    out = {"kernel": "kvq_stream_read (LDS DMA, 16 KiB per workgroup step)", "bytes": buf.numel(), "unit": "GB/s"}
    for name, nt in (("non_temporal", True), ("default_policy", False)):
        kvq.kvq_stream_read(buf, nt, res)  # warm-up
        times = []
        for _ in range(batches):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(per_batch):
                kvq.kvq_stream_read(buf, nt, res)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) / per_batch)
        ms = sorted(times)[len(times) // 2]
        out[name] = round(buf.numel() / (ms * 1e-3) / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, sample_tokens, min_seconds=10.0, max_repeats=60):
    """The oracle (fp64, OpenMP over heads) on one layer of the workload,
    restricted to its first `sample_tokens` positions; repeated until about
    `min_seconds` of CPU work have run, median reported."""
    import numpy as np

    import oracle
    import workloads as wl
    T = min(sample_tokens, w.seq_len)
    lay = wl.page_layout(wl.shrink(w, seq_len=T), [T])
    shape = oracle.q4_pool_shape(lay.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    kp, vp = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
    q = wl.q4_query(w, 0)
    for t0 in range(0, T, 32768):
        n = min(32768, T - t0)
        k, v = wl.q4_kv_tokens(w, 0, t0, n)
        wl.plant(w, k, q, t0)
        oracle.q4_store(kp, vp, k.float().numpy(), v.float().numpy(), np.arange(t0, t0 + n), w.page_size)
    times = []
    while len(times) < max_repeats and (len(times) < 3 or sum(times) < min_seconds):
        t0 = time.perf_counter()
        oracle.q4_attention(kp, vp, q.numpy(), lay.page_table.numpy(), np.array([T], np.int32), w.sm_scale)
        times.append(time.perf_counter() - t0)
    repeats = len(times)
    dt = sorted(times)[len(times) // 2]
    kv_bytes = T * w.n_kv_heads * 2 * w.row_bytes
    threads = min(oracle.num_threads(), w.batch * w.n_q_heads)
    return {"value": round(kv_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"layer 0 of {w.name}, first {T} positions, all {w.n_q_heads} query heads "
                      f"(decode attention + merge in fp64; median {dt:.3f} s of {repeats} runs, {sum(times):.1f} s in all)",
            "seconds": round(dt, 3)}


def _median_timing(fn, min_seconds, max_repeats=50):
    """Median wall time (s) of fn() repeated until about min_seconds have run."""
    times = []
    while len(times) < max_repeats and (len(times) < 3 or sum(times) < min_seconds):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return sorted(times)[len(times) // 2], len(times)


def cpu_per_config(min_seconds=1.0):
    """The oracle timed on a bounded sample of each workload configuration
    (decode attention + merge in fp64, KV bytes read per second), and its
    store (rotate + quantise + pack in fp32) in cache rows per second, a row
    being one (token, KV head) K or V vector."""
    import numpy as np

    import oracle
    import workloads as wl
    out = {}

    def q4_pools(w, lens):
        lay = wl.page_layout(w, lens)
        shape = oracle.q4_pool_shape(lay.num_pages, w.n_kv_heads, w.page_size, w.head_dim, w.bits)
        kp, vp = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
        off = 0
        for b, T in enumerate(lens):
            for t0 in range(0, T, 32768):
                n = min(32768, T - t0)
                k, v = wl.q4_kv_tokens(w, 0, off + t0, n)
                slots = wl.slots_for(lay.page_table[b], np.arange(t0, t0 + n), w.page_size).numpy()
                oracle.q4_store(kp, vp, k.float().numpy(), v.float().numpy(), slots, w.page_size)
            off += T
        return lay, kp, vp

    # 4-bit dense configurations: tiny (whole), 32K (whole), ragged (first two sequences)
    for name, lens in (("tiny_q4_d128_t1024", None), ("gqa_q4_32k", None), ("gqa_q8_32k", None), ("gqa_q6_32k", None),
                       ("ragged_q4_b16", "first2")):
        w = wl.WORKLOADS[name]
        if lens is None:
            lens = [w.seq_len] * w.batch
            sample = f"all {sum(lens)} positions"
        else:
            lens = [int(x) for x in wl.seq_lens(w)[:2]]
            sample = f"sequences 0-1 of the batch ({lens[0]} and {lens[1]} positions)"
        lay, kp, vp = q4_pools(w, lens)
        q = wl.q4_query(wl.shrink(w, batch=len(lens)), 0).numpy()
        sl = np.array(lens, np.int32)
        dt, n = _median_timing(lambda: oracle.q4_attention(kp, vp, q, lay.page_table.numpy(), sl, w.sm_scale),
                               min_seconds)
        kvb = sum(lens) * w.n_kv_heads * 2 * w.row_bytes
        out[name] = {"value": round(kvb / dt / 1e9, 4), "unit": "GB/s", "seconds": round(dt, 4), "runs": n,
                     "sample": sample + f", all {w.n_q_heads} query heads"}
    # fp8 latent: the first 4096 positions of the 262K context, all 128 heads
    w = wl.MLA_262K
    T = 4096
    lay = wl.page_layout(wl.shrink(w, seq_len=T), [T])
    n_slots = lay.num_pages * w.page_size
    codes, scales = np.zeros((n_slots, w.head_dim), np.uint8), np.zeros((n_slots, 2), np.float32)
    x = wl.mla_rows(w, 0, 0, T).numpy()
    slots = wl.slots_for(lay.page_table[0], np.arange(T), w.page_size).numpy()
    oracle.fp8_store(codes, scales, x, slots, w.rope_dim)
    q = wl.mla_query(w, 0).numpy()
    dt, n = _median_timing(lambda: oracle.mla_attention(codes, scales, q, lay.page_table.numpy(),
                                                         np.array([T], np.int32), w.sm_scale, w.rope_dim,
                                                         w.page_size), min_seconds)
    out["mla_fp8_262k"] = {"value": round(T * MlaBench.ROW_BYTES / dt / 1e9, 4), "unit": "GB/s", "seconds": round(dt, 4),
                           "runs": n, "sample": f"first {T} of {w.seq_len} positions, all {w.n_heads} heads"}
    # stores, rows per second: 4096 tokens of the 4-bit shape (4 KV heads, K and V) and of the latent
    w = wl.GQA_262K
    n_tok = 4096
    lay = wl.page_layout(wl.shrink(w, seq_len=n_tok), [n_tok])
    shape = oracle.q4_pool_shape(lay.num_pages, w.n_kv_heads, w.page_size, w.head_dim)
    kp, vp = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
    k, v = wl.q4_kv_tokens(w, 0, 0, n_tok)
    k, v = k.float().numpy(), v.float().numpy()
    sl = np.arange(n_tok)
    dt, n = _median_timing(lambda: oracle.q4_store(kp, vp, k, v, sl, w.page_size), min_seconds)
    rows = n_tok * w.n_kv_heads * 2
    out["store_q4"] = {"value": round(rows / dt, 1), "unit": "rows/s", "seconds": round(dt, 4), "runs": n,
                       "sample": f"{n_tok} tokens x {w.n_kv_heads} KV heads x (K, V), head_dim {w.head_dim}"}
    w = wl.MLA_262K
    x = wl.mla_rows(w, 0, 0, n_tok).numpy()
    codes, scales = np.zeros((n_tok, w.head_dim), np.uint8), np.zeros((n_tok, 2), np.float32)
    dt, n = _median_timing(lambda: oracle.fp8_store(codes, scales, x, sl, w.rope_dim), min_seconds)
    out["store_fp8"] = {"value": round(n_tok / dt, 1), "unit": "rows/s", "seconds": round(dt, 4), "runs": n,
                        "sample": f"{n_tok} latent rows of {w.kv_lora} + {w.rope_dim}"}
    return out


def gpu_store_rates(steps=20):
    """kvq_store throughput on the GPU in cache rows per second (a row = one
    (token, KV head) K or V vector, or one latent row), for a 32768-token
    chunk of the 4-bit shape and of the fp8 latent, event-timed over `steps`
    back-to-back calls."""
    import numpy as np
    import torch

    import fp8_quantized_kv_amd as kvq
    import workloads as wl
    out = {}
    n_tok = 32768
    w = wl.GQA_262K
    lay = wl.page_layout(wl.shrink(w, seq_len=n_tok), [n_tok])
    c = kvq.Q4Cache(lay.num_pages, w.n_kv_heads, w.head_dim, w.page_size, "cuda")
    k, v = wl.q4_kv_tokens(w, 0, 0, n_tok, "cuda")
    slots = wl.slots_for(lay.page_table[0], np.arange(n_tok), w.page_size).cuda()
    wm = wl.MLA_262K
    cl = kvq.Fp8Cache(lay.num_pages, wm.head_dim, wm.rope_dim, wm.page_size, "cuda")
    x = wl.mla_rows(wm, 0, 0, n_tok, "cuda")
    for name, fn, rows, what in (
            ("store_q4", lambda: kvq.kvq_store(c, k, v, slots), n_tok * w.n_kv_heads * 2,
             f"{n_tok} tokens x {w.n_kv_heads} KV heads x (K, V), {str(k.dtype).split('.')[-1]} rows of {w.head_dim}"),
            ("store_fp8", lambda: kvq.kvq_store(cl, x, None, slots), n_tok,
             f"{n_tok} latent rows of {wm.kv_lora} + {wm.rope_dim}, {str(x.dtype).split('.')[-1]}")):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        out[name] = {"value": round(rows / (us * 1e-6), 1), "unit": "rows/s", "us_per_call": round(us, 3),
                     "sample": what}
    del c, cl
    torch.cuda.empty_cache()
    return out


def profile_run(name, steps, warmup):
    """One workload's step, `warmup` + `steps` times with nothing else in the
    process: the command the rocprofv3 summaries under profiles/ run."""
    import torch

    import workloads as wl
    w = wl.WORKLOADS[name]
    cls = {"ragged_q4_b16": RaggedBench, "chunk_q4_32k": ChunkBench, "mla_fp8_262k": MlaBench,
           "mla_tq4_262k": TqBench, "mla_tq4_32k": TqBench}.get(name, Q4Bench)
    torch.cuda.set_device(0)
    b = cls(w)
    ms, _ = time_steps(b, steps, warmup)
    print(json.dumps({"profile": name, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
                      "us_per_layer": round(ms * 1e3 / w.n_layers, 3)}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 50 untimed steps (about 50 ms at 262K): after the setup the first timed steps ran ~4% slower
    # with 3 warm-up steps than with 50 (61.1-61.5 vs 58.9-59.0 us per layer); later timings in
    # the same run did not move
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gqa_q4_262k")
    ap.add_argument("--cpu-sample-tokens", type=int, default=262144)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the 32K and fp8-latent side measurements")
    ap.add_argument("--profile-workload", metavar="NAME",
                    help="only run NAME's step (--warmup + --steps times) and print its time: for profilers")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the decode path is "
              "built and measured for a single GPU's share of the work", file=sys.stderr)
        sys.exit(2)
    if args.profile_workload:
        profile_run(args.profile_workload, args.steps, args.warmup)
        return

    import torch

    import workloads as wl
    w = wl.WORKLOADS[args.workload]
    assert isinstance(w, wl.Q4Workload), "the headline benchmark is the 4-bit decode"
    torch.cuda.set_device(0)
    _log(f"bench: setting up {w.name} ({w.n_layers} layers, T={w.seq_len})")
    b = Q4Bench(w)
    _log(f"bench: timing {args.steps} steps after {args.warmup} warm-up steps "
         f"(then decode + merge alone, the step as a HIP graph, {args.steps} event-bracketed steps)")
    m = measure(b, args.steps, args.warmup)
    kvb = b.kv_bytes_per_layer
    rows = {}
    if not args.no_extras:
        # drafted rows of the same sequence over the same layer caches (shared vs separate reads)
        for R in (4,):
            for shared in (True, False):
                name = f"rows{R}_q4_262k_{'shared' if shared else 'batch'}"
                _log(f"bench: side measurement {name}")
                br = RowsBench(b, R, shared)
                mr = measure(br, args.steps, args.warmup, side=True)
                rows[name] = {"rows": R, "lens": f"{min(br.lens)}..{max(br.lens)}", "split_keys": w.split_keys,
                              "entry": "kvq_decode_attn_rows" if shared else "kvq_decode_attn (page-table row repeated)",
                              "us_per_layer": round(mr["us_per_layer"], 3),
                              "decode_us": round(mr["decode_us"], 3),
                              "decode_us_per_row": round(mr["decode_us"] / R, 3),
                              "decode_vs_one_row": round(mr["decode_us"] / m["decode_us"], 3)}
                del br
    rec = {
        "metric": METRIC, "value": round(m["step_gbs"], 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(m["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16 MFMA operands, f32 accumulate", "data": "synthetic",
        "config": {"workload": w.name, "layers": w.n_layers, "batch": w.batch, "seq_len": w.seq_len,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "split_keys": w.split_keys, "kv_bytes_per_layer": kvb},
        "us_per_layer": round(m["us_per_layer"], 3),
        "step_entry": ("kvq_decode_step (store and query rotation inside the decode launch, then the merge)"
                       if b.fused else "kvq_store_rotate_q, kvq_decode_attn, kvq_merge"),
        "decode_merge_us_per_layer": round(m["decode_merge_us_per_layer"], 3),
        "graph_us_per_layer": round(m["graph_us_per_layer"], 3),
        "pct_hbm_peak": round(100 * m["step_gbs"] / HBM_PEAK_GBS, 2),
        "roofline": {"kernel": "kvq_decode_attn (4-bit split-K)", "bound": "hbm",
                     "achieved": round(m["decode_gbs"], 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(m["decode_gbs"] / HBM_PEAK_GBS, 4), "avg_launch_us": round(m["decode_us"], 3),
                     "avg_launch_us_event_pair_each": round(m["decode_us_bracketed"], 3),
                     "traffic": decode_traffic(),
                     "traffic_source": "rocprofv3 FETCH_SIZE and WRITE_SIZE of this kernel build, calibrated by a "
                                       "256 MiB copy (profiles/decode_q4_mfma_gqa_q4_262k.md); null when the kernel "
                                       "sources differ from the build the counters were taken on"},
        "wall_s": round(m["wall_s"], 3),
    }
    if "us_per_layer_three_launches" in m:
        rec["us_per_layer_three_launches"] = round(m["us_per_layer_three_launches"], 3)
    del b
    torch.cuda.empty_cache()
    _log("bench: HBM read ceiling (kvq_stream_read over 2 GiB)")
    ceil = read_ceiling()
    rec["hbm_read_ceiling"] = ceil
    rec["roofline"]["frac_of_read_ceiling"] = round(m["decode_gbs"] / ceil["non_temporal"], 4)
    if rows:
        rec["drafted_rows"] = rows
    if not args.no_extras:
        extras = {}
        for name, cls in (("gqa_q4_32k", Q4Bench), ("gqa_q8_32k", Q4Bench), ("gqa_q6_32k", Q4Bench),
                          ("ragged_q4_b16", RaggedBench), ("chunk_q4_32k", ChunkBench), ("mla_fp8_262k", MlaBench),
                          ("mla_tq4_262k", TqBench), ("mla_tq4_32k", TqBench)):
            wx = wl.WORKLOADS[name]
            _log(f"bench: side measurement {name}")
            bx = cls(wx)
            steps = max(3, min(args.steps, 10)) if issubclass(cls, MlaBench) else args.steps
            mx = measure(bx, steps, args.warmup, side=True)
            e = {"layers": wx.n_layers, "seq_len": wx.seq_len or f"{min(bx.lens)}..{max(bx.lens)} x {len(bx.lens)}",
                 "split_keys": wx.split_keys, "steps": steps,
                 "kv_bytes_per_layer": bx.kv_bytes_per_layer, "us_per_layer": round(mx["us_per_layer"], 3),
                 "decode_merge_us_per_layer": round(mx["decode_merge_us_per_layer"], 3),
                 "graph_us_per_layer": round(mx["graph_us_per_layer"], 3),
                 "step_kv_gbs": round(mx["step_gbs"], 2), "decode_us": round(mx["decode_us"], 3),
                 "decode_kv_gbs": round(mx["decode_gbs"], 2),
                 "decode_frac_hbm": round(mx["decode_gbs"] / HBM_PEAK_GBS, 4)}
            if "decode_tflops" in mx:
                e["decode_tflops"] = round(mx["decode_tflops"], 2)
            if "us_per_layer_three_launches" in mx:
                e["us_per_layer_three_launches"] = round(mx["us_per_layer_three_launches"], 3)
            if getattr(bx, "STEP", None) and "kvq_decode_step" in [bx.raw[0][i][0] for i in bx.STEP]:
                e["step_entry"] = "kvq_decode_step"
            if cls is ChunkBench:
                # the chunk's attention is a dense contraction: its roofline is the f16 matrix-core peak
                e["chunk_rows"] = wx.chunk_rows
                e["attended_keys"] = int(bx.flops_per_layer // (4 * wx.n_q_heads * wx.head_dim))
                e["roofline"] = {"kernel": "kvq_prefill_attn", "bound": "mfma", "achieved": round(mx["decode_tflops"], 2),
                                 "peak": 2500.0, "unit": "TFLOP/s",
                                 "frac": round(mx["decode_tflops"] / 2500.0, 4)}
            if "chunk_store_us" in mx:
                e["chunk_store_us"] = round(mx["chunk_store_us"], 3)
                # 2048 tokens x 4 KV heads x (K, V): bf16 rows in, 144-byte rows out
                cb = wx.prefill_chunk * wx.n_kv_heads * 2 * (2 * wx.head_dim + wx.row_bytes)
                e["chunk_store_gbs"] = round(cb / (mx["chunk_store_us"] * 1e-6) / 1e9, 2)
            extras[name] = e
            if cls is MlaBench:
                # selected rows (DSA gather) over the same layer caches
                # splits as measured best: short lists need short splits to give the GPU workgroups
                for n_sel, batch, split in ((2048, 1, 64), (4096, 1, 64), (2048, 16, 256)):
                    dname = f"dsa_fp8_262k_sel{n_sel}_b{batch}"
                    _log(f"bench: side measurement {dname}")
                    bd = DsaBench(bx, n_sel, batch, split)
                    md = measure(bd, args.steps, args.warmup, side=True)
                    extras[dname] = {
                        "layers": wx.n_layers, "context": wx.seq_len, "batch": batch, "n_sel": n_sel,
                        "split_keys": split, "steps": args.steps,
                        "gathered_bytes_per_layer": bd.kv_bytes_per_layer,
                        "us_per_layer": round(md["us_per_layer"], 3),
                        "graph_us_per_layer": round(md["graph_us_per_layer"], 3),
                        "decode_us": round(md["decode_us"], 3),
                        "decode_gathered_gbs": round(md["decode_gbs"], 2),
                        "decode_tflops": round(md["decode_tflops"], 2),
                        "note": "decode over the selection + merge per layer; the batch shares the layer's "
                                "context; the gathered rows stay cache-resident across steps"}
                    del bd
            del bx
            torch.cuda.empty_cache()
        rec["extras"] = extras
    if not args.no_extras:
        _log("bench: kvq_store throughput (rows/s)")
        rec["store"] = gpu_store_rates()
    if not args.no_cpu_baseline:
        _log(f"bench: oracle CPU baseline on {args.cpu_sample_tokens} positions, then per configuration")
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_tokens)
        rec["cpu_baseline"]["per_config"] = cpu_per_config()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
