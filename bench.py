"""Benchmark of the rotated INT4 paged KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the whole hot path over the Llama-3-8B-shaped layer
(32 query / 8 KV heads, head_dim 128, batch 64 x 4096 context, page 16,
Hadamard block 64): append one new token per sequence (rotate + quantize +
scatter) and run paged decode attention over the 4096-token context.  Inputs
are resident in HBM; successive steps cycle through RING copies of the cache
so the 256 MB Infinity Cache cannot hold the working set.

Prints one JSON line.  ``value`` is the INT4 decode attention rate in GB/s of
algorithmic bytes (packed codes + fp16 sidecars + query + output + page table)
over the measured decode time; the same line carries the prefill
rotate+quantize rate (Mtokens/s, 32768 ragged tokens), plain-INT4 and bf16-KV
comparisons, the roofline of the decode kernel and the CPU oracle timed on a
bounded sample.

The Hadamard-block variants (0 = plain INT4, 16, 32, 64, 128) are each timed
alone in a decode-only loop, and ``rotated_over_plain_decode`` compares block
64 with plain INT4 under that same loop.

Other modes (for rocprofv3 runs): ``--mode decode`` times only the headline
decode; ``--mode prefill`` only the prefill append; ``--mode concurrency``
only the concurrency sweep; ``--mode serving --batch B --cache C`` the
70B-shaped serving step of one batch size and cache kind; ``--mode variant
--cache C`` one decode variant (int8, int4g64, mxfp4, windowed, bf16) on the
headline workload; ``--mode ceiling`` what the memory system gives the
path's access patterns (probe kernels); ``--mode quality`` the accuracy
report alone (reconstruction and attention error of every cache kind on the
prefill, long-context and serving data; also in the full line); ``--mode
copy`` runs a plain 1 GiB device copy used to calibrate the FETCH_SIZE /
WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
METRIC = "INT4-KV decode attn HBM GB/s (% of peak); rotate+quant Mtokens/s"
RING = 4
PREFILL_RING = 8   # prefill input/cache sets: 8 x 170 MB, well past the Infinity Cache
PREFILL_SEEDS = (3, 13, 23, 33, 43, 63, 93, 103)   # seeds whose length draws stay in [512, 4096]


# ---------------------------------------------------------------- accounting

def overhead_bits(bits: int, group: int) -> float:
    """Bits of a per-group parameter averaged over the numbers of the group."""
    return bits / group


def int4_bytes_per_vector(d: int) -> int:
    """Stored bytes of one (token, KV head, K|V) vector: D nibbles + fp16 scale + fp16 zero."""
    return d // 2 + 4


def decode_bytes(seq_lens, hkv, hq, d, kv_bytes_per_vector, q_bytes=2, page=16) -> int:
    """Algorithmic HBM bytes of one decode call: K and V of every context token,
    the query, the fp32 output, the page-table entries used and seq_lens."""
    toks = int(sum(int(x) for x in seq_lens))
    pages = int(sum((int(x) + page - 1) // page for x in seq_lens))
    b = len(seq_lens)
    return toks * hkv * 2 * kv_bytes_per_vector + b * hq * d * (q_bytes + 4) + pages * 4 + b * 4


def append_bytes(tokens, hkv, d, kv_bytes_per_vector, in_bytes=2) -> int:
    """Algorithmic HBM bytes of one append: read K and V, the slot map, write the
    stored vectors."""
    return tokens * hkv * 2 * d * in_bytes + tokens * 4 + tokens * hkv * 2 * kv_bytes_per_vector


# ---------------------------------------------------------------- helpers

def _src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_kv_cache_block_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


DECODE_SOURCES = ("decode_int4.hip", "decode_int4_launch.hpp", "decode_int4_body.hpp", "dev_common.hpp", "kvq_internal.hpp")


def _traffic(alg_bytes: int):
    """HBM bytes per launch of the decode kernel from the committed counter
    record (calibrated FETCH_SIZE + WRITE_SIZE), or None when the kernel's
    sources changed after the counters were taken."""
    path = os.path.join(ROOT, "profiles", "counters_decode_int4_llama8b.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    if rec.get("source_sha") != _src_hash(*DECODE_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


def _time_back_to_back(torch, fn, iters):
    """Mean ms per call of iters consecutive calls of fn() between one pair of
    HIP events on the current stream (no event between the calls)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def _time_events(torch, fn, iters):
    """Mean ms of fn() over iters launches, HIP events on the current stream."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(iters)]
    for i in range(iters):
        starts[i].record()
        fn(i)
        ends[i].record()
    torch.cuda.synchronize()
    ms = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return sum(ms) / len(ms), ms[len(ms) // 2]


class DecodeBench:
    """Full-size Llama-3-8B layer: RING cache copies, per-step new tokens."""

    def __init__(self, torch, kvq, workloads, block, seed=2):
        self.torch, self.kvq = torch, kvq
        dev = "cuda"
        w = workloads.llama8b_decode(seed, device=dev, batch=64, context=4096, block=block)
        self.w = w
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.sl = torch.from_numpy(w.seq_lens).to(dev)
        self.ws = torch.empty(max(16, kvq.kvq_decode_workspace_bytes(w.batch, w.hq, w.hkv, w.d,
                                                                     w.max_seq_len)),
                              dtype=torch.uint8, device=dev)
        self.out = torch.empty((w.batch, w.hq, w.d), dtype=torch.float32, device=dev)
        # per-step new token (position 4095 of every sequence) and query
        g = torch.Generator(device=dev)
        g.manual_seed(77)
        last = (w.token_pos == w.seq_lens[w.token_seq] - 1)
        self.new_slots = w.slot_mapping[torch.from_numpy(last).to(dev)].contiguous()
        shape = (RING, w.batch, w.hkv, w.d)
        self.knew = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
        self.vnew = torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)
        self.qs = torch.randn((RING, w.batch, w.hq, w.d), generator=g, device=dev).to(torch.bfloat16)
        self.block = block
        self.int4 = [kvq.Int4Cache(w.num_pages, w.hkv, w.d, block, dev) for _ in range(RING)]
        for c in self.int4:
            kvq.kvq_append_paged(c, w.k, w.v, w.slot_mapping)
        self.bf16 = None
        torch.cuda.synchronize()

    def refill(self, block):
        w, kvq = self.w, self.kvq
        self.block = block
        for c in self.int4:
            c.hadamard_block = block
            kvq.kvq_append_paged(c, w.k, w.v, w.slot_mapping)
        self.torch.cuda.synchronize()

    def make_bf16(self):
        w, kvq = self.w, self.kvq
        self.bf16 = [kvq.Bf16Cache(w.num_pages, w.hkv, w.d, "cuda") for _ in range(2)]
        for c in self.bf16:
            kvq.kvq_append_paged_bf16(c, w.k, w.v, w.slot_mapping)
        self.torch.cuda.synchronize()

    def append(self, i):
        self.kvq.kvq_append_paged(self.int4[i % RING], self.knew[i % RING], self.vnew[i % RING],
                                  self.new_slots)

    def decode(self, i):
        w = self.w
        self.kvq.kvq_decode_attn(self.int4[i % RING], self.qs[i % RING], self.bt, self.sl,
                                 w.max_seq_len, w.sm_scale, out=self.out, workspace=self.ws)

    def decode_bf16(self, i):
        w = self.w
        self.kvq.kvq_decode_attn_bf16(self.bf16[i % 2], self.qs[i % RING], self.bt, self.sl,
                                      w.max_seq_len, w.sm_scale, out=self.out, workspace=self.ws)

    def free(self):
        self.int4 = self.bf16 = None
        self.torch.cuda.empty_cache()


def prefill_rates(torch, kvq, workloads, blocks=(64, 0), iters=50, chunk=10):
    """Rotate+quantize append of 32768 ragged tokens (8 KV heads, d 128) into a
    page-16 pool, for each Hadamard block in ``blocks``: Mtokens/s and GB/s
    over PREFILL_RING input/cache sets.  The blocks are timed in alternating runs of
    ``chunk`` consecutive calls so that they see the same clocks: ``us`` is the
    mean per call of a run timed as a whole (one event pair around the run,
    as a prefill appends layer after layer), ``us_per_call_events`` the mean
    with an event pair around every call (which adds the events' gap between
    calls)."""
    sets = {}
    for blk in blocks:
        sets[blk] = []
        for r in range(PREFILL_RING):
            w = workloads.prefill_append(PREFILL_SEEDS[r], device="cuda", block=blk)
            sets[blk].append((w, kvq.Int4Cache(w.num_pages, w.hkv, w.d, blk, "cuda")))

    def run(blk, i):
        w, c = sets[blk][i % PREFILL_RING]
        kvq.kvq_append_paged(c, w.k, w.v, w.slot_mapping)

    for blk in blocks:
        for i in range(10):
            run(blk, i)
    tot = {blk: [] for blk in blocks}
    per_call = {blk: [] for blk in blocks}
    for i0 in range(0, iters, chunk):
        for blk in blocks:
            n = min(chunk, iters - i0)
            tot[blk].append((_time_back_to_back(torch, lambda i: run(blk, i0 + i), n), n))
        for blk in blocks:
            n = min(chunk, iters - i0)
            mean_ms, _ = _time_events(torch, lambda i: run(blk, i0 + i), n)
            per_call[blk].append((mean_ms, n))
    res = {}
    for blk in blocks:
        mean_ms = sum(m * n for m, n in tot[blk]) / sum(n for _, n in tot[blk])
        ev_ms = sum(m * n for m, n in per_call[blk]) / sum(n for _, n in per_call[blk])
        w = sets[blk][0][0]
        tok = w.num_tokens
        nbytes = append_bytes(tok, w.hkv, w.d, int4_bytes_per_vector(w.d))
        res[blk] = {"mtok_s": tok / (mean_ms * 1e-3) / 1e6, "gb_s": nbytes / (mean_ms * 1e-3) / 1e9,
                    "us": mean_ms * 1e3, "us_per_call_events": ev_ms * 1e3, "bytes": nbytes, "tokens": tok}
    return res


def windowed_bytes(seq_lens, hkv, hq, d, w_total, page=16) -> int:
    """Algorithmic bytes of a decode with high-precision windows of w_total
    tokens: INT4 tokens outside the windows, bf16 tokens inside, the query,
    the fp32 output, both page tables and seq_lens."""
    b = len(seq_lens)
    win = sum(min(int(x), w_total) for x in seq_lens)
    toks = sum(int(x) for x in seq_lens)
    pages = sum((int(x) + page - 1) // page for x in seq_lens)
    wpages = b * ((w_total + page - 1) // page)
    return ((toks - win) * hkv * 2 * int4_bytes_per_vector(d) + win * hkv * 2 * d * 2
            + b * hq * d * (2 + 4) + (pages + wpages) * 4 + b * 4)


def windowed_rate(torch, kvq, workloads, db, iters, plain_gb_s, plain_bytes, w_sink=4, w_recent=124):
    """The headline workload decoded with bf16 windows of the first 4 and the
    last 124 tokens (128 in all, as in InnerQ Figure 5) next to the INT4 cache
    (Hadamard block 64), decode-only loop over the cache ring."""
    w = db.w
    rng = __import__("numpy").random.default_rng(9)
    wbt, npages = workloads.window_layout(w.batch, w_sink, w_recent, rng)
    slots = workloads.window_slots(wbt, w.token_seq, w.token_pos, w.seq_lens, w_sink, w_recent)
    sl_dev = torch.from_numpy(slots).to("cuda")
    wins = []
    for _ in range(RING):
        c = kvq.Bf16Cache(npages, w.hkv, w.d, "cuda")
        kvq.kvq_append_paged_bf16(c, w.k, w.v, sl_dev)
        wins.append(c)
    wbt_dev = torch.from_numpy(wbt).to("cuda")
    ws = torch.empty(kvq.kvq_decode_windowed_workspace_bytes(w.batch, w.hq, w.hkv, w.d, w.max_seq_len),
                     dtype=torch.uint8, device="cuda")

    def run(i):
        kvq.kvq_decode_attn_windowed(db.int4[i % RING], wins[i % RING], db.qs[i % RING], db.bt, wbt_dev,
                                     db.sl, w.max_seq_len, w_sink, w_recent, w.sm_scale, out=db.out,
                                     workspace=ws)

    for i in range(10):
        run(i)
    ms, _ = _time_events(torch, run, iters)
    nbytes = windowed_bytes(w.seq_lens, w.hkv, w.hq, w.d, w_sink + w_recent)
    plain_us = plain_bytes / (plain_gb_s * 1e9) * 1e6
    del wins
    return {"w_sink": w_sink, "w_recent": w_recent, "us": round(ms * 1e3, 2), "bytes": nbytes,
            "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "time_over_int4_block64": round(ms * 1e3 / plain_us, 4)}


def variant_rates(torch, kvq, workloads, db, iters, int4_gb_s, int4_bytes, kind):
    """A cache variant on the headline workload (Hadamard block 64):
    decode-only loop over two cache copies (timed per call with an event pair
    around each, and as one run of back-to-back calls), and the prefill append of 32768
    ragged tokens over PREFILL_RING input/cache sets (consecutive calls timed
    as a whole).  kind "int8": token-wise INT8
    (D code bytes + 4 sidecar bytes per vector); "int4g64": INT4 with one
    scale/zero per 64 channels (D/2 + 4 D/64 bytes); "mxfp4": E2M1 codes with
    one E8M0 byte per 32 channels (D/2 + D/32 bytes)."""
    w = db.w
    if kind == "int8":
        make = lambda nb: kvq.Int8Cache(nb, w.hkv, w.d, 64, "cuda")
        app_fn, dec_fn, vec_bytes = kvq.kvq_append_paged_int8, kvq.kvq_decode_attn_int8, w.d + 4
    elif kind == "mxfp4":
        make = lambda nb: kvq.MxFp4Cache(nb, w.hkv, w.d, 64, "cuda")
        app_fn, dec_fn, vec_bytes = kvq.kvq_append_paged_mxfp4, kvq.kvq_decode_attn_mxfp4, w.d // 2 + w.d // 32
    else:
        make = lambda nb: kvq.Int4GroupedCache(nb, w.hkv, w.d, 64, 64, "cuda")
        app_fn, dec_fn, vec_bytes = kvq.kvq_append_paged_int4g, kvq.kvq_decode_attn_int4g, w.d // 2 + 4 * (w.d // 64)
    caches = [make(w.num_pages) for _ in range(2)]
    for c in caches:
        app_fn(c, w.k, w.v, w.slot_mapping)

    def dec(i):
        dec_fn(caches[i % 2], db.qs[i % RING], db.bt, db.sl, w.max_seq_len, w.sm_scale, out=db.out,
               workspace=db.ws)

    for i in range(10):
        dec(i)
    ms, _ = _time_events(torch, dec, iters)
    b2b_ms = _time_back_to_back(torch, dec, iters)   # the same calls with no event between them
    nbytes = decode_bytes(w.seq_lens, w.hkv, w.hq, w.d, vec_bytes)
    res = {"decode": {"us": round(ms * 1e3, 2), "bytes": nbytes,
                      "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                      "pct_of_peak": round(100.0 * nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                      "us_back_to_back": round(b2b_ms * 1e3, 2),
                      "pct_of_peak_back_to_back": round(100.0 * nbytes / (b2b_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
                      "time_over_int4": round(ms * 1e3 / (int4_bytes / (int4_gb_s * 1e9) * 1e6), 4)}}
    del caches
    torch.cuda.empty_cache()
    sets = []
    for r in range(PREFILL_RING):
        pw = workloads.prefill_append(PREFILL_SEEDS[r], device="cuda", block=64)
        sets.append((pw, make(pw.num_pages)))

    def app(i):
        pw, c = sets[i % PREFILL_RING]
        app_fn(c, pw.k, pw.v, pw.slot_mapping)

    for i in range(10):
        app(i)
    ms = _time_back_to_back(torch, app, iters)   # consecutive appends, as the headline prefill
    pw = sets[0][0]
    abytes = append_bytes(pw.num_tokens, pw.hkv, pw.d, vec_bytes)
    res["prefill_append"] = {"us": round(ms * 1e3, 2), "mtok_s": round(pw.num_tokens / (ms * 1e-3) / 1e6, 1),
                             "gb_s": round(abytes / (ms * 1e-3) / 1e9, 1), "bytes": abytes}
    del sets
    torch.cuda.empty_cache()
    return res


def variant_decode(torch, kvq, workloads, db, kind, iters, warm):
    """One decode variant alone on the headline workload (block 64), two
    cache copies alternating, timed per call (and back to back): the kernels for profiles."""
    w = db.w
    if kind == "windowed":
        res = windowed_rate(torch, kvq, workloads, db, iters, 1.0, 1)
        res.pop("time_over_int4_block64")
        return res
    if kind == "bf16":
        db.int4 = db.int4[:1]
        db.make_bf16()
        fn, caches = kvq.kvq_decode_attn_bf16, db.bf16
        vec = 2 * w.d
    else:
        make, app_fn, fn, vec = {
            "int8": (lambda: kvq.Int8Cache(w.num_pages, w.hkv, w.d, 64, "cuda"), kvq.kvq_append_paged_int8,
                     kvq.kvq_decode_attn_int8, w.d + 4),
            "int4g64": (lambda: kvq.Int4GroupedCache(w.num_pages, w.hkv, w.d, 64, 64, "cuda"),
                        kvq.kvq_append_paged_int4g, kvq.kvq_decode_attn_int4g, w.d // 2 + 4 * (w.d // 64)),
            "mxfp4": (lambda: kvq.MxFp4Cache(w.num_pages, w.hkv, w.d, 64, "cuda"), kvq.kvq_append_paged_mxfp4,
                      kvq.kvq_decode_attn_mxfp4, w.d // 2 + w.d // 32),
        }[kind]
        caches = [make() for _ in range(2)]
        for c in caches:
            app_fn(c, w.k, w.v, w.slot_mapping)

    def dec(i):
        fn(caches[i % 2], db.qs[i % RING], db.bt, db.sl, w.max_seq_len, w.sm_scale, out=db.out,
           workspace=db.ws)

    for i in range(warm):
        dec(i)
    ms, _ = _time_events(torch, dec, iters)
    b2b_ms = _time_back_to_back(torch, dec, iters)
    nbytes = decode_bytes(w.seq_lens, w.hkv, w.hq, w.d, vec)
    return {"us": round(ms * 1e3, 2), "bytes": nbytes, "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "us_back_to_back": round(b2b_ms * 1e3, 2)}


def long_context_rate(torch, kvq, workloads, iters=30):
    """Qwen3-4B-shaped long-context decode (8 x 131072 tokens, 65536 pages):
    split-K over pages plus the reduce, timed per call on two cache copies,
    Hadamard block 64 and plain INT4."""
    w = workloads.long_context_decode(4, device="cuda", batch=8, context=131072, block=64)
    bt = torch.from_numpy(w.block_table).to("cuda")
    sl = torch.from_numpy(w.seq_lens).to("cuda")
    nbytes = decode_bytes(w.seq_lens, w.hkv, w.hq, w.d, int4_bytes_per_vector(w.d))
    splits = kvq.kvq_decode_workspace_bytes(w.batch, w.hq, w.hkv, w.d, w.max_seq_len) // \
        (w.batch * w.hq * (w.d + 2) * 4)
    res = {"workload": "8 sequences x 131072 tokens, 32 q / 8 kv heads, head_dim 128, page 16, "
                       "per-channel scales in [0.1, 10]", "splits": int(splits), "bytes": nbytes}
    for blk in (64, 0):
        caches = [kvq.Int4Cache(w.num_pages, w.hkv, w.d, blk, "cuda") for _ in range(2)]
        for c in caches:
            kvq.kvq_append_paged(c, w.k, w.v, w.slot_mapping)
        out = torch.empty((w.batch, w.hq, w.d), dtype=torch.float32, device="cuda")
        ws = torch.empty(max(16, kvq.kvq_decode_workspace_bytes(w.batch, w.hq, w.hkv, w.d, w.max_seq_len)),
                         dtype=torch.uint8, device="cuda")

        def run(i):
            kvq.kvq_decode_attn(caches[i % 2], w.q, bt, sl, w.max_seq_len, w.sm_scale, out=out, workspace=ws)

        for i in range(5):
            run(i)
        ms, _ = _time_events(torch, run, iters)
        key = "int4_block64" if blk else "int4_plain"
        res[key] = {"us": round(ms * 1e3, 2), "gb_s": round(nbytes / (ms * 1e-3) / 1e9, 1)}
        del caches
        torch.cuda.empty_cache()
    res["rotated_over_plain"] = round(res["int4_plain"]["us"] / res["int4_block64"]["us"], 4)
    return res


RING_BYTES = 1 << 30   # each concurrency-sweep ring of layer caches holds at least 1 GiB


class ServingRing:
    """The 70B-shaped serving step at one batch size for one cache kind
    ("int4_block64", "int4_plain" or "bf16"): a ring of layer caches of at
    least RING_BYTES in all (successive layers of one decode step, so the
    256 MB Infinity Cache cannot hold what a step reads), each filled with the
    whole context and every step's token (a timed step rewrites its token's
    slot with the same bytes, so every layer holds valid data for every
    step).  Step i appends its token to layer i mod R and decodes it."""

    def __init__(self, torch, kvq, fill, steps, name, ws, out):
        self.kvq, self.st, self.ws, self.out = kvq, steps, ws, out
        self.bt = torch.from_numpy(steps[0].block_table).to("cuda")
        self.sls = [torch.from_numpy(x.seq_lens).to("cuda") for x in steps]
        self.maxlen = int(steps[-1].max_seq_len)
        if name == "bf16":
            make = lambda: kvq.Bf16Cache(fill.num_pages, fill.hkv, fill.d, "cuda")
            self.app, self.dec = kvq.kvq_append_paged_bf16, kvq.kvq_decode_attn_bf16
            vec = 2 * fill.d
        else:
            blk = 64 if name == "int4_block64" else 0
            make = lambda: kvq.Int4Cache(fill.num_pages, fill.hkv, fill.d, blk, "cuda")
            self.app, self.dec = kvq.kvq_append_paged, kvq.kvq_decode_attn
            vec = int4_bytes_per_vector(fill.d)
        layer = decode_bytes(steps[-1].seq_lens, fill.hkv, fill.hq, fill.d, vec)
        self.ring = max(2, -(-RING_BYTES // layer))
        self.caches = []
        for _ in range(self.ring):
            c = make()
            self.app(c, fill.k, fill.v, fill.slot_mapping)
            for x in steps:
                self.app(c, x.k, x.v, x.slot_mapping)
            self.caches.append(c)

    def run(self, i):
        c, x = self.caches[i % self.ring], self.st[i]
        self.app(c, x.k, x.v, x.slot_mapping)
        self.dec(c, x.q, self.bt, self.sls[i], self.maxlen, x.sm_scale, out=self.out, workspace=self.ws)


def concurrency_sweep(torch, kvq, workloads, steps=48, warm=8, block_steps=8,
                      batches=(1, 8, 32, 128, 256), eager_rounds=6):
    """70B-shaped layer (64 q / 8 kv heads): per batch size and cache kind
    (rotated INT4, plain INT4, bf16), a ServingRing of layer caches; ``warm``
    untimed steps on each, then ``steps`` more per kind.  Tokens/s = batch /
    time per step (one layer).  The steps are timed twice, the kinds
    alternating with the first of each round rotating so that all three see
    the same clocks: called one by one from Python (the host's per-call cost
    included; it bounds the small batches), all ``steps`` in one window per
    kind and round, ``eager_rounds`` rounds, the median window reported (a
    window starts from an idle GPU, so short windows would weigh that start
    on every few steps, and near the host's bound one round's jitter moves a
    mean); and captured in HIP graphs of ``block_steps`` steps and replayed,
    one graph per kind and round."""
    out = {"workload": "64 q / 8 kv heads, head_dim 128, lognormal contexts (median 2048, "
                       "sigma 1, cap 32768), page 16, one new token per sequence per step; "
                       "successive steps on successive layers of a ring of >= 1 GiB per cache kind",
           "steps": steps}
    names = ("int4_block64", "int4_plain", "bf16")
    for b in batches:
        fill, st = workloads.concurrency_step(5, device="cuda", batch=b, block=64, steps=warm + steps)
        maxlen = int(st[-1].max_seq_len)
        ws = torch.empty(max(16, kvq.kvq_decode_workspace_bytes(b, fill.hq, fill.hkv, fill.d, maxlen)),
                         dtype=torch.uint8, device="cuda")
        o = torch.empty((b, fill.hq, fill.d), dtype=torch.float32, device="cuda")
        rings = {name: ServingRing(torch, kvq, fill, st, name, ws, o) for name in names}
        torch.cuda.synchronize()

        def run(name, i):
            rings[name].run(i)

        for name in names:
            for i in range(warm):
                run(name, i)
        wins = {name: [] for name in names}
        for rnd in range(eager_rounds):
            # the variant that runs first after the synchronisation changes
            # from round to round, so none is always first
            order = names[rnd % len(names):] + names[:rnd % len(names)]
            for name in order:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                for i in range(warm, warm + steps):
                    run(name, i)
                e1.record()
                torch.cuda.synchronize()
                wins[name].append(e0.elapsed_time(e1))
        ms = {name: sorted(w)[len(w) // 2] for name, w in wins.items()}
        # The same steps captured in HIP graphs (one per run of block_steps)
        # and replayed in the same rotating order: the GPU time of a step
        # without the host's per-call cost, as a serving loop that replays
        # captured decode steps sees it.  Replays write the same tokens into
        # the same slots, so the caches stay as the eager steps left them.
        graphs = {name: [] for name in names}
        for name in names:
            for i0 in range(warm, warm + steps, block_steps):
                g = torch.cuda.CUDAGraph()
                torch.cuda.synchronize()
                with torch.cuda.graph(g):
                    for i in range(i0, min(i0 + block_steps, warm + steps)):
                        run(name, i)
                graphs[name].append(g)
        for name in names:
            graphs[name][0].replay()
        gms = {name: 0.0 for name in names}
        for rnd in range(len(graphs[names[0]])):
            order = names[rnd % len(names):] + names[:rnd % len(names)]
            for name in order:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                graphs[name][rnd].replay()
                e1.record()
                torch.cuda.synchronize()
                gms[name] += e0.elapsed_time(e1)
        row = {"context_tokens": int(fill.seq_lens.sum()),
               "ring_layers": {name: rings[name].ring for name in names}}
        for name in names:
            row[name] = {"us_per_step": round(ms[name] * 1e3 / steps, 2),
                         "tokens_s": round(b * steps / (ms[name] * 1e-3), 1),
                         "graph_us_per_step": round(gms[name] * 1e3 / steps, 2),
                         "graph_tokens_s": round(b * steps / (gms[name] * 1e-3), 1)}
        row["rotated_over_plain"] = round(row["int4_block64"]["tokens_s"] / row["int4_plain"]["tokens_s"], 4)
        row["int4_over_bf16"] = round(row["int4_block64"]["tokens_s"] / row["bf16"]["tokens_s"], 3)
        row["graph_rotated_over_plain"] = round(row["int4_block64"]["graph_tokens_s"]
                                                / row["int4_plain"]["graph_tokens_s"], 4)
        row["graph_int4_over_bf16"] = round(row["int4_block64"]["graph_tokens_s"]
                                            / row["bf16"]["graph_tokens_s"], 3)
        del graphs, rings
        out[f"batch{b}"] = row
        del fill, st
        torch.cuda.empty_cache()
    return out


def serving_mode(torch, kvq, workloads, batch, name, steps, warm):
    """One cache kind's serving steps at one batch size (ServingRing), timed
    back to back: the kernels of the 70B-shaped step alone, for profiles."""
    fill, st = workloads.concurrency_step(5, device="cuda", batch=batch, block=64, steps=warm + steps)
    maxlen = int(st[-1].max_seq_len)
    ws = torch.empty(max(16, kvq.kvq_decode_workspace_bytes(batch, fill.hq, fill.hkv, fill.d, maxlen)),
                     dtype=torch.uint8, device="cuda")
    o = torch.empty((batch, fill.hq, fill.d), dtype=torch.float32, device="cuda")
    ring = ServingRing(torch, kvq, fill, st, name, ws, o)
    for i in range(warm):
        ring.run(i)
    ms, _ = _time_events(torch, lambda i: ring.run(warm + i), steps)
    return {"batch": batch, "cache": name, "ring_layers": ring.ring, "us_per_step": round(ms * 1e3, 2),
            "tokens_s": round(batch / (ms * 1e-3), 1)}


def ceiling_mode(torch, iters=20):
    """What the memory system gives the hot path's access patterns on this
    GPU, from the probe kernels of libkvq_probe.so: the decode's gather of
    2176-byte page slabs in a seeded random order (1.14 GB, four layers'
    worth of the headline cache), a streaming read of 4 GiB, and streaming
    reads with a 4:1 and a 1:1 read:write mix (the append moves about 4 bytes
    in per byte out), the pieces in flight spread over the grid; then the
    4:1 mix with each workgroup on a contiguous stretch, its output
    contiguous or in 1 KiB pieces at seeded permuted places (as page slabs of
    a permuted page table), with plain and non-temporal stores.  TB/s of the
    bytes each probe moves."""
    import ctypes as C
    import numpy as np
    import bit_kv_cache_block_amd as kvq_pkg

    L = C.CDLL(os.path.join(os.path.dirname(kvq_pkg.__file__), "libkvq_probe.so"))
    p, i32, i64 = C.c_void_p, C.c_int32, C.c_int64
    L.kvq_probe_gather.argtypes = [p, i32, p, i32, i32, p, p]
    L.kvq_probe_stream.argtypes = [p, i64, i32, p, i32, p, p]
    L.kvq_probe_stream_block.argtypes = [p, i64, p, i32, i32, p, p]
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    grid = 2048
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    res = {}

    def timed(fn, nbytes):
        for _ in range(3):
            fn()
        ms, _ = _time_events(torch, lambda i: fn(), iters)
        return round(nbytes / (ms * 1e-3) / 1e12, 3)

    slab, nslab = 2176, 4 * 16384 * 8
    pool = torch.empty(nslab * slab, dtype=torch.uint8, device="cuda").fill_(3)
    rng = np.random.default_rng(7)
    ids = torch.from_numpy(rng.permutation(nslab).astype(np.int32)).to("cuda")

    def gather():
        assert L.kvq_probe_gather(p(pool.data_ptr()), slab, p(ids.data_ptr()), nslab, grid,
                                  p(sink.data_ptr()), stream) == 0

    res["gather_2176B_slabs_tb_s"] = timed(gather, nslab * slab)
    del pool, ids
    src = torch.empty(1 << 32, dtype=torch.uint8, device="cuda").fill_(5)

    def read():
        assert L.kvq_probe_stream(p(src.data_ptr()), (1 << 32) // 16, 1, None, grid,
                                  p(sink.data_ptr()), stream) == 0

    res["stream_read_tb_s"] = timed(read, 1 << 32)
    for ratio in (4, 1):
        items = (1 << 32) // 16 // ratio
        dst = torch.empty(items * 16, dtype=torch.uint8, device="cuda")

        def mix():
            assert L.kvq_probe_stream(p(src.data_ptr()), items, ratio, p(dst.data_ptr()), grid,
                                      None, stream) == 0

        res[f"stream_{ratio}to1_read_write_tb_s"] = timed(mix, items * 16 * (ratio + 1))
        del dst
    items = (1 << 32) // 16 // 4
    dst = torch.empty(items * 16, dtype=torch.uint8, device="cuda")
    perm = torch.from_numpy(rng.permutation(items // 64).astype(np.int32)).to("cuda")
    for scatter in (False, True):
        for nt in (0, 1):
            def blk():
                assert L.kvq_probe_stream_block(p(src.data_ptr()), items, p(dst.data_ptr()), 1024, nt,
                                                p(perm.data_ptr()) if scatter else None, stream) == 0

            key = "stream_4to1_block_" + ("scatter1k" if scatter else "contiguous") + ("_nt" if nt else "")
            res[key + "_tb_s"] = timed(blk, items * 16 * 5)
    del dst, perm
    return res


def cpu_baseline(w, budget_s=15.0):
    """The oracle (as it stands) on the host cores over a bounded sample of the
    same workload: host copies of whole sequences are appended (rotate +
    quantize) and attended in fp64 for all 32 query heads, one sequence at a
    time until the time budget is spent."""
    import numpy as np
    import torch

    import oracle
    from workloads import bits

    pool = oracle.new_int4_pool(w.num_pages, w.hkv, w.d)
    qh = bits(w.q)
    t_app = t_dec = 0.0
    done = []
    for b in range(w.batch):
        sel = torch.from_numpy(w.token_seq == b).to(w.k.device)
        kh, vh = bits(w.k[sel]), bits(w.v[sel])
        sm = w.slot_mapping[sel].cpu().numpy()
        t0 = time.perf_counter()
        oracle.append_int4(pool, w.num_pages, w.hkv, w.d, w.block, kh, vh, oracle.BF16, sm)
        t1 = time.perf_counter()
        mask = np.zeros((w.batch, w.hq), np.uint8)
        mask[b] = 1
        oracle.decode_int4(pool, w.hkv, w.d, w.block, qh, oracle.BF16, w.block_table, w.seq_lens,
                           w.sm_scale, mask=mask)
        t2 = time.perf_counter()
        t_app += t1 - t0
        t_dec += t2 - t1
        done.append(b)
        if t_app + t_dec > budget_s:
            break
    lens = [int(w.seq_lens[b]) for b in done]
    dbytes = decode_bytes(lens, w.hkv, w.hq, w.d, int4_bytes_per_vector(w.d))
    tokens = sum(lens)
    cores = oracle.num_threads()
    # the first sampled sequence again on one thread (same codes, same output)
    b = done[0]
    sel = torch.from_numpy(w.token_seq == b).to(w.k.device)
    kh, vh = bits(w.k[sel]), bits(w.v[sel])
    sm = w.slot_mapping[sel].cpu().numpy()
    mask = np.zeros((w.batch, w.hq), np.uint8)
    mask[b] = 1
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.append_int4(pool, w.num_pages, w.hkv, w.d, w.block, kh, vh, oracle.BF16, sm)
        t1 = time.perf_counter()
        oracle.decode_int4(pool, w.hkv, w.d, w.block, qh, oracle.BF16, w.block_table, w.seq_lens,
                           w.sm_scale, mask=mask)
        t2 = time.perf_counter()
    finally:
        oracle.set_num_threads(cores)
    one_bytes = decode_bytes([lens[0]], w.hkv, w.hq, w.d, int4_bytes_per_vector(w.d))
    return {
        "value": dbytes / t_dec / 1e9, "unit": "GB/s", "cores": cores,
        "kind": "oracle",
        "sample": f"{len(done)} of {w.batch} sequences x {lens[0]} tokens, all {w.hq} q heads, "
                  f"block {w.block}: oracle append then fp64 decode; decode {t_dec:.2f} s, "
                  f"append {t_app:.2f} s",
        "append_mtok_s": tokens / t_app / 1e6,
        "one_thread": {"value": round(one_bytes / (t2 - t1) / 1e9, 5),
                       "append_mtok_s": round(lens[0] / (t1 - t0) / 1e6, 5),
                       "sample": f"sequence {b} ({lens[0]} tokens) on one thread"},
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


# ---------------------------------------------------------------- accuracy
# What each cache does to the numbers, measured from the library's own pools:
# the stored codes and sidecars of a sample of tokens decoded here in torch
# from the page layouts the header documents (not through the test oracle),
# and each cache's decode attention against the bf16-KV decode of the same
# tokens.

def hadamard_rotate(torch, x, block):
    """x [..., D] in the basis a pool of Hadamard block b stores:
    blockdiag(H_b) / sqrt(b) x with H_b in Sylvester order (H_1 = [1],
    H_2n = [[H, H], [H, -H]]); b = 0 leaves x as it is."""
    if block == 0:
        return x
    h = torch.ones((1, 1), dtype=torch.float64, device=x.device)
    while h.shape[0] < block:
        h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
    h = (h / math.sqrt(block)).to(torch.float32)
    shp = x.shape
    return (x.reshape(*shp[:-1], shp[-1] // block, block) @ h).reshape(shp)


_E2M1 = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def dequant_pool(torch, kind, cache, slots, group=64):
    """K and V [n][Hkv][D] (fp32, the pool's basis) of the tokens in `slots`
    (int64 tensor on the pool's device), read from the pool bytes: kind
    int4 (token-wise INT4, also the scale-search pool), int8, int4g (grouped,
    |scale| as the decode takes it) or mxfp4."""
    P, D, hkv = 16, cache.head_dim, cache.num_kv_heads
    pool = cache.pool.view(cache.num_pages, hkv, -1)
    dev = pool.device
    page, off = slots // P, slots % P
    S = pool[page]                                    # [n][Hkv][slab]
    n = S.shape[0]
    ar = lambda m: torch.arange(m, device=dev)

    def take(idx):                                    # byte offsets [n][m] -> [n][Hkv][m]
        return torch.gather(S, 2, idx[:, None, :].expand(-1, hkv, -1)).long()

    def nibbles(b):                                   # [..., m] bytes -> [..., 2m], low nibble first
        return torch.stack([b & 15, b >> 4], -1).reshape(*b.shape[:-1], -1)

    def halves(base):                                 # fp16 (scale, zero) at byte base + [0, 4)
        b = take(base[:, None] + ar(4)[None, :]).to(torch.uint8)
        return b.contiguous().view(torch.float16).float()   # [n][Hkv][2]

    def grouped_v(codes_at):                          # word w*P + t: channels w + (D/8) j
        w = ar(D // 8)
        idx = codes_at + 4 * (w[None, :, None] * P + off[:, None, None]) + ar(4)[None, None, :]
        nib = nibbles(take(idx.reshape(n, -1)).reshape(n, hkv, D // 8, 4))   # [n][Hkv][D/8][8]
        return nib.transpose(2, 3).reshape(n, hkv, D)

    if kind in ("int4", "int4g", "mxfp4"):
        kc = nibbles(take(off[:, None] * (D // 2) + ar(D // 2)[None, :]))
    if kind == "int4":
        w = ar(D // 8)
        idx = P * D // 2 + 4 * (w[None, :, None] * P + off[:, None, None]) + ar(4)[None, None, :]
        vc = nibbles(take(idx.reshape(n, -1)))
        ks, vs = halves(P * D + 4 * off), halves(P * D + 4 * P + 4 * off)
        return (kc * ks[..., :1] + ks[..., 1:], vc * vs[..., :1] + vs[..., 1:])
    if kind == "int8":
        kc = take(off[:, None] * D + ar(D)[None, :])
        w, h = ar(D // 8), ar(2)
        word = (w[:, None] * P + off[:, None, None]) * 2 + h[None, :]     # [n][D/8][2]
        vc = take((P * D + 4 * word[..., None] + ar(4)).reshape(n, -1))
        ks, vs = halves(2 * P * D + 4 * off), halves(2 * P * D + 4 * P + 4 * off)
        return (kc * ks[..., :1] + ks[..., 1:], vc * vs[..., :1] + vs[..., 1:])
    vc = grouped_v(P * D // 2)
    if kind == "int4g":
        ng = D // group

        def side(base):   # (scale, zero) of token t, group i at base + 4 (t * ng + i)
            start = base + 4 * (off[:, None] * ng + ar(ng)[None, :])          # [n][ng]
            b = take((start[..., None] + ar(4)).reshape(n, -1)).to(torch.uint8).reshape(n, hkv, ng, 4)
            return b.contiguous().view(torch.float16).float()                 # [n][Hkv][ng][2]

        ks, vs = side(P * D), side(P * D + 4 * P * ng)

        def apply(c, sz):
            c = c.float().reshape(n, hkv, ng, group)
            return (c * sz[..., :1].abs() + sz[..., 1:]).reshape(n, hkv, D)

        return apply(kc, ks), apply(vc, vs)
    # mxfp4: E2M1 codes, one E8M0 exponent per 32 channels
    lut = torch.tensor(_E2M1, device=dev)

    def e2m1(c):
        return lut[c & 7] * torch.where((c & 8) != 0, -1.0, 1.0)

    nb = D // 32

    def scales(base):
        e = take(base + off[:, None] * nb + ar(nb)[None, :]).float()
        return torch.exp2(e - 127.0).repeat_interleave(32, dim=2)

    return e2m1(kc) * scales(P * D), e2m1(vc) * scales(P * D + P * D // 32)


QUALITY_CACHES = (
    # name, pool kind, Hadamard block, append entry, decode entry
    ("int4_plain", "int4", 0, "kvq_append_paged", "kvq_decode_attn"),
    ("int4_block64", "int4", 64, "kvq_append_paged", "kvq_decode_attn"),
    ("int4_block64_key_search", "int4", 64, "kvq_append_paged_int4_search", "kvq_decode_attn"),
    ("int4_groups64_block64", "int4g", 64, "kvq_append_paged_int4g", "kvq_decode_attn_int4g"),
    ("int4_groups64_block64_hybrid", "int4g", 64, "kvq_append_paged_int4g_hybrid", "kvq_decode_attn_int4g"),
    ("int8_block64", "int8", 64, "kvq_append_paged_int8", "kvq_decode_attn_int8"),
    ("mxfp4_block64", "mxfp4", 64, "kvq_append_paged_mxfp4", "kvq_decode_attn_mxfp4"),
)


def quality_of(torch, kvq, name, k, v, slot_mapping, num_pages, hq, q, block_table, seq_lens,
               max_seq_len, sample=8192, seed=11):
    """Reconstruction and attention error of every cache kind on one set of
    tokens: relative MSE of K and V (sum of squared errors over the sample /
    sum of squares of the input; the rotation is orthonormal, so this equals
    the error in the original basis) and the decode output's relative L2 and
    largest absolute difference from the bf16-KV decode."""
    hkv, d = k.shape[1], k.shape[2]
    g = torch.Generator(device="cpu").manual_seed(seed)
    pick = torch.randperm(k.shape[0], generator=g)[:sample].to(k.device)
    keep = slot_mapping[pick] >= 0
    pick = pick[keep]
    slots = slot_mapping[pick].long()
    bt = block_table
    ref_cache = kvq.Bf16Cache(num_pages, hkv, d, "cuda")
    kvq.kvq_append_paged_bf16(ref_cache, k, v, slot_mapping)
    ref = kvq.kvq_decode_attn_bf16(ref_cache, q, bt, seq_lens, max_seq_len)
    del ref_cache
    xk, xv = k[pick].float(), v[pick].float()
    res = {"workload": name, "tokens_sampled": int(pick.numel())}
    for cname, kind, blk, app, dec in QUALITY_CACHES:
        if kind == "int4":
            cache = kvq.Int4Cache(num_pages, hkv, d, blk, "cuda")
        elif kind == "int8":
            cache = kvq.Int8Cache(num_pages, hkv, d, blk, "cuda")
        elif kind == "int4g":
            cache = kvq.Int4GroupedCache(num_pages, hkv, d, blk, 64, "cuda")
        else:
            cache = kvq.MxFp4Cache(num_pages, hkv, d, blk, "cuda")
        getattr(kvq, app)(cache, k, v, slot_mapping)
        dk, dv = dequant_pool(torch, kind, cache, slots)
        rk, rv = hadamard_rotate(torch, xk, blk), hadamard_rotate(torch, xv, blk)
        out = getattr(kvq, dec)(cache, q, bt, seq_lens, max_seq_len)
        torch.cuda.synchronize()
        res[cname] = {
            "k_rel_mse": float(((dk - rk) ** 2).sum() / (xk ** 2).sum()),
            "v_rel_mse": float(((dv - rv) ** 2).sum() / (xv ** 2).sum()),
            "attn_rel_l2": float((out - ref).norm() / ref.norm()),
            "attn_max_abs": float((out - ref).abs().max()),
        }
        del cache
    torch.cuda.empty_cache()
    return res


def quality_report(torch, kvq, workloads):
    """The accuracy of every cache kind on the prefill (Student-t), the
    long-context (per-channel scales) and the 70B-shaped serving (lognormal
    lengths) data; the prefill has no queries, so its attention uses 32
    query heads (GQA 4) drawn N(0, 1) from a fixed seed."""
    rep = {}
    pw = workloads.prefill_append(PREFILL_SEEDS[0], device="cuda", block=64)
    g = torch.Generator(device="cuda").manual_seed(5)
    q = torch.randn((pw.batch, 32, pw.d), generator=g, device="cuda").to(torch.bfloat16)
    rep["prefill_student_t"] = quality_of(
        torch, kvq, "32768 tokens over 16 sequences, 8 kv heads, head_dim 128, bf16 Student-t(3); "
        "32 query heads N(0,1)", pw.k, pw.v, pw.slot_mapping, pw.num_pages, 32, q,
        torch.from_numpy(pw.block_table).cuda(), torch.from_numpy(pw.seq_lens).cuda(), pw.max_seq_len)
    del pw
    lw = workloads.long_context_decode(4, device="cuda", batch=8, context=131072, block=64)
    rep["long_context_channel_scales"] = quality_of(
        torch, kvq, "8 x 131072 tokens, 32 q / 8 kv heads, head_dim 128, per-channel scales in [0.1, 10]",
        lw.k, lw.v, lw.slot_mapping, lw.num_pages, lw.hq, lw.q, torch.from_numpy(lw.block_table).cuda(),
        torch.from_numpy(lw.seq_lens).cuda(), lw.max_seq_len)
    del lw
    torch.cuda.empty_cache()
    fill, st = workloads.concurrency_step(5, device="cuda", batch=32, block=64, steps=1)
    s0 = st[0]
    k = torch.cat([fill.k, s0.k]).contiguous()
    v = torch.cat([fill.v, s0.v]).contiguous()
    sm = torch.cat([fill.slot_mapping, s0.slot_mapping]).contiguous()
    rep["serving_70b_lognormal"] = quality_of(
        torch, kvq, "batch 32, lognormal contexts (median 2048, cap 32768) + 1 step, 64 q / 8 kv heads, "
        "head_dim 128", k, v, sm, s0.num_pages, s0.hq, s0.q, torch.from_numpy(s0.block_table).cuda(),
        torch.from_numpy(s0.seq_lens).cuda(), s0.max_seq_len)
    return rep


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["full", "decode", "prefill", "copy", "concurrency", "serving",
                                       "variant", "ceiling", "quality"], default="full")
    ap.add_argument("--batch", type=int, default=256, help="serving mode: batch size")
    ap.add_argument("--cache", default="int4_block64",
                    help="serving mode: int4_block64, int4_plain or bf16; variant mode: int8, "
                         "int4g64, mxfp4, windowed or bf16")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the path shards by "
                                   "KV head or sequence with no exchange, see the design notes",
                          "n_gpus": args.gpus}))
        return 2

    import torch
    import bit_kv_cache_block_amd as kvq
    import workloads

    if args.mode == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read": n, "bytes_written": n, "launches": 5}))
        return 0

    if args.mode == "ceiling":
        print(json.dumps({"mode": "ceiling", **ceiling_mode(torch)}))
        return 0

    if args.mode == "quality":
        print(json.dumps({"mode": "quality", **quality_report(torch, kvq, workloads)}))
        return 0

    if args.mode == "serving":
        print(json.dumps({"mode": "serving", **serving_mode(torch, kvq, workloads, args.batch, args.cache,
                                                            args.steps, args.warmup)}))
        return 0

    if args.mode == "concurrency":
        print(json.dumps({"mode": "concurrency", **concurrency_sweep(torch, kvq, workloads)}))
        return 0

    if args.mode == "prefill":
        r = prefill_rates(torch, kvq, workloads, blocks=(64,), iters=args.steps)[64]
        print(json.dumps({"mode": "prefill", **r}))
        return 0

    db = DecodeBench(torch, kvq, workloads, block=64)
    w = db.w
    kvb = int4_bytes_per_vector(w.d)
    dec_bytes = decode_bytes(w.seq_lens, w.hkv, w.hq, w.d, kvb)
    app_bytes = append_bytes(w.batch, w.hkv, w.d, kvb)

    if args.mode == "decode":
        for i in range(args.warmup):
            db.decode(i)
        ms, _ = _time_events(torch, db.decode, args.steps)
        print(json.dumps({"mode": "decode", "us": ms * 1e3, "gb_s": dec_bytes / (ms * 1e-3) / 1e9}))
        return 0

    if args.mode == "variant":
        print(json.dumps({"mode": "variant", "cache": args.cache,
                          **variant_decode(torch, kvq, workloads, db, args.cache, args.steps, args.warmup)}))
        return 0

    # ---- headline: K steps of append + decode ------------------------------
    # untimed steps for about 0.25 s first: the GPU reaches its steady clocks
    # only under sustained load, and a short warm-up right after the set-up
    # measured up to 4% slow; then the W warm-up steps
    t_ramp = time.perf_counter()
    i = 0
    while time.perf_counter() - t_ramp < 0.25:
        for _ in range(20):
            db.append(i)
            db.decode(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        db.append(i)
        db.decode(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record()
        db.append(i)
        ev[i][1].record()
        db.decode(i)
        ev[i][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    app_ms = [e[0].elapsed_time(e[1]) for e in ev]
    dec_ms = [e[1].elapsed_time(e[2]) for e in ev]
    dec_mean = sum(dec_ms) / len(dec_ms)
    app_mean = sum(app_ms) / len(app_ms)

    def pct(xs):
        s = sorted(xs)
        at = lambda f: s[min(len(s) - 1, int(f * (len(s) - 1) + 0.5))]
        return {"p10": round(at(0.1) * 1e3, 2), "p50": round(at(0.5) * 1e3, 2), "p90": round(at(0.9) * 1e3, 2)}
    value = dec_bytes / (dec_mean * 1e-3) / 1e9
    # the same decode launched back to back (one event pair around the whole
    # run): the kernel's own duration without the per-call event gap
    for i in range(10):
        db.decode(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(args.steps):
        db.decode(i)
    e1.record()
    torch.cuda.synchronize()
    dec_b2b_ms = e0.elapsed_time(e1) / args.steps

    # ---- variants on the same workload, all timed alone (decode only) ---------
    variants = {}
    for blk in (64, 0, 16, 32, 128):
        if blk != 64:
            db.refill(blk)
        for i in range(10):
            db.decode(i)
        ms, _ = _time_events(torch, db.decode, args.steps)
        variants[f"int4_block{blk}" if blk else "int4_plain"] = dec_bytes / (ms * 1e-3) / 1e9
    db.refill(64)
    windowed = windowed_rate(torch, kvq, workloads, db, args.steps, variants["int4_block64"], dec_bytes)
    int8 = variant_rates(torch, kvq, workloads, db, args.steps, variants["int4_block64"], dec_bytes, "int8")
    int4g = variant_rates(torch, kvq, workloads, db, args.steps, variants["int4_block64"], dec_bytes, "int4g64")
    mxfp4 = variant_rates(torch, kvq, workloads, db, args.steps, variants["int4_block64"], dec_bytes, "mxfp4")
    db.int4 = db.int4[:1]
    torch.cuda.empty_cache()
    db.make_bf16()
    for i in range(10):
        db.decode_bf16(i)
    ms_bf16, _ = _time_events(torch, db.decode_bf16, args.steps)
    bf16_bytes = decode_bytes(w.seq_lens, w.hkv, w.hq, w.d, 2 * w.d)
    cb = None
    if not args.no_cpu:
        cb = cpu_baseline(w)
        cb["cpu_model"] = _cpu_model()
    db.free()
    del db

    pre = prefill_rates(torch, kvq, workloads)
    prefill_rot, prefill_plain = pre[64], pre[0]
    del pre
    torch.cuda.empty_cache()
    long_ctx = long_context_rate(torch, kvq, workloads)
    conc = concurrency_sweep(torch, kvq, workloads)
    torch.cuda.empty_cache()
    quality = quality_report(torch, kvq, workloads)

    traffic = _traffic(dec_bytes)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-mfma/fp32",
        "data": "synthetic",
        "config": {
            "workload": "llama3-8b-shaped layer decode: 32 q / 8 kv heads, head_dim 128, "
                        "batch 64 x 4096 context, page 16, hadamard block 64, bf16 K/V with "
                        "4 key outlier channels x15; step = append 1 token/seq + decode",
            "global_batch": w.batch, "seq_len": int(w.max_seq_len), "parallelism": "none",
        },
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "decode_us": round(dec_mean * 1e3, 2),
        "decode_us_per_step": pct(dec_ms),
        "append_us": round(app_mean * 1e3, 2),
        "append_us_per_step": pct(app_ms),
        "decode_bytes": dec_bytes,
        "rotate_quant_mtok_s": round(prefill_rot["mtok_s"], 1),
        "prefill_append": {
            "workload": "32768 new tokens over 16 ragged sequences (512-4096), 8 kv heads, "
                          "head_dim 128, bf16 Student-t(3), page-16 pool, block 64",
            "rotated": {k: round(v, 2) for k, v in prefill_rot.items()},
            "plain": {k: round(v, 2) for k, v in prefill_plain.items()},
            "rotated_over_plain": round(prefill_rot["mtok_s"] / prefill_plain["mtok_s"], 4),
        },
        "decode_variants_gb_s": {k: round(v, 1) for k, v in sorted(variants.items())},
        "rotated_over_plain_decode": round(variants["int4_block64"] / variants["int4_plain"], 4),
        "windowed_decode": windowed,
        "int8_kv": int8,
        "int4_groups64": int4g,
        "mxfp4": mxfp4,
        "long_context_decode": long_ctx,
        "concurrency_sweep": conc,
        "quality": quality,
        "bf16_kv": {"gb_s": round(bf16_bytes / (ms_bf16 * 1e-3) / 1e9, 1),
                    "us": round(ms_bf16 * 1e3, 2), "bytes": bf16_bytes,
                    "int4_speedup": round(ms_bf16 / dec_mean, 3)},
        "roofline": {
            "bound": "hbm", "achieved": round(value, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(value / PEAK_HBM_GBS, 4),
            "kernel_us_back_to_back": round(dec_b2b_ms * 1e3, 2),
            "frac_kernel": round(dec_bytes / (dec_b2b_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "kernel": "decode_quant_kernel<128, 1, true, 4, 0, 1, 0> (one kvq_decode_attn call; at this shape the split "
                      "plan is one split per (sequence, KV head), so no reduce kernel runs)",
        },
    }
    line["cpu_baseline"] = None if cb is None else \
        {k: (round(v, 5) if isinstance(v, float) else v) for k, v in cb.items()}
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
