"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and lays out page tables; it holds none
of the method's arithmetic (no rotation, no quantization, no attention), so
both the GPU path and the CPU oracle can be fed from it.

Shapes follow the decode/prefill workloads the pages measure on (Llama-,
Qwen3- and 70B-shaped attention layers, page size 16, grouped-query heads);
no dataset, prompt or model weight is involved.  Values are drawn in fp32 and
rounded to the input dtype with torch's round-to-nearest-even cast.

Conventions:
  * ``k``, ``v``: [T][Hkv][D] new tokens in arrival order, ``slot_mapping[t]``
    = physical slot (page * 16 + offset); ``q``: [B][Hq][D].
  * ``block_table``: [B][max_pages] int32, unused entries -1; pages of the pool
    are a seeded permutation, each sequence takes a contiguous slice of it.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

PAGE = 16


@dataclasses.dataclass
class Workload:
    name: str
    hq: int
    hkv: int
    d: int
    block: int
    dtype: torch.dtype            # torch.float16 or torch.bfloat16
    seq_lens: np.ndarray          # [B] int32, context after the append
    block_table: np.ndarray       # [B][max_pages] int32
    num_pages: int
    k: torch.Tensor               # [T][Hkv][D]
    v: torch.Tensor
    slot_mapping: torch.Tensor    # [T] int32
    q: torch.Tensor | None        # [B][Hq][D] or None for append-only work
    token_seq: np.ndarray         # [T] sequence index of each new token
    token_pos: np.ndarray         # [T] position of each new token

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.k.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def paged_layout(seq_lens, capacity_lens, rng: np.random.Generator, extra_pages: int = 0):
    """Page table over a seeded permutation of the pool.  ``capacity_lens[b]``
    tokens of room are reserved for sequence b."""
    npages = [(int(c) + PAGE - 1) // PAGE for c in capacity_lens]
    total = sum(npages) + extra_pages
    perm = rng.permutation(total).astype(np.int32)
    maxp = max(1, max(npages) if npages else 1)
    bt = np.full((len(npages), maxp), -1, np.int32)
    off = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, total


def slots_for(block_table: np.ndarray, seq: np.ndarray, pos: np.ndarray) -> np.ndarray:
    pages = block_table[seq, pos // PAGE]
    return (pages.astype(np.int64) * PAGE + pos % PAGE).astype(np.int32)


def _normal(shape, g, device):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def _outliers(x: torch.Tensor, n_channels: int, factor: float, g, device):
    """Scale n_channels seeded channels of each KV head by ``factor`` (x: [T][Hkv][D])."""
    hkv, d = x.shape[1], x.shape[2]
    for h in range(hkv):
        ch = torch.randperm(d, generator=g, device=device)[:n_channels]
        x[:, h, ch] *= factor
    return x


def _student_t3(shape, g, device):
    z = _normal(shape, g, device)
    chi = sum(_normal(shape, g, device) ** 2 for _ in range(3))
    return z / torch.sqrt(chi / 3.0)


def _fill_tokens(seq_lens):
    seq = np.concatenate([np.full(int(n), b, np.int64) for b, n in enumerate(seq_lens)]) \
        if len(seq_lens) else np.zeros(0, np.int64)
    pos = np.concatenate([np.arange(int(n), dtype=np.int64) for n in seq_lens]) \
        if len(seq_lens) else np.zeros(0, np.int64)
    return seq, pos


def _make(name, hq, hkv, d, block, dtype, seq_lens, k32, v32, q32, rng, device,
          capacity_lens=None, token_seq=None, token_pos=None):
    seq_lens = np.asarray(seq_lens, np.int32)
    cap = seq_lens if capacity_lens is None else np.asarray(capacity_lens)
    bt, total = paged_layout(seq_lens, cap, rng)
    if token_seq is None:
        token_seq, token_pos = _fill_tokens(seq_lens)
    slots = slots_for(bt, token_seq, token_pos)
    return Workload(
        name=name, hq=hq, hkv=hkv, d=d, block=block, dtype=dtype, seq_lens=seq_lens,
        block_table=bt, num_pages=total, k=k32.to(dtype), v=v32.to(dtype),
        slot_mapping=torch.from_numpy(slots).to(device),
        q=None if q32 is None else q32.to(dtype), token_seq=token_seq, token_pos=token_pos)


# ---------------------------------------------------------------------------
# The five workloads.  Every size can be shrunk for parity tests; the defaults
# are the full shapes.


def tiny_decode(seed: int = 1, device="cpu", block: int = 64) -> Workload:
    """1 layer, 8 q heads / 2 KV heads, head_dim 64, 4 sequences x 256 tokens,
    page 16 with a shuffled page table; K, V fp16 N(0,1) with 2 outlier
    channels per KV head (drawn separately for K and V) scaled x20; one query
    per sequence.  The whole cache is appended, then attended."""
    g = _gen(1000 + seed, device)
    rng = np.random.default_rng(np.random.SeedSequence(1000 + seed))
    b, length, hq, hkv, d = 4, 256, 8, 2, 64
    t = b * length
    k = _outliers(_normal((t, hkv, d), g, device), 2, 20.0, g, device)
    v = _outliers(_normal((t, hkv, d), g, device), 2, 20.0, g, device)
    q = _normal((b, hq, d), g, device)
    return _make("tiny_decode", hq, hkv, d, block, torch.float16, [length] * b, k, v, q, rng, device)


def llama8b_decode(seed: int = 2, device="cpu", batch: int = 64, context: int = 4096,
                   block: int = 64) -> Workload:
    """Llama-3-8B-shaped layer: 32 q heads / 8 KV heads, head_dim 128, bf16;
    K ~ N(0,1) with 4 key outlier channels per KV head x15; V, q ~ N(0,1)."""
    g = _gen(2000 + seed, device)
    rng = np.random.default_rng(np.random.SeedSequence(2000 + seed))
    hq, hkv, d = 32, 8, 128
    t = batch * context
    k = _outliers(_normal((t, hkv, d), g, device), 4, 15.0, g, device)
    v = _normal((t, hkv, d), g, device)
    q = _normal((batch, hq, d), g, device)
    return _make("llama8b_decode", hq, hkv, d, block, torch.bfloat16, [context] * batch, k, v, q,
                 rng, device)


def prefill_lengths(total: int, nseq: int, lo: int, hi: int, rng: np.random.Generator) -> np.ndarray:
    """``nseq`` ragged lengths in [lo, hi] summing exactly to ``total``: a
    uniform draw shares out the tokens above ``lo``, the last length takes the
    rounding remainder."""
    u = rng.uniform(0.0, 1.0, nseq)
    extra = total - lo * nseq
    lens = lo + np.round(extra * u / u.sum()).astype(np.int64)
    lens[-1] = total - lens[:-1].sum()
    if lens.min() < lo or lens.max() > hi:
        raise ValueError("draw outside [lo, hi]; pick another seed")
    return lens.astype(np.int32)


def prefill_append(seed: int = 3, device="cpu", total: int = 32768, nseq: int = 16,
                   lo: int = 512, hi: int = 4096, block: int = 64) -> Workload:
    """Write path only: ``total`` new tokens over ``nseq`` ragged sequences for
    8 KV heads x head_dim 128, bf16 Student-t (nu = 3) values, scattered into a
    shuffled page-16 pool."""
    g = _gen(3000 + seed, device)
    rng = np.random.default_rng(np.random.SeedSequence(3000 + seed))
    hkv, d = 8, 128
    lens = prefill_lengths(total, nseq, lo, hi, rng)
    k = _student_t3((total, hkv, d), g, device)
    v = _student_t3((total, hkv, d), g, device)
    return _make("prefill_append", hkv, hkv, d, block, torch.bfloat16, lens, k, v, None, rng, device)


def long_context_decode(seed: int = 4, device="cpu", batch: int = 8, context: int = 131072,
                        block: int = 64) -> Workload:
    """Qwen3-4B-shaped layer: 32 q heads / 8 KV heads, head_dim 128, bf16 K, V
    ~ N(0,1) times a per-(KV head, channel) scale log-uniform in [0.1, 10]
    (separately for K and V); randomly permuted page table."""
    g = _gen(4000 + seed, device)
    rng = np.random.default_rng(np.random.SeedSequence(4000 + seed))
    hq, hkv, d = 32, 8, 128
    t = batch * context
    lo, hi = math.log(0.1), math.log(10.0)
    ks = torch.exp(lo + (hi - lo) * torch.rand((hkv, d), generator=g, device=device))
    vs = torch.exp(lo + (hi - lo) * torch.rand((hkv, d), generator=g, device=device))
    k = _normal((t, hkv, d), g, device) * ks
    v = _normal((t, hkv, d), g, device) * vs
    q = _normal((batch, hq, d), g, device)
    return _make("long_context_decode", hq, hkv, d, block, torch.bfloat16, [context] * batch, k, v,
                 q, rng, device)


def lognormal_contexts(batch: int, rng: np.random.Generator, median: float = 2048.0,
                       sigma: float = 1.0, cap: int = 32768) -> np.ndarray:
    x = np.exp(rng.normal(math.log(median), sigma, batch))
    return np.clip(np.round(x), 1, cap).astype(np.int32)


def concurrency_step(seed: int = 5, device="cpu", batch: int = 32, block: int = 64,
                     steps: int = 1, cap: int = 32768) -> tuple[Workload, list[Workload]]:
    """70B-shaped layer: 64 q heads / 8 KV heads, head_dim 128, ragged contexts
    lognormal (median 2048, capped at ``cap``).  Returns the prefill workload
    (whole context) and ``steps`` decode steps, each appending 1 token per
    sequence at the next position and then attending over it."""
    g = _gen(5000 + seed, device)
    rng = np.random.default_rng(np.random.SeedSequence(5000 + seed))
    hq, hkv, d = 64, 8, 128
    ctx = lognormal_contexts(batch, rng, cap=cap)
    cap_lens = ctx + steps
    bt, total = paged_layout(ctx, cap_lens, rng)
    seq, pos = _fill_tokens(ctx)
    t = int(ctx.sum())
    k = _normal((t, hkv, d), g, device)
    v = _normal((t, hkv, d), g, device)
    fill = Workload("concurrency_fill", hq, hkv, d, block, torch.bfloat16, ctx.astype(np.int32),
                    bt, total, k.to(torch.bfloat16), v.to(torch.bfloat16),
                    torch.from_numpy(slots_for(bt, seq, pos)).to(device), None, seq, pos)
    out = []
    for s in range(steps):
        sseq = np.arange(batch, dtype=np.int64)
        spos = (ctx + s).astype(np.int64)
        kk = _normal((batch, hkv, d), g, device)
        vv = _normal((batch, hkv, d), g, device)
        q = _normal((batch, hq, d), g, device)
        out.append(Workload("concurrency_step", hq, hkv, d, block, torch.bfloat16,
                            (ctx + s + 1).astype(np.int32), bt, total, kk.to(torch.bfloat16),
                            vv.to(torch.bfloat16),
                            torch.from_numpy(slots_for(bt, sseq, spos)).to(device),
                            q.to(torch.bfloat16), sseq, spos))
    return fill, out


def random_decode(seed: int, device="cpu", batch: int = 3, hq: int = 8, hkv: int = 2,
                  d: int = 128, block: int = 64, dtype=torch.bfloat16, seq_lens=None,
                  outlier_factor: float = 10.0) -> Workload:
    """Small generic decode case for edge-case tests (ragged lengths, empty
    sequences, partial pages)."""
    g = _gen(9000 + seed, device)
    rng = np.random.default_rng(np.random.SeedSequence(9000 + seed))
    if seq_lens is None:
        seq_lens = rng.integers(1, 200, batch)
    seq_lens = np.asarray(seq_lens, np.int32)
    t = int(seq_lens.sum())
    k = _outliers(_normal((t, hkv, d), g, device), 2, outlier_factor, g, device)
    v = _outliers(_normal((t, hkv, d), g, device), 2, outlier_factor, g, device)
    q = _normal((len(seq_lens), hq, d), g, device)
    return _make("random_decode", hq, hkv, d, block, dtype, seq_lens, k, v, q, rng, device)


# ---------------------------------------------------------------------------
# High-precision windows: the first w_sink tokens and the last w_recent tokens
# of each sequence also live as bf16 in a separate window pool.  Window
# position of token t: t for t < w_sink, else w_sink + (t - w_sink) % w_recent
# (a ring, so a new token overwrites the one that leaves the window).


def window_layout(batch: int, w_sink: int, w_recent: int, rng: np.random.Generator):
    """Window block table [batch][pages per window] over a seeded permutation
    of the window pool; returns (table, pool pages)."""
    per = max(1, (w_sink + w_recent + PAGE - 1) // PAGE)
    perm = rng.permutation(batch * per).astype(np.int32)
    return perm.reshape(batch, per), batch * per


def window_slots(win_bt: np.ndarray, seq: np.ndarray, pos: np.ndarray, final_len: np.ndarray,
                 w_sink: int, w_recent: int) -> np.ndarray:
    """Window-pool slot of each token (seq[i], pos[i]) that is still inside
    its sequence's windows once the sequence has final_len[seq] tokens; -1 for
    the others (so one append call never writes a ring slot twice)."""
    seq = np.asarray(seq)
    pos = np.asarray(pos).astype(np.int64)
    flen = np.asarray(final_len)[seq].astype(np.int64)
    keep = (pos < w_sink) | (pos >= flen - w_recent)
    wpos = np.where(pos < w_sink, pos, w_sink + (pos - w_sink) % max(w_recent, 1))
    pages = win_bt[seq, wpos // PAGE]
    slots = pages.astype(np.int64) * PAGE + wpos % PAGE
    return np.where(keep, slots, -1).astype(np.int32)


def bits(x: torch.Tensor) -> np.ndarray:
    """16-bit float tensor -> numpy uint16 bit patterns (host copy)."""
    return x.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
