"""Serving steps (append one token per sequence, then decode) captured in a
HIP graph through torch.cuda.graph.  The entry points only launch kernels (no
allocation, no memset), so a captured step can be replayed: every replay,
with eager work and synchronisations between replays, must give the eager
result bit for bit, outputs and cache pages alike."""
import pytest
import torch

import bit_kv_cache_block_amd as kvq
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _setup(kind, fill):
    if kind == "bf16":
        cache = kvq.Bf16Cache(fill.num_pages, fill.hkv, fill.d, DEV)
        fns = (kvq.kvq_append_paged_bf16, kvq.kvq_decode_attn_bf16)
    else:
        cache = kvq.Int4Cache(fill.num_pages, fill.hkv, fill.d, 64 if kind == "int4_rot" else 0, DEV)
        fns = (kvq.kvq_append_paged, kvq.kvq_decode_attn)
    fns[0](cache, fill.k, fill.v, fill.slot_mapping)
    return cache, fns


@pytest.mark.parametrize("batch", [1, 8, 32])
@pytest.mark.parametrize("kind", ["int4_rot", "int4_plain", "bf16"])
def test_graph_replay_matches_eager(kind, batch):
    fill, st = workloads.concurrency_step(5, device=DEV, batch=batch, block=64, steps=3)
    bt = torch.from_numpy(st[0].block_table).to(DEV)
    sls = [torch.from_numpy(x.seq_lens).to(DEV) for x in st]
    maxlen = int(st[-1].max_seq_len)
    nws = kvq.kvq_decode_workspace_bytes(batch, fill.hq, fill.hkv, fill.d, maxlen)
    print(f"graph {kind} batch {batch}: workspace {nws} bytes", flush=True)

    def steps(cache, fns, outs, ws):
        for i, x in enumerate(st):
            fns[0](cache, x.k, x.v, x.slot_mapping)
            fns[1](cache, x.q, bt, sls[i], maxlen, x.sm_scale, out=outs[i], workspace=ws)

    def buffers():
        outs = [torch.empty((batch, fill.hq, fill.d), dtype=torch.float32, device=DEV) for _ in st]
        return outs, torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)

    cache_e, fns = _setup(kind, fill)
    outs_e, ws_e = buffers()
    steps(cache_e, fns, outs_e, ws_e)
    torch.cuda.synchronize()

    cache_g, _ = _setup(kind, fill)
    outs_g, ws_g = buffers()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps(cache_g, fns, outs_g, ws_g)
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(4):
        for o in outs_g:
            o.fill_(float("nan"))
        ws_g.fill_(0xFF)                     # stale workspace bytes between replays
        scratch.mul_(1.0001).add_(0.5)       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(len(st)):
            assert torch.equal(outs_g[i], outs_e[i]), f"{kind} batch {batch} replay {rep} step {i}"
        assert torch.equal(cache_g.pool, cache_e.pool), f"{kind} batch {batch} replay {rep}: pages"
