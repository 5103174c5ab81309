"""GPU parity of the two-stream pinned-host pipeline: resident slots in HBM,
the full K|V store in pinned host memory, copies on a background stream.

Run A synchronises after every layer-step and checks each step against the
oracle: scores, top-K, plan and slot tables, and attention over the resident
store (which must hold exactly the host tiles its slot table names, byte for
byte).  Run B repeats the same steps free-running, ordered only by the
pipeline's events, and must reproduce run A bit for bit.  Runs C and D do the
same with a bounded delay kernel (a clock spin that always ends) enqueued
before every fused step on the main stream (C), or before every copy on the
copy stream (D).  C holds each attention back while the copy stream is free:
a copy not ordered after the attention that last read its slots (the WAR
hazard of v2 §3.3.1's per-layer event ordering) would overwrite them first.
D holds each copy back: a next-step attention not ordered after the copy
into its slots (RAW) would read the old tiles.  Either missing event makes
C or D differ from A deterministically, not by timing luck.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_kv_block_quest_amd import _lib, ops, pipeline, synth
from test_gpu_step import check_step, small

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)


def build(wl, dev, n_layers, opts=None, want_scores=True, host_capacity=None, host_workers=1):
    layers, q0s, full = [], [], []
    for l in range(n_layers):
        qf = synth.queries(wl, dev, layer=l)
        keys = synth.keys(wl, qf[:, 0], dev, layer=l)
        vt = synth.v_tiles(synth.values(wl, dev, layer=l), wl.B)
        kt = keys.view(wl.R, wl.H, wl.n_blk, wl.B, wl.D)
        store, k, v = synth.interleave_kv(kt, vt)
        summ = ops.build_summaries(k, wl.B)
        q0 = qf.to(wl.dtype)
        if host_capacity is None:
            host = torch.empty(store.shape, dtype=store.dtype, pin_memory=True)
            host.copy_(store)
            layers.append(pipeline.PipelineLayer(wl, host, summ, q0, dev, opts=opts,
                                                 want_scores=want_scores))
        else:  # remote memory holds whole blocks [R][n_blk][H][2][B][D]
            whole = store.permute(0, 2, 1, 3, 4, 5).contiguous()
            remote = torch.empty(whole.shape, dtype=whole.dtype, pin_memory=True)
            remote.copy_(whole.cpu())
            layers.append(pipeline.PipelineLayer(wl, None, summ, q0, dev, opts=opts,
                                                 want_scores=want_scores, remote_store=remote,
                                                 host_capacity=host_capacity,
                                                 host_workers=host_workers))
        q0s.append(q0)
        full.append((k, v, store))
    return pipeline.Pipeline(layers), q0s, full


def query_steps(wl, dev, n_layers, n_steps):
    """[t][l] stacked queries in wl.dtype, the AR(1) drift of each layer's first queries."""
    out = [[None] * n_layers for _ in range(n_steps)]
    for l in range(n_layers):
        g = synth.generator(wl.seed + 1000 * l, synth.S_DRIFT, "cuda")
        cur = synth.queries(wl, dev, layer=l)
        for t in range(n_steps):
            out[t][l] = cur.to(wl.dtype)
            cur = synth.drift(cur[:, 0], wl.rho, g)
    return out


def resident_matches_host(layer, blk):
    """Every filled slot holds the host tiles of the block its slot table names
    (from the full host store, or from remote memory through the cache)."""
    R, H, K = blk.shape
    b = blk.long()
    assert bool((b >= 0).all()), "pipeline slots are all filled after seeding"
    r = torch.arange(R, device=b.device)[:, None, None]
    g = torch.arange(H, device=b.device)[None, :, None]
    if layer.tier is None:
        want = layer.host.to(b.device)[r, g, b]
    else:
        want = layer.remote.to(b.device)[r, b, g]
    assert torch.equal(layer.res.view(torch.int16), want.view(torch.int16))


# Bounded spin of the delay kernel (torch.cuda._sleep counts shader clock
# cycles): ~0.5 ms at the MI355X's 2.4 GHz, far longer than a small fused step
# or copy, and it always ends.
DELAY_CYCLES = 1_200_000


def run_pipeline_case(cuda, wl, n_layers, n_steps, units=None, opts=None, host_capacity=None,
                      host_workers=1, n_runs=3):
    dev = cuda
    qs = query_steps(wl, dev, n_layers, n_steps)
    n_valid = np.full(wl.R, wl.n_blk, np.int32)
    if units is None:
        units = [(r, g) for r in range(wl.R) for g in range(wl.H)]

    # run A: checked step by step
    pa, q0s, full = build(wl, dev, n_layers, opts, host_capacity=host_capacity,
                          host_workers=host_workers)
    pa.seed(q0s)
    pa.drain()
    torch.cuda.synchronize()
    outs_a = []
    models = None
    if host_capacity is not None:  # replay the GPU's plans through the reference cache
        nb = wl.n_blk
        models = [oracle.HostTierModel([host_capacity] * wl.R, nb) for _ in range(n_layers)]
        for l, L in enumerate(pa.layers):
            models[l].fetch(1, L.plan["plan_count"].cpu().numpy(), L.plan["plan_src"].cpu().numpy(),
                            L.blk[0].cpu().numpy())
    for l, layer in enumerate(pa.layers):
        resident_matches_host(layer, pa.resident_blocks(l, 0))
    for t in range(n_steps):
        for l in range(n_layers):
            say(f"  pipeline A step {t} layer {l}")
            L = pa.layers[l]
            res = pa.layer_step(t, l, qs[t][l])
            pa.drain()
            torch.cuda.synchronize()
            a, b = t % 2, 1 - t % 2
            k, v, _ = full[l]
            check_step(wl, qs[t][l], L.summ, k, v, L.blk[a], L.stamp[a], L.blk[b], L.stamp[b],
                       res, t + 1, n_valid, None, None, units)
            outs_a.append((res["out"].clone(), res["lse"].clone(), res["topk_idx"].clone()))
            resident_matches_host(L, L.blk[b])
            if models is not None:
                models[l].fetch(t + 2, L.plan["plan_count"].cpu().numpy(),
                                L.plan["plan_src"].cpu().numpy(), L.blk[b].cpu().numpy())
                np.testing.assert_array_equal(L.map.numpy(), models[l].map)
                assert L.tier.state()[2]["failed"] == 0
    del pa

    # runs B (free-running, events only), C (delay before every fused step on
    # the main stream) and D (delay before every copy on the copy stream)
    for name, delay in (("B", None), ("C", "main"), ("D", "copy"))[:n_runs]:
        pb, q0s, _ = build(wl, dev, n_layers, opts, want_scores=False,
                           host_capacity=host_capacity, host_workers=host_workers)
        pb.seed(q0s)
        outs_b = []
        for t in range(n_steps):
            for l in range(n_layers):
                if delay == "main":
                    torch.cuda._sleep(DELAY_CYCLES)  # the current (main) stream
                elif delay == "copy":  # lands before this layer-step's copy
                    with torch.cuda.stream(pb.copy_stream):
                        torch.cuda._sleep(DELAY_CYCLES)
                res = pb.layer_step(t, l, qs[t][l])
                outs_b.append((res["out"].clone(), res["lse"].clone(), res["topk_idx"].clone()))
        pb.drain()
        torch.cuda.synchronize()
        say(f"  pipeline {name} done")
        for i, (xa, xb) in enumerate(zip(outs_a, outs_b)):
            for ta, tb in zip(xa, xb):
                assert torch.equal(ta, tb), f"run {name}: layer-step {i} differs from run A"
        for l in range(n_layers):
            resident_matches_host(pb.layers[l], pb.resident_blocks(l, n_steps))
        del pb


def test_pipeline_small(cuda):
    wl = small("qwen3-8b-1layer", R=2, H=2, Hq=8, L=2048, K=16, cap=4)
    say("pipeline small: R=2 H=2 K=16 cap=4, 2 layers x 4 steps")
    run_pipeline_case(cuda, wl, 2, 4)


def test_pipeline_full_shape(cuda):
    """The Qwen3-8B pipeline shape (R=8, 32K context, K=128, cap 16), two layers."""
    wl = synth.workload("qwen3-8b-pipeline", layers=2)
    say("pipeline qwen3-8b shape, 2 layers x 2 steps")
    run_pipeline_case(cuda, wl, 2, 2, units=[(0, 0), (3, 5), (7, 7)], n_runs=1)


def test_pipeline_cache_budget_too_small(cuda):
    """A decode-host budget below the union of the heads' working sets: the
    seeding fetch finds no evictable block for some planned blocks.  The
    dispatcher still launches the gather and records the copy event (nothing
    waits forever), and the failure comes back as EINVAL from the host wait
    that the pipeline makes before using that event.  The reference cache on
    the same plan fails the same way (v2 §3.2.3: the budget must hold the
    working set)."""
    wl = small("qwen3-8b-1layer", R=2, H=2, Hq=8, L=2048, K=16, cap=4)
    cap = 20  # per request; the two heads' seeding sets hold up to 32 blocks
    say(f"pipeline with decode-host cache of {cap} blocks per request (too small)")
    p, q0s, _ = build(wl, cuda, 1, host_capacity=cap)
    p.seed(q0s)
    with pytest.raises(_lib.OasisError) as e:
        p.drain()
    assert e.value.status == _lib.OASIS_EINVAL
    torch.cuda.synchronize()
    L = p.layers[0]
    stats = L.tier.state()[2]
    assert stats["failed"] > 0
    # the same plan in the reference cache also runs out of evictable blocks
    model = oracle.HostTierModel([cap] * wl.R, wl.n_blk)
    with pytest.raises(RuntimeError):
        model.fetch(1, L.plan["plan_count"].cpu().numpy(), L.plan["plan_src"].cpu().numpy(),
                    L.blk[0].cpu().numpy())


@pytest.mark.parametrize("cap,workers", [(40, 1), (36, 1), (36, 3)])
def test_pipeline_with_decode_host_cache(cuda, cap, workers):
    """Remote memory holds whole blocks; a bounded decode-host cache (2 heads x
    16 slots = at most 32 working-set blocks per request) feeds the gather
    through its union map; the cache evicts and refetches as the sets drift.
    The fetch runs on its own stream, on `workers` host threads."""
    wl = small("qwen3-8b-1layer", R=2, H=2, Hq=8, L=2048, K=16, cap=4)
    say(f"pipeline with decode-host cache, capacity {cap}, {workers} fetch workers")
    run_pipeline_case(cuda, wl, 2, 5, host_capacity=cap, host_workers=workers)


def test_pipeline_with_decode_host_cache_full_shape(cuda):
    """The Qwen3-8B pipeline shape with f_Host = 0.6 (1229 cached blocks per
    request of 2048), four fetch workers, two layers."""
    wl = synth.workload("qwen3-8b-pipeline", layers=2)
    say("pipeline qwen3-8b shape with decode-host cache 1229, 2 layers x 2 steps")
    run_pipeline_case(cuda, wl, 2, 2, units=[(0, 0), (3, 5), (7, 7)], host_capacity=1229,
                      host_workers=4, n_runs=1)
