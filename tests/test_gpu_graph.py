"""The whole path captured in a HIP graph (as bench.py times it) replays to
the same bytes as eager launches, replay after replay, with eager work and
synchronisations in between, and matches the oracle on the tiny config."""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pipeline():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_indexer_logits_amd.pipeline import IndexerStep
    return IndexerStep


def _step(IndexerStep, d, cfg, outputs=None):
    return IndexerStep(d["q"], d["k"], d["w"], d["limit"], cfg.topk, d["kv_fp4"], d["kv_scale"],
                       d["block_table"], d["row_seq"], d["q_scale"], d["k_scale"],
                       outputs=outputs)


@pytest.mark.parametrize("name", ["tiny", "flash_decode", "flash_prefill"])
def test_graph_replays_match_eager(pipeline, name):
    x = workloads.inputs(name)
    cfg = x["cfg"]
    print(f"[graph] config={name}", flush=True)
    d = workloads.to_device(x)
    step = _step(pipeline, d, cfg)
    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in step.outputs()]
    # a second input copy writing the same buffers, to interleave eager work
    other = _step(pipeline, {**d, "q": d["q"].clone(), "w": d["w"].clone() * 2}, cfg,
                  outputs=step.outputs())

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in step.outputs():
            t.fill_(-7)        # stale contents must be overwritten by the replay
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(step.outputs(), eager):
            assert torch.equal(a, b), f"{name}: replay {rep} differs from eager"
        other()                # eager work between replays
        torch.cuda.synchronize()
    if name == "tiny":
        idx = step.idx.cpu().numpy()
        ref = oracle.indexer_topk(step.logits.cpu().numpy().reshape(cfg.rows, cfg.K),
                                  x["limit"].reshape(-1), cfg.topk)
        assert np.array_equal(idx, ref)


def test_paged_step_keeps_its_key_cache(pipeline):
    """A paged-key step built from a key cache that nothing else references
    (bench.py's per-copy clones) still reads that cache after the caller's
    reference is gone and its old block could be handed out again: the step
    holds every tensor its C arguments point to."""
    name = "flash_decode_fp4"
    x = workloads.inputs(name)
    cfg = x["cfg"]
    print(f"[graph] paged step lifetime, config={name}", flush=True)
    d = workloads.to_device(x)

    def paged(kc, outputs=None):
        return pipeline(d["q"], None, d["w"], d["limit"], cfg.topk, d["kv_fp4"], d["kv_scale"],
                        d["block_table"], d["row_seq"], d["q_scale"], None, outputs=outputs,
                        k_cache=kc, k_cache_scale=d["kc_scale"], K=cfg.K)

    base = paged(d["kc"])
    base()
    torch.cuda.synchronize()
    eager = [t.clone() for t in base.outputs()]
    other = paged(d["kc"].clone(), outputs=base.outputs())   # the only reference to the clone
    junk = [torch.full_like(d["kc"], 0x77) for _ in range(3)]  # would take a freed block
    other()
    torch.cuda.synchronize()
    del junk
    for a, b in zip(base.outputs(), eager):
        assert torch.equal(a, b), "a step on a copy of the key cache differs from the original's"
