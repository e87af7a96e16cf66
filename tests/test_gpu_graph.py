"""The layer step captured as one HIP graph and replayed (the way bench.py
times it) gives bit-identical results to the eager launches, on every replay,
with eager work and synchronisations between the replays: the absorbed step
(configs 2, 3, 4) and the pooled one (configs 5 and 6)."""
import pytest
import torch

import bench
from sparse_attention_scores_amd import workloads as W
from tests.parity import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    from sparse_attention_scores_amd import binding
    binding.load()
    return binding


@pytest.mark.parametrize("cfg,over", [(2, dict(B=4, Tk=3000)), (4, dict(B=2, Tk=20000)),
                                      (3, dict(Tq=300, Tk=300))])
def test_step_graph_replay_matches_eager(dsa, cfg, over):
    note(f"graph replay config {cfg} {over}")
    inp = W.make(cfg, device="cuda", **over)
    step = bench.Step(dsa, inp)

    def run_once():
        for s in step.stages:
            getattr(step, s)()

    run_once()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (step.S, step.idx, step.out, step.lse)]
    g = bench.capture_step(torch, run_once)
    # other inputs in between: the graph must reread its inputs on every replay
    other = W.make(cfg, device="cuda", seed=inp["seed"] + 7, **over)
    other_step = bench.Step(dsa, other)
    for rep in range(3):
        for t in (step.S, step.idx, step.out, step.lse):
            t.fill_(-7)  # eager work on the outputs between the replays
        other_step.index()
        other_step.topk()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("scores", "idx", "out", "lse"),
                              (step.S, step.idx, step.out, step.lse), ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"


@pytest.mark.parametrize("cfg,over", [(5, dict(L=1030)), (6, dict(L=5000))])
def test_pooled_step_graph_replay_matches_eager(dsa, cfg, over):
    """The pooled step (pool keys, pooled scores, pool select, per-head
    attention: the masked-tile kernels on config 5's shape, the per-head
    gather on config 6's) captured once and replayed three times, with other
    inputs' eager work and poisoned outputs between the replays."""
    note(f"graph replay, pooled config {cfg} {over}")
    inp = W.make(cfg, device="cuda", **over)
    step = bench.PooledStep(dsa, inp)

    def run_once():
        for s in step.stages:
            getattr(step, s)()

    run_once()
    torch.cuda.synchronize()
    outs = (step.pk, step.npools, step.S, step.tok, step.out, step.lse)
    names = ("pooled keys", "n_pools", "scores", "tok", "out", "lse")
    ref = [t.clone() for t in outs]
    g = bench.capture_step(torch, run_once)
    other = W.make(cfg, device="cuda", seed=inp["seed"] + 7, **over)
    other_step = bench.PooledStep(dsa, other)
    for rep in range(3):
        for t in outs:
            t.fill_(-7)
        for s in other_step.stages:
            getattr(other_step, s)()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, outs, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"
