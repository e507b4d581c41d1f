"""GPU tests of the layer's stream behaviour.

* Stream capture: the forward captured into a graph on a side stream of
  torch's own, replayed several times with eager work and synchronisations in
  between, gives the eager result bitwise on every replay (the library
  enqueues no memset or copy, only kernels).
* Host threads: two threads, each with its own stream and workspace, calling
  the layer repeatedly at the same time, give the single-threaded result
  bitwise; threads that call the forward once and exit match too, and leave
  no side stream behind (the forward uses none).
* The backward runs its shared experts' branch on a side stream, one per
  host thread and device: threads that call it once and exit destroy theirs.
"""
import sys
import threading

import pytest
import torch

import workloads
from parity import Case

pytestmark = pytest.mark.gpu
C = workloads.CONFIGS


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _forward(case, out, ws):
    import mixture_experts_layer_mk_amd as moe
    c, d = case.cfg, case.dev
    moe.moe_layer_forward(d["x"], d["w_gate"], d["routed"], d["shared"], c.top_k,
                          score=c.score, norm_topk=c.norm_topk, n_groups=c.n_groups,
                          topk_groups=c.topk_groups, select_bias=d["select_bias"],
                          logit_bias=d["logit_bias"], routed_scale=c.routed_scale,
                          out=out, workspace=ws)


def _workspace(case):
    import mixture_experts_layer_mk_amd as moe
    c = case.cfg
    desc = moe.make_desc(c.T, c.d, c.n_routed, c.top_k, c.inner, c.n_shared, c.shared_inner,
                         n_groups=c.n_groups, topk_groups=c.topk_groups, score=c.score,
                         norm_topk=c.norm_topk, routed_scale=c.routed_scale, dtype=c.dtype)
    return torch.empty(moe.workspace_size(desc), dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("name,cfg", [
    ("skewed-16b-small", C["skewed-16b-small"]),
    ("16b-T2600", C["deepseekmoe-16b"].replace(T=2600, seed=9)),
])
def test_forward_graph_capture_replays_match_eager(name, cfg):
    case = Case(cfg)
    say(f"[graph] {name}")
    ws = _workspace(case)
    ref = torch.empty_like(case.dev["x"])
    _forward(case, ref, ws)                      # eager; creates the side stream
    torch.cuda.synchronize()
    out = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _forward(case, out, ws)                  # warm-up on the capturing stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _forward(case, out, ws)
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {i} differs from the eager call"
        scratch = torch.empty_like(ref)          # eager work between the replays
        _forward(case, scratch, ws)
        torch.cuda.synchronize()
        assert torch.equal(scratch, ref)
    say(f"[graph] {name}: 3 replays equal")


def test_forward_concurrent_host_threads():
    case = Case(C["deepseekmoe-16b"].replace(T=1500, seed=10))
    ws0 = _workspace(case)
    ref = torch.empty_like(case.dev["x"])
    _forward(case, ref, ws0)
    torch.cuda.synchronize()
    results, errors = {}, []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            ws = _workspace(case)
            outs = [torch.empty_like(ref) for _ in range(4)]
            with torch.cuda.stream(s):
                for o in outs:
                    _forward(case, o, ws)
            s.synchronize()
            results[k] = outs
        except Exception as e:   # reported below, in the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not errors, errors
    assert sorted(results) == [0, 1]
    for k in results:
        for o in results[k]:
            assert torch.equal(o, ref)
    say("[threads] 2 threads x 4 calls equal")


def test_forward_short_lived_threads():
    """Threads that call the forward once and exit: results bitwise equal to
    the main thread's, and no side stream is created."""
    import mixture_experts_layer_mk_amd as moe
    case = Case(C["deepseekmoe-16b"].replace(T=1200, seed=11))
    ws0 = _workspace(case)
    ref = torch.empty_like(case.dev["x"])
    _forward(case, ref, ws0)
    torch.cuda.synchronize()
    base = moe.side_stream_count()
    results, errors = {}, []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            ws = _workspace(case)
            out = torch.empty_like(ref)
            with torch.cuda.stream(s):
                _forward(case, out, ws)
            s.synchronize()
            results[k] = out
        except Exception as e:   # reported below, in the main thread
            errors.append(repr(e))

    for wave in range(4):        # 4 waves of 3 concurrent short-lived threads
        threads = [threading.Thread(target=worker, args=(3 * wave + j,)) for j in range(3)]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
    assert not errors, errors
    assert sorted(results) == list(range(12))
    for k, o in results.items():
        assert torch.equal(o, ref), f"thread {k} differs"
    assert moe.side_stream_count() == base
    say("[threads] 12 short-lived forward threads equal")


def test_backward_short_lived_threads_release_side_streams():
    """Threads that call the backward once and exit: each gets its own side
    stream (gradients bitwise equal to the main thread's) and destroys it on
    exit, so the library's side-stream count returns to where it was."""
    import time
    import mixture_experts_layer_mk_amd as moe
    import workloads as wl
    cfg = C["deepseekmoe-16b"].replace(T=300, d=256, inner=128, shared_inner=128, seed=12)
    case = Case(cfg)
    d = case.dev
    dout = torch.from_numpy(wl.make_inputs(cfg).dout()).to(torch.bfloat16).cuda()

    def bwd():
        return moe.moe_layer_backward(d["x"], d["w_gate"], d["routed"], d["shared"], cfg.top_k,
                                      dout)
    ref = bwd()
    torch.cuda.synchronize()
    base = moe.side_stream_count()
    assert base >= 1            # the main thread's own
    results, errors, during = {}, [], []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                g = bwd()
            s.synchronize()
            during.append(moe.side_stream_count())
            results[k] = g
        except Exception as e:   # reported below, in the main thread
            errors.append(repr(e))

    for wave in range(4):
        threads = [threading.Thread(target=worker, args=(3 * wave + j,)) for j in range(3)]
        for t in threads:
            t.start()
        for t in threads:
            t.join(timeout=120)
    assert not errors, errors
    assert sorted(results) == list(range(12))
    for k, g in results.items():
        assert torch.equal(g["dx"], ref["dx"]), f"thread {k}: dx differs"
        for part in ("routed", "shared"):
            for a, b in zip(g[part], ref[part]):
                assert torch.equal(a, b), f"thread {k}: {part} gradients differ"
    assert min(during) >= base + 1
    # join() returns when the Python thread is done; the thread-exit
    # destructors run just after, as the OS thread ends
    deadline = time.time() + 10
    while moe.side_stream_count() != base and time.time() < deadline:
        time.sleep(0.05)
    assert moe.side_stream_count() == base, "side streams of exited threads were kept"
    say(f"[threads] 12 short-lived backward threads equal; side streams back to {base}")
