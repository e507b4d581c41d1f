"""GPU parity: the HIP layer (through the C ABI) against the CPU oracle.

Sizes: every workload at reduced T (full hidden/inner/expert shapes)
compared on every token, spanning several GEMM tiles with ragged tails; the
full-size workloads compared on every token as well, plus properties that
hold at any size; and the edge cases of the method.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from parity import Case, check_case

pytestmark = pytest.mark.gpu

C = workloads.CONFIGS


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


REDUCED = {
    "tiny-fp32": C["tiny-fp32"],
    "tiny-fp32-ragged": C["tiny-fp32"].replace(T=203, seed=3),
    "2b-T2000": C["deepseekmoe-2b"].replace(T=2000),
    "16b-T2600": C["deepseekmoe-16b"].replace(T=2600),
    "16b-T1000": C["deepseekmoe-16b"].replace(T=1000, seed=1),
    # 1024 tokens: the fused router and the side stream's fork at the start of
    # the call; 1023: the split router and the fork after the dispatch.
    "16b-T1023": C["deepseekmoe-16b"].replace(T=1023, seed=6),
    "16b-T1024": C["deepseekmoe-16b"].replace(T=1024, seed=7),
    "v3-d512-T4096": C["deepseek-v3"].replace(d=512, inner=256, shared_inner=256),
    "v3-d512-T700": C["deepseek-v3"].replace(T=700, d=512, inner=256,
                                             shared_inner=256, seed=2),
    "skewed-16b-small": C["skewed-16b-small"],
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_reduced_all_tokens(name):
    cfg = REDUCED[name]
    say(f"[parity] {name}: {cfg}")
    info = check_case(Case(cfg))
    say(f"[parity] {name}: {info}")


def test_tiny_fp32_routing_bit_exact():
    """On the tiny workload no token is near a tie: indices and counts must be
    exactly the oracle's."""
    case = Case(C["tiny-fp32"])
    info = check_case(case)
    assert info["ambiguous"] == 0


@pytest.mark.parametrize("name", ["deepseekmoe-2b", "deepseekmoe-16b", "deepseek-v3"])
def test_full_size_all_tokens(name):
    """The full-size workloads in the launch configuration the benchmark times,
    every token against the oracle (run expert by expert)."""
    cfg = C[name]
    say(f"[parity-full] {name}: generating inputs")
    case = Case(cfg)
    say(f"[parity-full] {name}: running")
    info = check_case(case)
    assert info["rows"] == cfg.T
    say(f"[parity-full] {name}: {info}")


def test_deterministic_bitwise():
    case = Case(C["deepseekmoe-16b"].replace(T=3000, seed=5))
    o1, r1 = case.run_gpu()
    o2, r2 = case.run_gpu()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    for k in r1:
        assert torch.equal(r1[k], r2[k])


@pytest.mark.parametrize("name,dtype", [("skewed-16b-small", None), ("v3-d512-T700", None),
                                        ("16b-T2600", None), ("16b-T2600", "fp8"),
                                        ("skewed-16b-small", "fp8"), ("16b-T1023", None),
                                        ("16b-T1024", None), ("v3-d512-T4096", "fp8")])
def test_traced_matches_untraced(name, dtype):
    """A traced call (events recorded between the stages) runs the same
    launches as an untraced one: the outputs are bitwise equal, on repeated
    calls too.  Cases: weight-streaming tiles (skewed batch, V3 routing),
    256-row tiles, FP8 layers, the router's split/fused switch at 1023/1024
    tokens."""
    from mixture_experts_layer_mk_amd import HipEvents, trace_stage_names
    cfg = REDUCED[name] if dtype is None else REDUCED[name].replace(dtype=dtype)
    case = Case(cfg)
    ev = HipEvents(len(trace_stage_names()) + 1)
    try:
        traced, _ = case.run_gpu(trace_events=ev.handles)
        traced = traced.clone()
        outs = [case.run_gpu()[0].clone() for _ in range(3)]
        torch.cuda.synchronize()
    finally:
        ev.close()
    for o in outs:
        assert torch.equal(o, traced)


def test_intermediates_dispatch_exact():
    """Counts, offsets and the expert-contiguous permutation are integers and
    copies: exact against the oracle's dispatch of the GPU's own choices."""
    import oracle
    from mixture_experts_layer_mk_amd import make_desc, workspace_layout, workspace_size
    cfg = C["deepseekmoe-16b"].replace(T=1500, seed=4)
    case = Case(cfg)
    desc = make_desc(cfg.T, cfg.d, cfg.n_routed, cfg.top_k, cfg.inner, cfg.n_shared,
                     cfg.shared_inner)
    lay = workspace_layout(desc)
    ws = torch.empty(workspace_size(desc), dtype=torch.uint8, device="cuda")
    out, routing = case.run_gpu(workspace=ws)
    torch.cuda.synchronize()
    T, K, d, E = cfg.T, cfg.top_k, cfg.d, cfg.n_routed

    def view(off, n, dt):
        nbytes = n * torch.empty((), dtype=dt).element_size()
        return ws[off:off + nbytes].view(dt).cpu()
    idx = routing["topk_idx"].cpu().numpy()
    dsp = oracle.dispatch(idx, E)
    assert np.array_equal(view(lay["counts_i32"], E, torch.int32).numpy(), dsp.counts)
    assert np.array_equal(view(lay["offsets_i32"], E + 1, torch.int32).numpy(), dsp.offsets)
    assert np.array_equal(view(lay["row_src_i32"], T * K, torch.int32).numpy(), dsp.row_src)
    assert np.array_equal(view(lay["slot_row_i32"], T * K, torch.int32).numpy().reshape(T, K),
                          dsp.slot_row)
    assert lay["xp"] == -1   # the gate/up GEMM gathers rows of x itself


def test_T_zero_and_one():
    case = Case(C["deepseekmoe-16b"].replace(T=1))
    check_case(case)
    d = case.dev
    x0 = d["x"][:0]
    from mixture_experts_layer_mk_amd import moe_layer_forward
    out = moe_layer_forward(x0, d["w_gate"], d["routed"], d["shared"], 6)
    assert out.shape == (0, 2048)
    # No tokens: the counts are still written (zeros), over whatever the
    # buffer held before -- called through the C ABI with a buffer of our own.
    import ctypes
    from mixture_experts_layer_mk_amd import _lib
    lib = _lib.load_library()
    cfg = case.cfg
    desc = _lib.make_desc(0, cfg.d, cfg.n_routed, cfg.top_k, cfg.inner, cfg.n_shared,
                          cfg.shared_inner)
    cnt = torch.full((cfg.n_routed,), 0x5a5a5a5a, dtype=torch.int32, device="cuda")
    w1, w3, w2 = d["routed"]
    s1, s3, s2 = d["shared"]
    ffn_r = _lib.FfnWeights(w1.data_ptr(), w3.data_ptr(), w2.data_ptr(), None, None, None)
    ffn_s = _lib.FfnWeights(s1.data_ptr(), s3.data_ptr(), s2.data_ptr(), None, None, None)
    torch.cuda.synchronize()
    st = lib.moe_layer_forward(ctypes.byref(desc), None, d["w_gate"].data_ptr(), None, None,
                               ffn_r, ffn_s, None, None, None, cnt.data_ptr(), None, 0,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, _lib.strerror(st)
    torch.cuda.synchronize()
    assert (cnt == 0).all(), "T = 0 left expert_counts unwritten"
    _, routing = moe_layer_forward(x0, d["w_gate"], d["routed"], d["shared"], 6,
                                   return_routing=True)
    assert (routing["expert_counts"] == 0).all()


def test_all_experts_kept_and_no_shared():
    cfg = C["deepseekmoe-16b"].replace(T=333, n_routed=8, top_k=8, n_shared=0,
                                       d=256, inner=128)
    check_case(Case(cfg))


def test_dense_reduction_bf16():
    """mN = mK = 1, K_s = 0: every token goes to the one expert with weight 1."""
    cfg = C["deepseekmoe-16b"].replace(T=777, n_routed=1, top_k=1, n_shared=0,
                                       d=512, inner=384)
    case = Case(cfg)
    info = check_case(case)
    out, routing = case.run_gpu()
    assert (routing["topk_w"] == 1.0).all() and (routing["topk_idx"] == 0).all()
    assert info["ambiguous"] == 0


def test_zero_gate_ties_take_lowest_index():
    """A zero gate makes every score equal: both sides keep experts 0..K-1."""
    cfg = C["deepseekmoe-16b"].replace(T=300, d=256, inner=128, shared_inner=128)
    case = Case(cfg)
    case.dev["w_gate"].zero_()
    out, routing = case.run_gpu()
    idx = routing["topk_idx"].cpu().numpy()
    assert (idx == np.arange(6)[None, :]).all()
    assert np.allclose(routing["topk_w"].cpu().numpy(), 1 / 64)


@pytest.mark.parametrize("T", [300, 2048])
def test_group_limit_ties_take_lowest_indices(T):
    """Group-limited routing on exact ties (a zero gate makes every sigmoid
    score 1/2; 8 groups of 32, 4 kept, 8 experts per token): with no
    selection bias groups 0..3 stay and experts 0..7 are kept; with four
    experts of groups 1 and 6 raised by 0.01, groups 1 and 6 lead with equal
    scores and groups 0 and 2 win the tie among the rest, so the raised
    experts come first (index order), then experts 0..3.  Both sides decide
    on the same fp32 values, so the choice must be exactly this (the 1e-5
    margin rule does not apply).  T = 300: the split router; 2048 tokens:
    more router blocks."""
    cfg = C["deepseek-v3"].replace(T=T, d=512, inner=256, shared_inner=256, seed=4)
    case = Case(cfg)
    case.dev["w_gate"].zero_()
    case.w_gate = np.zeros_like(case.w_gate)
    zero = torch.zeros(256, dtype=torch.float32)
    case.dev["select_bias"] = zero.cuda()
    case.select_bias = zero.numpy()
    out, routing = case.run_gpu()
    idx = routing["topk_idx"].cpu().numpy()
    assert (idx == np.arange(8)[None, :]).all()
    assert (routing["topk_w"].cpu().numpy() == np.float32(1 / 8)).all()
    check_case(case, out=out, routing=routing)
    raised = [32 + 5, 32 + 17, 192 + 3, 192 + 30]
    bias = torch.zeros(256, dtype=torch.float32)
    bias[raised] = 0.01
    case.dev["select_bias"] = bias.cuda()
    case.select_bias = bias.numpy()
    out, routing = case.run_gpu()
    idx = routing["topk_idx"].cpu().numpy()
    assert (idx == np.array(raised + [0, 1, 2, 3])[None, :]).all()
    assert (routing["topk_w"].cpu().numpy() == np.float32(1 / 8)).all()
    cnt = routing["expert_counts"].cpu().numpy()
    assert (cnt[raised + [0, 1, 2, 3]] == T).all() and cnt.sum() == 8 * T
    check_case(case, out=out, routing=routing)


def test_disabled_experts_never_chosen():
    """A logit bias of -inf switches experts off (the top-expert ablation is
    expressed this way): they get no tokens, the rest of the layer is exact."""
    cfg = C["deepseekmoe-16b"].replace(T=500, d=256, inner=128, shared_inner=128)
    case = Case(cfg)
    lb = torch.zeros(64, dtype=torch.float32)
    lb[[0, 5, 17, 63]] = -float("inf")
    case.dev["logit_bias"] = lb.cuda()
    case.logit_bias = lb.numpy()
    info = check_case(case)
    out, routing = case.run_gpu()
    cnt = routing["expert_counts"].cpu().numpy()
    assert (cnt[[0, 5, 17, 63]] == 0).all()


def test_routed_scale():
    cfg = C["deepseekmoe-16b"].replace(T=400, d=256, inner=128, shared_inner=128,
                                       routed_scale=2.5)
    check_case(Case(cfg))


def test_pending_hip_error_is_not_this_calls_failure():
    """An error left pending in the thread's HIP error state by an earlier,
    unrelated runtime call (here hipSetDevice on a device that does not exist,
    which fails without touching the GPU) must not make the next forward or
    backward report a failed launch; the results equal a clean call's."""
    import ctypes
    import mixture_experts_layer_mk_amd as moe
    hip = ctypes.CDLL("libamdhip64.so")
    cfg = C["deepseekmoe-16b"].replace(T=300, d=256, inner=128, shared_inner=128, seed=7)
    case = Case(cfg)
    d = case.dev
    ref = moe.moe_layer_forward(d["x"], d["w_gate"], d["routed"], d["shared"], cfg.top_k)
    dout = torch.ones_like(d["x"])
    gref = moe.moe_layer_backward(d["x"], d["w_gate"], d["routed"], d["shared"], cfg.top_k,
                                  dout)
    torch.cuda.synchronize()
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0      # leaves an error pending
    out = moe.moe_layer_forward(d["x"], d["w_gate"], d["routed"], d["shared"], cfg.top_k)
    assert hip.hipSetDevice(ctypes.c_int(1 << 20)) != 0
    g = moe.moe_layer_backward(d["x"], d["w_gate"], d["routed"], d["shared"], cfg.top_k, dout)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    assert torch.equal(g["dx"], gref["dx"])
    assert torch.equal(g["routed"][0], gref["routed"][0])
