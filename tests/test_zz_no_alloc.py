"""moe_forward_noalloc, the forward without a workspace argument (a static
8 MiB device array instead), against moe_forward with a caller workspace.

Two calls in a row, the second with a smaller batch (so the second reads an
array the first has filled): the bf16 layer at 500 then 37 tokens, and the
int4 top-1 serving path at 64 then 5 tokens.  Routing must be bit-exact and
y within the layer's bf16 tolerance of moe_forward's (whole tensor 1e-2,
every token row 3e-2; the kernels are the same, so the bits match too).  A
batch whose workspace does not fit the array is refused."""
import numpy as np
import pytest

import oracle.moe_oracle as om
from fine_grained_moe_amd import synth
from tests import _helpers as H

pytestmark = pytest.mark.gpu


def _compare(dims, x, w, bias):
    import torch
    from fine_grained_moe_amd import moe
    y_ref = torch.empty_like(x)
    r_ref = moe.alloc_routing(dims)
    moe.moe_forward(dims, x, w, bias, y_ref, r_ref, moe.alloc_workspace(dims))
    y = torch.full_like(x, float("nan"))
    r = moe.alloc_routing(dims)
    for t in r.values():
        t.fill_(-7)
    moe.moe_forward_noalloc(dims, x, w, bias, y, r)
    torch.cuda.synchronize()
    for n in r:
        assert torch.equal(r[n], r_ref[n]), n
    H.check_close(y.float().cpu().numpy(), y_ref.float().cpu().numpy(), "bf16", f"noalloc T={dims.T} y:")
    assert torch.equal(y, y_ref)


def test_bf16_layer_two_calls_second_smaller():
    import torch
    from fine_grained_moe_amd import moe
    for T, seed in ((500, 71), (37, 72)):
        inp = synth.make_workload("layer_t4096", T=T, seed=seed)
        H.remove_near_ties(inp)
        x, w = H.to_gpu(inp)
        dims = moe.make_dims(T, inp.d, inp.E, inp.F, inp.Fs, inp.k, "bf16")
        assert moe.moe_workspace_bytes(dims) <= moe.MOE_NOALLOC_SCRATCH_BYTES
        _compare(dims, x, w, torch.from_numpy(inp.bias).cuda())


def test_int4_decode_two_calls_second_smaller():
    import torch
    from fine_grained_moe_amd import moe
    base = synth.make_layer(T=1, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", seed=73)
    qg, sg = om.quantize_int4(base.w_gate_up)
    qd, sd = om.quantize_int4(base.w_down)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device="cuda", dtype=torch.bfloat16)
    w = dict(w_router=bf(base.w_router), w_gate_up=torch.from_numpy(qg).cuda(), s_gate_up=bf(sg),
             w_down=torch.from_numpy(qd).cuda(), s_down=bf(sd), w_sh_gate_up=bf(base.w_sh_gate_up),
             w_sh_down=bf(base.w_sh_down))
    for T, seed in ((64, 74), (5, 75)):
        inp = synth.make_layer(T=T, d=1024, E=64, F=512, Fs=2048, k=1, act="bf16", seed=seed)
        inp.w_router = base.w_router
        H.remove_near_ties(inp, bias_states=[np.zeros(64, np.float32)])
        dims = moe.make_dims(T, 1024, 64, 512, 2048, 1, "bf16", w_routed="int4")
        _compare(dims, bf(inp.x), w, torch.zeros(64, device="cuda"))


def test_too_large_is_refused():
    import torch
    from fine_grained_moe_amd import moe
    dims = moe.make_dims(4096, 1024, 64, 512, 2048, 2, "bf16")
    assert moe.moe_workspace_bytes(dims) > moe.MOE_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(4096, 1024, dtype=torch.bfloat16, device="cuda")
    inp = synth.make_workload("layer_t4096", T=1)
    _, w = H.to_gpu(inp)
    r = moe.alloc_routing(dims)
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(dims, x, w, torch.zeros(64, device="cuda"), torch.empty_like(x), r)
    assert ei.value.code == moe.MOE_E_WORKSPACE


def test_captured_in_a_graph_replays_exactly():
    """The allocation-free forward is for callers under HIP graph capture:
    captured once for the bf16 layer (300 tokens), every replay gives
    exactly the eager moe_forward result, with other eager calls of the
    entry point on another batch (sharing the static array) and host
    synchronisations between the replays."""
    import torch
    from fine_grained_moe_amd import moe
    inp = synth.make_workload("layer_t4096", T=300, seed=76)
    H.remove_near_ties(inp)
    x, w = H.to_gpu(inp)
    dims = moe.make_dims(300, inp.d, inp.E, inp.F, inp.Fs, inp.k, "bf16")
    bias = torch.from_numpy(inp.bias).cuda()
    y_ref, r_ref = torch.empty_like(x), moe.alloc_routing(dims)
    moe.moe_forward(dims, x, w, bias, y_ref, r_ref, moe.alloc_workspace(dims))
    other = synth.make_workload("layer_t4096", T=77, seed=77)
    xo, _ = H.to_gpu(other)
    dims_o = moe.make_dims(77, inp.d, inp.E, inp.F, inp.Fs, inp.k, "bf16")
    y, r = torch.empty_like(x), moe.alloc_routing(dims)
    # an eager call first: the entry point takes its array's device address
    # on its first call on a device, outside the capture
    moe.moe_forward_noalloc(dims_o, xo, w, bias, torch.empty_like(xo), moe.alloc_routing(dims_o))
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        moe.moe_forward_noalloc(dims, x, w, bias, y, r, stream=s)
    for rep in range(3):
        y.fill_(float("nan"))
        for t in r.values():
            t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), rep
        for n in r:
            assert torch.equal(r[n], r_ref[n]), (rep, n)
        moe.moe_forward_noalloc(dims_o, xo, w, bias, torch.empty_like(xo), moe.alloc_routing(dims_o))
        torch.cuda.synchronize()
