"""The forward inside a captured HIP graph (torch.cuda.CUDAGraph): it
allocates nothing, records no memset and synchronises nothing, so a serving
loop can capture it once and replay it.  Each replay is compared bitwise
with the eager result (the kernels are deterministic), with eager work and a
device synchronisation between the replays, and a replay after the inputs
change in place must give the new inputs' result."""
import pytest
import torch

from blocked_local_self_amd import halo_attn_fwd, _native
from blocked_local_self_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

SHAPES = [
    # (B, heads, H, W, d, block, halo, stride, dtype)
    (2, 3, 24, 24, 16, 8, 3, 1, "bf16"),     # 32-query groups of the ring kernel
    (1, 2, 36, 36, 32, 12, 3, 1, "bf16"),    # 18x18 window: 4x4-patch tile kernel
    (2, 2, 24, 24, 16, 8, 3, 2, "bf16"),     # strided queries
    (1, 2, 64, 64, 16, 32, 3, 1, "bf16"),    # 38x38 window: streaming kernel
    (1, 2, 16, 16, 16, 4, 1, 1, "fp32"),     # generic kernel
]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _native.load()


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_forward_replays_in_a_graph(shape):
    B, heads, H, W, d, block, halo, stride, dtype = shape
    print(f"graph case {shape}", flush=True)
    dev = torch.device("cuda:0")
    q, k, v, rh, rw = (t.to(dev) for t in make_inputs(B, heads, H, W, d, block, halo, dtype=dtype, seed=11))
    q2 = make_inputs(B, heads, H, W, d, block, halo, dtype=dtype, seed=12)[0].to(dev)
    eager = halo_attn_fwd(q, k, v, rh, rw, block, halo, stride)
    eager2 = halo_attn_fwd(q2, k, v, rh, rw, block, halo, stride)
    torch.cuda.synchronize()

    out = torch.empty_like(eager)
    qin = q.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        halo_attn_fwd(qin, k, v, rh, rw, block, halo, stride, out=out)
    for _ in range(3):
        out.fill_(float("nan"))                 # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
    qin.copy_(q2)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out, eager2)


BWD_SHAPES = [
    (2, 3, 24, 24, 16, 8, 3, 1),     # column-walk (strip) backward
    (1, 2, 36, 36, 32, 12, 3, 1),    # 16-query tile backward (18x18 window)
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_backward_replays_in_a_graph(shape):
    # with the workspace and the gradients passed in, the backward allocates
    # nothing either; its sums run in a fixed order, so replays are bitwise
    from blocked_local_self_amd import halo_attn_bwd, bwd_workspace_bytes
    from blocked_local_self_amd.inputs import make_grad_output
    B, heads, H, W, d, block, halo, stride = shape
    print(f"graph backward case {shape}", flush=True)
    dev = torch.device("cuda:0")
    q, k, v, rh, rw = (t.to(dev) for t in make_inputs(B, heads, H, W, d, block, halo, dtype="bf16", seed=13))
    g = make_grad_output(B, heads, H // stride, W // stride, d, dtype="bf16", seed=14).to(dev)
    out, lse = halo_attn_fwd(q, k, v, rh, rw, block, halo, stride, return_lse=True)
    need = bwd_workspace_bytes(B, heads, H, W, d, block, halo, stride, "bf16")
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    eager = halo_attn_bwd(q, k, v, rh, rw, g, block, halo, stride, out=out, lse=lse, workspace=ws)
    eager = tuple(t.clone() for t in eager)
    torch.cuda.synchronize()

    grads = tuple(torch.empty_like(t) for t in eager)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        halo_attn_bwd(q, k, v, rh, rw, g, block, halo, stride, out=out, lse=lse, workspace=ws, grads=grads)
    for _ in range(3):
        for t in grads:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(grads, eager):
            assert torch.equal(got, want)


@pytest.mark.parametrize("kernel", ["split", "fused"])
def test_layer_replays_in_a_graph(kernel):
    # the whole layer (projections, attention, to_out) with its workspace
    # passed in: the split path's three kernels, or the one-kernel path
    from blocked_local_self_amd import halo_layer_fwd, layer_workspace_bytes
    from blocked_local_self_amd.inputs import make_layer_inputs
    B, H, W, heads, d, block, halo = 2, 32, 32, 4, 16, 8, 3
    C = heads * d
    print(f"graph layer case {kernel}", flush=True)
    dev = torch.device("cuda:0")
    x, w_q, w_kv, w_o, b_o, rh, rw = (t.to(dev) for t in make_layer_inputs(B, H, W, C, heads, d, block, halo,
                                                                          dtype="bf16", seed=15))
    ws = torch.empty(max(layer_workspace_bytes(B, H, W, heads, d), 16), dtype=torch.uint8, device=dev)
    eager = halo_layer_fwd(x, w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads, workspace=ws, kernel=kernel)
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        halo_layer_fwd(x, w_q, w_kv, w_o, b_o, rh, rw, block, halo, heads, workspace=ws, out=out, kernel=kernel)
    for _ in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
