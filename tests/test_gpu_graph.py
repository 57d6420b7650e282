"""HIP graph replay of the MX linear step (dual packs + fwd/dgrad/wgrad
GEMMs, captured through the C ABI on torch's capture stream): every replay,
with eager work and synchronizations in between, must reproduce the eager
results bit for bit."""
import numpy as np
import pytest
import torch

from microscaling_block_scaled_mx_amd import inputs as I

pytestmark = pytest.mark.gpu


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


@pytest.mark.parametrize("fmt,mode,had", [(2, 0, True), (1, 0, False), (3, 1, False)])
def test_linear_step_graph_replays_match_eager(fmt, mode, had):
    from microscaling_block_scaled_mx_amd import mx
    assert torch.cuda.is_available() and mx.device_supported(0)
    M, N, K = 512, 256, 768
    X, W, dY = I.linear(11 + fmt, M, N, K)
    Xd, Wd, dYd = dev(X), dev(W), dev(dY)
    P = lambda r, k: mx.alloc_packed(r, k, fmt)
    Xr, Xc, Wr, Wc, dYr, dYc = P(M, K), P(K, M), P(N, K), P(K, N), P(M, N), P(N, M)
    e16 = lambda *s: torch.zeros(s, dtype=torch.int16, device="cuda")
    Y, dX, dW = e16(M, N), e16(M, K), e16(N, K)
    outs = [Xr[0], Xr[1], Xc[0], Xc[1], Wr[0], Wc[0], dYr[0], dYc[0], Y, dX, dW]

    def step():
        mx.quantize(Xd, M, K, fmt, mode, had, row=Xr, col=Xc)
        mx.quantize(Wd, N, K, fmt, mode, had, row=Wr, col=Wc)
        mx.quantize(dYd, M, N, fmt, mode, had, row=dYr, col=dYc)
        mx.gemm(Xr, Wr, M, N, K, fmt, Y)
        mx.gemm(dYr, Wc, M, K, N, fmt, dX)
        mx.gemm(dYc, Xc, N, K, M, fmt, dW)

    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for o in outs:
            o.fill_(0x55 if o.dtype == torch.uint8 else 0x5555)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(o, w), f"replay {rep}: output {i} differs from the eager step"
