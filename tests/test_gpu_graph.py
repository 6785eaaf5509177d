"""moe_w2_forward captured in a HIP graph: every replay (with eager work and synchronisations
between replays) reproduces the eager result bit for bit, on the decode and the GEMM path."""
import numpy as np
import pytest
import torch

import bit_routed_expert_amd as moe
import workloads

from gpu_helpers import dev, dev_bf16, pack

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,path,I", [(8, moe.PATH_DECODE, 512), (100, moe.PATH_DECODE_SORTED, 512),
                                      (200, moe.PATH_GEMM, 512),
                                      (200, moe.PATH_GEMM, 2048)])   # the down GEMM streamed across tiles
def test_graph_replays_match_eager(gpu, T, path, I):
    rng = np.random.default_rng(5 + T)
    K, E, top_k = 512, 16, 4
    planes = workloads.draw_planes(rng, E, K, I)
    h = pack(planes)
    a = [(dev_bf16(workloads.draw_x(rng, T, K)),) + tuple(dev(v) for v in workloads.uniform_routing(rng, T, E, top_k))
         for _ in range(2)]
    ws = moe.alloc_workspace(h, T, top_k)
    ws_other = moe.alloc_workspace(h, T, top_k)
    y = torch.empty((T, K), dtype=torch.float32, device="cuda")
    eager = moe.moe_w2_forward(h, *a[0], out_dtype=moe.OUT_F32, workspace=ws, path=path).clone()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        moe.moe_w2_forward(h, *a[0], out_dtype=moe.OUT_F32, workspace=ws, path=path, y=y)
    for rep in range(4):
        y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), eager.view(torch.int32)), rep
        # eager work in between, on another workspace
        moe.moe_w2_forward(h, *a[1], out_dtype=moe.OUT_F32, workspace=ws_other, path=path)
        torch.cuda.synchronize()
