"""The launch configuration bench.py times, checked against the oracle: the workload's
shapes tuned on this GPU, the stem's first two convs as one pair kernel and its third
fused with the max pool, every layer recorded
once into the library's stack graph and replayed. The replays must agree bit for bit
with each other, and the last map with the oracle chain end to end."""
import numpy as np
import pytest
import torch

import workloads as wl
from parity import gate, to64
from test_gpu_conv import oracle_chain

pytestmark = pytest.mark.gpu

c2d = pytest.importorskip("conv2d_bias_activation_amd")
bench = pytest.importorskip("bench")
DEV = torch.device("cuda")


@pytest.mark.parametrize("key,builder,workspace", [("resnet", wl.conv5_resnet18d, True),
                                                   ("resnet", wl.conv5_resnet18d, False),
                                                   ("ifnet", wl.conv4_ifnet_block, True),
                                                   ("ifnet", wl.conv4_ifnet_block, False)])
def test_tuned_stack_graph_end_to_end(key, builder, workspace):
    """workspace False: the stack recorded without a workspace, so every op takes a variant
    that needs none (channel-first convs on the general kernel, no split-K)."""
    work = builder()
    c2d.tune_clear()
    try:
        tuned = bench.tune_workload(work)
        assert tuned >= 1
        net = bench.Net(work, DEV, fuse_pool=True, weights_ohwi=workspace, workspace=workspace)
        names = [L["plan"] for L in net.layers]
        if key == "ifnet":
            # channel-first convs: channel-last copies in the workspace, else the general kernel
            assert all(n.startswith("x_to_nhwc+" if workspace else "igemm_nchw") for n in names), names
        if not workspace:
            assert all("splitk=" not in n or "splitk=1" in n for n in names), names
        if key == "resnet":
            # the stem's first two convs run as one pair kernel (the first output never stored)
            assert "stem3x3+halo3x3_pair" in names[0], names
        g = c2d.StackGraph(net.ops(), layout=work.layout,
                           dtype={"bf16": c2d.DTYPE_BF16, "f16": c2d.DTYPE_F16}[work.dtype],
                           workspace=None if workspace else False)
        if key == "ifnet" and workspace:
            assert g.workspace is not None and g.workspace.numel() >= 2 * 68 * 120 * 240 * 2
        out = net.t[net.out_name]
        outs = []
        for _ in range(3):
            out.zero_()
            g.launch()
            torch.cuda.synchronize()
            outs.append(out.clone())
        g.close()
    finally:
        c2d.tune_clear()
    assert all(torch.equal(outs[0], o) for o in outs[1:]), "graph replays differ"
    _, ref = oracle_chain(key, work)
    gate(to64(outs[0]), ref[work.layers[-1].out], work.dtype, what=f"{key} tuned stack graph", elementwise=False)
