"""The entry points under HIP graph capture (torch.cuda.graph on the current stream).

Every call only enqueues kernels on its stream -- no allocation inside the library, no
device-to-host copy, no memset (the dynamic schedule's claim counters are zeroed by a
kernel of their own) -- so a captured call replays the same work.  Each case runs once
eagerly, is captured, then replayed several times with other device work and host
synchronisations in between and the output refilled with NaN before each replay; every
replay must reproduce the eager output bit for bit.  The cases cover one launch (static
schedule), the dynamic schedule (reset kernel + GEMM), split-K (GEMM + reduction), the
exact fp8 product and the entry point without a workspace argument.
"""
import pytest
import torch

import grouped_gemm_expert_offsets_amd as kgw
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")]

DEV = "cuda"
REPLAYS = 4


def check_replays(call, out):
    """`call()` writes `out`; eager result vs every replay of the captured call."""
    out.fill_(float("nan"))
    call()
    torch.cuda.synchronize()
    eager = out.clone()
    assert not torch.isnan(eager).any()
    # warm-up on a side stream, as torch's capture recipe asks
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    bits = torch.int32 if out.element_size() == 4 else torch.int16
    other = torch.randn(1 << 20, device=DEV)
    for k in range(REPLAYS):
        out.fill_(float("nan"))
        other.mul_(1.0001).add_(0.5)           # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(bits), eager.view(bits)), f"replay {k} differs from the eager call"
    del g


def bf16_case(counts, hidden, n, seed):
    return workloads.make_operands(counts, hidden, n, "bf16", torch.float32, False, seed=seed, device=DEV,
                                   std=1.0)


def test_graph_bf16_static_schedule():
    wl = bf16_case([512, 0, 768, 256], 768, 512, seed=301)
    assert kgw.kgw_workspace_bytes(4, 768, 512, wl.tokens_sum) == 0
    out = torch.empty((4, 768, 512), device=DEV)
    check_replays(lambda: kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out), out)


def test_graph_bf16_dynamic_schedule():
    # long experts, eight rounds of items: claim counters in the workspace, zeroed by a kernel
    counts = [1024 + 256 * (e % 5) for e in range(32)]
    wl = bf16_case(counts, 2048, 2048, seed=302)
    assert kgw.kgw_workspace_bytes(32, 2048, 2048, wl.tokens_sum) == 256
    out = torch.empty((32, 2048, 2048), device=DEV)
    check_replays(lambda: kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out), out)


def test_graph_bf16_split_k():
    wl = bf16_case([8192, 0, 16384], 512, 512, seed=303)
    assert kgw.kgw_workspace_bytes(3, 512, 512, wl.tokens_sum) > 256
    out = torch.empty((3, 512, 512), device=DEV)
    check_replays(lambda: kgw.kgw_wgrad_bf16(wl.A, wl.B, wl.offsets, out), out)


def test_graph_fp8_exact():
    wl = workloads.make_operands([384, 0, 1152, 256], 512, 768, "fp8", torch.bfloat16, False, seed=304, device=DEV)
    out = torch.empty((4, 512, 768), dtype=torch.bfloat16, device=DEV)
    check_replays(lambda: kgw.kgw_wgrad_fp8(wl.A, wl.sfa, wl.B, wl.sfb, wl.offsets, out), out)


def test_graph_bf16_without_workspace_argument():
    # split-K partials in the library's fixed per-device scratch
    wl = bf16_case([8192, 0, 16384], 512, 512, seed=305)
    out = torch.empty((3, 512, 512), device=DEV)
    check_replays(lambda: kgw.kgw_wgrad_bf16_noalloc(wl.A, wl.B, wl.offsets, out), out)
