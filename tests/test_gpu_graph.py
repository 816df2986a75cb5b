"""Graph capture of a decode call (split + combine launches, attn_decode, or
attn_decode_one_launch).

The launches allocate nothing, set no memory and never synchronise with the
host (the one-launch path's completion counters are reset by the kernel
itself; the shared latent's cooperative launch resets its barrier count the
same way), so a caller can capture them into a HIP graph and replay it every
decode step. Each replay here runs after eager work on the same stream and a
change of q, and must equal an eager call on the same inputs bit for bit.
"""

import numpy as np
import pytest

import synthetic
from harness import decode_call
from synthetic.torch_io import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import split_kv_flash_amd.binding as B

    B.lib()  # fail loudly if the HIP library is missing


CASES = {
    "gqa-f32": lambda: synthetic.qwen9b_like(4096, "f32", seed=8001),
    "gqa-bf16-paged": lambda: synthetic.gqa_case(
        "graph-paged", seq_lens=[900, 2100, 33], num_q_heads=8, num_kv_heads=2, head_dim=128,
        q_dtype="bf16", kv_dtype="bf16", layout="paged", seed=8002),
    # Contiguous 16-bit caches of wide groups or head width 64 run on the
    # query-tile kernel with one query (its one-launch form resets its
    # counters inside the kernel too).
    "qtile-f16-g6-d256": lambda: synthetic.gqa_case(
        "graph-qtile-f16", seq_lens=[3000], num_q_heads=24, num_kv_heads=4, head_dim=256,
        q_dtype="f32", kv_dtype="f16", seed=8005, peaky_fraction=0.01),
    "qtile-bf16-d64": lambda: synthetic.gqa_case(
        "graph-qtile-bf16", seq_lens=[2500, 700], num_q_heads=8, num_kv_heads=2, head_dim=64,
        q_dtype="bf16", kv_dtype="bf16", seed=8006),
    "latent-f32": lambda: synthetic.latent_case("graph-latent32", seq_len=1500, kv_dtype="f32",
                                                seed=8003, scale=1.0 / 24.0),
    "latent-f16": lambda: synthetic.latent_case("graph-latent16", seq_len=1500, kv_dtype="f16",
                                                seed=8004, scale=1.0 / 24.0),
}


@pytest.mark.parametrize("mode", ["two-launch", "whole-call", "one-launch"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_captured_call_replays_match_eager_calls(name, mode):
    import torch

    case = CASES[name]()
    t = to_device(case)
    dc = decode_call(case, t)
    if name.startswith("qtile"):
        from split_kv_flash_amd import attn_decode_kernel_info

        # The query-tile kernel stages K/V tiles in LDS (40 KB or more); the
        # vector split kernel holds at most 33 KB.
        assert attn_decode_kernel_info(dc.desc, dc.plan).lds_bytes >= 40960
    call = {"two-launch": dc, "whole-call": dc.decode, "one-launch": dc.decode_one_launch}[mode]
    q0 = t["q"].clone()
    q1 = (t["q"].float() * 0.5).to(t["q"].dtype)

    def eager(q):
        t["q"].copy_(q)
        call()
        torch.cuda.synchronize()
        return dc.out.clone(), dc.lse.clone()

    want = [eager(q0), eager(q1)]

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        call()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        call()
    torch.cuda.synchronize()

    for rep in range(3):
        q = q0 if rep % 2 == 0 else q1
        t["q"].copy_(q)
        dc.out.fill_(float("nan"))  # eager work between replays
        dc.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out, lse = want[rep % 2]
        assert torch.equal(dc.out, out), f"{name} {mode}: replay {rep} output differs"
        assert torch.equal(dc.lse, lse), f"{name} {mode}: replay {rep} lse differs"
        assert np.isfinite(dc.out.cpu().numpy()).all()
        assert int(dc.counters().abs().sum().item()) == 0
    del graph
