"""Helpers shared by the GPU tests: run a synthetic case through the C ABI and
compare with the float64 oracle."""

from __future__ import annotations

import math

import numpy as np

import oracle
from synthetic.torch_io import to_device

# Gates: max |gpu - oracle| (spec tolerance by KV storage type), and a
# relative L2 bound that keeps the test powerful when outputs are small
# (at L = 262,144 outputs are ~3e-3, so 2e-3 absolute alone would be weak).
ABS_GATE = {"f32": 1e-4, "f16": 2e-3, "bf16": 2e-3}
REL_L2_GATE = {"f32": 1e-5, "f16": 1e-3, "bf16": 1e-3}
# Every GQA kernel computes in f32 from the exact stored values, so its error
# is f32 rounding only; this tighter bound catches slips the gates would miss.
REL_L2_F32_ARITH = 2e-5
# lse of a path whose arithmetic is f32 (q and the weights used exactly, or in
# 16-bit parts that together carry 22-24 bits): the f32 gate.
LSE_F32_ARITH = 1e-4


def decode_call(case, tensors, *, n_splits: int = 0, cu_count=None):
    from split_kv_flash_amd import DecodeCall

    return DecodeCall(
        tensors["q"], tensors["k"], tensors["v"], tensors["seq_lens"], case.seq_lens,
        scale=case.scale, block_table=tensors["block_table"], page_size=case.page_size,
        v_cols=case.head_dim_v if case.kv_shared else None, n_splits=n_splits, cu_count=cu_count)


def run_gpu(case, *, n_splits: int = 0, tensors=None, call=None):
    """Run split + combine with a NaN-filled workspace; returns (out, lse, call)."""
    import torch

    if tensors is None:
        tensors = to_device(case)
    if call is None:
        call = decode_call(case, tensors, n_splits=n_splits)
    call.workspace.view(torch.uint8).fill_(0xFF)  # all-ones bytes: NaN in every f32 slot
    call.out.fill_(float("nan"))
    call.lse.fill_(float("nan"))
    call()
    torch.cuda.synchronize()
    return call.out.double().cpu().numpy(), call.lse.double().cpu().numpy(), call


def oracle_out(case, heads=None):
    return oracle.attend_f64(case.q, case.k_rows(), case.v_rows(), case.seq_lens, case.scale,
                             q_dtype=case.q_dtype, kv_dtype=case.kv_dtype,
                             v_cols=case.head_dim_v if case.kv_shared else None, heads=heads)


def errors(got, ref):
    """(max abs, relative L2, cosine) over the entries ref defines (non-NaN)."""
    mask = ~np.isnan(ref)
    g, r = got[mask], ref[mask]
    d = g - r
    rel = math.sqrt(float((d * d).sum()) / max(float((r * r).sum()), 1e-300))
    cos = float((g * r).sum()) / max(math.sqrt(float((g * g).sum()) * float((r * r).sum())), 1e-300)
    return float(np.abs(d).max()), rel, cos


def assert_parity(case, got, ref, *, tight: bool = True, label: str = ""):
    assert np.all(np.isfinite(got[~np.isnan(ref)])), f"{label}: non-finite output"
    ea, er, _ = errors(got, ref)
    gate_a, gate_r = ABS_GATE[case.kv_dtype], REL_L2_GATE[case.kv_dtype]
    assert ea <= gate_a, f"{label}: max abs err {ea:.3e} > {gate_a:.1e}"
    assert er <= gate_r, f"{label}: relL2 {er:.3e} > {gate_r:.1e}"
    if tight:
        assert er <= REL_L2_F32_ARITH, f"{label}: relL2 {er:.3e} > {REL_L2_F32_ARITH:.1e} (f32 arithmetic)"
    return ea, er


def run_gpu_fused(case, *, n_splits: int = 0, tensors=None, call=None):
    """Run the one-launch decode (attn_decode_one_launch) with a poisoned workspace: every
    byte 0xFF (NaN partials), then the completion counters zeroed as the
    header requires. Returns (out, lse, call); the counters must be back at
    zero afterwards."""
    import torch

    if tensors is None:
        tensors = to_device(case)
    if call is None:
        call = decode_call(case, tensors, n_splits=n_splits)
    call.workspace.view(torch.uint8).fill_(0xFF)
    call.init_workspace()
    call.out.fill_(float("nan"))
    call.lse.fill_(float("nan"))
    call.decode_one_launch()
    torch.cuda.synchronize()
    assert int(call.counters().abs().sum().item()) == 0, "completion counters not reset"
    return call.out.double().cpu().numpy(), call.lse.double().cpu().numpy(), call
