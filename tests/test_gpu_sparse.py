"""GPU parity of sparse (index-list) decode against the float64 oracle.

Layout SK_KV_INDEXED: position j of sequence b reads pool row indices[b][j]
("The Kernel Level: Attention and MoE", sparsity: the sparse decode kernel
gathers the top-k tokens from the KV pool by index). Separate K and V run the
GQA split kernel with pages of one row; a shared latent runs the latent
kernels with index-list tiles. Pools hold more rows than any list names, so a
kernel that ignores the list reads the wrong rows; -1 entries past each list
are never read.
"""

import itertools

import numpy as np
import pytest

import synthetic
from harness import (ABS_GATE, assert_parity, decode_call, oracle_out, run_gpu, run_gpu_fused)
from synthetic.torch_io import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import split_kv_flash_amd.binding as B

    B.lib()  # fail loudly if the HIP library is missing


def free():
    import torch

    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("G,D,kv", list(itertools.product([1, 4, 6, 8], [64, 128, 256],
                                                          ["f32", "f16", "bf16"])))
def test_gqa_index_list_matches_oracle(G, D, kv):
    q_dtype = ["f32", "f16", "bf16"][(G + D // 64) % 3]
    case = synthetic.indexed_case(f"sparse-G{G}-D{D}-{kv}", pool_rows=3000, seq_lens=[1000, 77, 1],
                                  num_q_heads=2 * G, num_kv_heads=2, head_dim=D, kv_dtype=kv,
                                  q_dtype=q_dtype, max_indices=1040, seed=9500 + G * 10 + D)
    ref, rlse = oracle_out(case)
    for S in (0, 7):
        out, lse, call = run_gpu(case, n_splits=S)
        assert_parity(case, out, ref, label=f"G={G} D={D} {kv} plan={call.plan}")
        np.testing.assert_allclose(lse, rlse, rtol=0, atol=1e-4)
    out, _, _ = run_gpu_fused(case)
    assert_parity(case, out, ref, label=f"G={G} D={D} {kv} one launch")


def test_gqa_top_2048_of_a_131072_row_cache():
    """A 9B-like layer (16/4 heads, head_dim 256, f16) attending 2048 rows
    chosen from 131,072."""
    case = synthetic.indexed_case("sparse-9b", pool_rows=131072, seq_lens=[2048],
                                  num_q_heads=16, num_kv_heads=4, head_dim=256, kv_dtype="f16",
                                  seed=9601)
    out, _, call = run_gpu(case)
    ref, _ = oracle_out(case)
    assert_parity(case, out, ref, label=f"9B-like sparse plan={call.plan}")
    free()


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_dsa_latent_top_2048(kv):
    """96 heads over a 576-column latent, top-2048 of 131,072 rows, with the
    heuristic plan; then the same list in another order."""
    case = synthetic.dsa_latent(topk=2048, pool_rows=131072, kv_dtype=kv, seed=9700)
    t = to_device(case)
    out, lse, call = run_gpu(case, tensors=t)
    ref, rlse = oracle_out(case)
    assert_parity(case, out, ref, tight=(kv == "f32"), label=f"dsa {kv} plan={call.plan}")
    np.testing.assert_allclose(lse, rlse, rtol=0, atol=ABS_GATE[kv])
    import torch

    perm = np.random.default_rng(3).permutation(2048)
    t["block_table"][0, :2048] = t["block_table"][0, :2048][torch.from_numpy(perm).cuda()]
    out2, _, _ = run_gpu(case, tensors=t)
    assert np.abs(out2 - out).max() <= ABS_GATE[kv] / 2
    del call, t
    free()


@pytest.mark.parametrize("kv,hq", [("f32", 32), ("f32", 64), ("f32", 96), ("f32", 128), ("f16", 32),
                                   ("f16", 64), ("f16", 96), ("f16", 128)])
def test_latent_index_list_head_counts(kv, hq):
    """Every head count over index lists; S = 130 takes the whole-head
    kernels (more than 128 (split, sequence) pairs), the others the split
    head groups."""
    for L, S in ((1000, 0), (33, 2), (1, 1), (4097, 5), (4097, 130)):
        case = synthetic.indexed_case(f"lat-idx-{kv}-{hq}-{L}", pool_rows=L + 2000, seq_lens=[L],
                                      num_q_heads=hq, num_kv_heads=1, head_dim=576, kv_dtype=kv,
                                      latent_value_dim=512, max_indices=L + 9, seed=9800 + hq + L,
                                      scale=1 / 24)
        out, _, call = run_gpu(case, n_splits=S)
        ref, _ = oracle_out(case)
        assert_parity(case, out, ref, tight=(kv == "f32"), label=f"{kv} hq={hq} L={L} plan={call.plan}")


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_in_order_list_of_the_whole_cache_equals_the_contiguous_path(kv):
    """indices = 0..L-1 over the cache rows: the index-list kernels read the
    same rows into the same tiles, so the partials are the same bits."""
    import torch

    L = 3000
    case = synthetic.latent_decode(L, kv, seed=9900)
    t = to_device(case)
    _, _, call = run_gpu(case, n_splits=5, tensors=t)
    want = [x.clone() for x in call.partials()]
    pool = t["k"][0]  # [L][1][576]
    table = torch.arange(L, dtype=torch.int32, device="cuda").view(1, L)
    from split_kv_flash_amd import DecodeCall

    ic = DecodeCall(t["q"], pool, None, t["seq_lens"], case.seq_lens, scale=case.scale,
                    block_table=table, v_cols=512, n_splits=5)
    ic.workspace.fill_(0xFF)
    ic()
    torch.cuda.synchronize()
    for a, b in zip(want, ic.partials()):
        assert torch.equal(a, b)
    assert torch.equal(call.out, ic.out)


def test_out_of_range_indices_poison_only_their_sequence():
    import torch

    case = synthetic.indexed_case("bad-idx", pool_rows=500, seq_lens=[300, 200, 100],
                                  num_q_heads=8, num_kv_heads=2, head_dim=128, kv_dtype="bf16",
                                  seed=9901)
    t = to_device(case)
    call = decode_call(case, t, n_splits=3)
    t["block_table"][1, 150] = 500  # one past the pool
    t["block_table"][2, 0] = -1
    out, _, _ = run_gpu(case, tensors=t, call=call)
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(out[2]))
    ref, _ = oracle_out(case)
    assert np.abs(out[0] - ref[0]).max() <= ABS_GATE["bf16"]


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_latent_out_of_range_index_gives_nan(kv):
    case = synthetic.indexed_case("bad-lat", pool_rows=3000, seq_lens=[2048], num_q_heads=96,
                                  num_kv_heads=1, head_dim=576, kv_dtype=kv,
                                  latent_value_dim=512, seed=9902, scale=1 / 24)
    t = to_device(case)
    t["block_table"][0, 1500] = 3000
    out, _, _ = run_gpu(case, tensors=t)
    assert np.all(np.isnan(out[0]))
    t["block_table"][0, 1500] = int(case.block_table[0, 1500])
    out, _, _ = run_gpu(case, tensors=t)
    ref, _ = oracle_out(case)
    assert_parity(case, out, ref, tight=(kv == "f32"))
