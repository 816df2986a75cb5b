"""GPU parity of every kernel instantiation the library dispatches to.

The long-context tests exercise the benchmark shapes; these small cases run
each GQA variant (group size x head width x storage type x layout) and each
latent head count once against the float64 oracle, with a ragged batch of
two sequences, NaN padding past each end, a NaN-filled workspace, and both
the heuristic plan and an explicit split count whose chunk is not a multiple
of any tile.
"""

import itertools

import pytest

import synthetic
from harness import assert_parity, oracle_out, run_gpu, run_gpu_fused

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import split_kv_flash_amd.binding as B

    B.lib()  # fail loudly if the HIP library is missing


GROUPS = [1, 2, 4, 6, 8]
WIDTHS = [64, 128, 256]
STORAGE = ["f32", "f16", "bf16"]
LAYOUTS = ["contiguous", "paged"]


@pytest.mark.parametrize("G,D,kv,layout", list(itertools.product(GROUPS, WIDTHS, STORAGE, LAYOUTS)))
def test_every_gqa_variant_matches_oracle(G, D, kv, layout):
    # q storage cycles through the three types so each appears with every group size.
    q_dtype = STORAGE[(G + D // 64) % 3]
    seed = 6000 + G * 100 + D + STORAGE.index(kv) * 7 + LAYOUTS.index(layout)
    case = synthetic.gqa_case(
        f"variant-G{G}-D{D}-{kv}-{layout}", seq_lens=[1000, 77], num_q_heads=2 * G, num_kv_heads=2,
        head_dim=D, q_dtype=q_dtype, kv_dtype=kv, layout=layout, capacity=1040, seed=seed)
    ref, _ = oracle_out(case)
    for S in (0, 7):
        out, _, call = run_gpu(case, n_splits=S)
        assert_parity(case, out, ref, label=f"G={G} D={D} {kv} {layout} q={q_dtype} plan={call.plan}")


@pytest.mark.parametrize("kv", ["f32", "f16", "bf16"])
def test_long_slice_variant_of_the_four_head_layer(kv):
    """Slices of 2,048 positions or more take the 4-head width-256 kernel with
    four rows per tile (64-row tiles): explicit plans put the tile boundary,
    the slice boundary and the sequence end at awkward places."""
    case = synthetic.gqa_case(f"long-slices-{kv}", seq_lens=[9000, 4097, 2049], num_q_heads=16,
                              num_kv_heads=4, head_dim=256, kv_dtype=kv, capacity=9010,
                              seed=6600 + len(kv))
    ref, _ = oracle_out(case)
    for S in (1, 2, 4):  # chunk 9000, 4500, 2250: every one at least 2,048
        out, _, call = run_gpu(case, n_splits=S)
        assert call.plan.chunk >= 2048
        assert_parity(case, out, ref, label=f"long slices {kv} plan={call.plan}")
        out1, _, _ = run_gpu_fused(case, call=call)
        assert_parity(case, out1, ref, label=f"long slices, one launch {kv} plan={call.plan}")


@pytest.mark.parametrize("kv", ["f32", "f16"])
@pytest.mark.parametrize("hq", [32, 64, 128])
def test_latent_head_counts(kv, hq):
    """32, 64 and 128 heads take other kernel variants than the 96-head layer
    (f32: two 16-head blocks per workgroup and 1, 2 or 4 workgroups per split;
    f16: 2 or 4 blocks per workgroup, and two workgroups per split at 128,
    whose 4-block workgroups split a tile's 36 wave-loads unevenly))."""
    # S = 130: more than 128 (split, sequence) pairs, so 64 and 96 f16 heads
    # stay in one workgroup per split; the short plans split them in two.
    for L, S in ((1000, 0), (33, 2), (4097, 5), (4097, 130)):
        case = synthetic.latent_case(f"latent{hq}-{kv}-L{L}", seq_len=L, kv_dtype=kv,
                                     num_q_heads=hq, capacity=L + 9, seed=7000 + hq + L,
                                     scale=1.0 / 24.0)  # NaN rows past the end
        out, _, call = run_gpu(case, n_splits=S)
        ref, _ = oracle_out(case)
        assert_parity(case, out, ref, tight=(kv == "f32"), label=f"latent hq={hq} {kv} L={L} plan={call.plan}")
