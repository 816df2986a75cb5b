"""Float64 CPU oracle for split-KV ("flash-decoding") decode attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it. It
shares no code with the HIP library and never imports it.

Pages this oracle follows (cited by the short key in brackets):

* [L06]  "Part 4 · Lecture 06 — Attention at 128k: Split Over Context, Split
  Over Heads" (jared-hpc AI inference engineer roadmap).
* [I3725] aprender issue #3725, "Qwen3.5 CUDA long-context DECODE is slow: the
  decode attention kernel runs 16 blocks — split-K needed ...", design note.
* [DB6]  "Decoder Block 6: Online Attention, the Capstone" (gpuflight lesson).
* [L07]  "The Kernel Level: Attention and MoE" (llm-serving.xyz, Lecture 07).

Every function here is pinned by a CPU test against something other than
itself (brute force with exact summation, a library routine, closed forms,
invariants, the worked merge example of [L07]); see ``tests/test_oracle.py``.
No function is "parity unpinned".
"""

from .attention import (  # noqa: F401
    attend_f64,
    attend_multiquery_f64,
    causal_limits,
    bf16_bits_to_f64,
    gather_indexed,
    gather_paged,
    merge_partials_f64,
    merge_partials_lse_f64,
    online_partial_f64,
    plan_splits,
    project_heads_f64,
    project_per_slice_f64,
    query_tile_twin_f64,
    split_partials_f64,
    split_ranges,
    split_twin_f64,
    widen,
)
