"""CPU oracle for the staged tensor-parallel GEMM share -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy code in float64. Only the test suite,
the smoke check and the benchmark's CPU-baseline leg may import it; the
product path never does, and shares no code with it (the two meet only in the
seeded inputs of the `synth` package).

Sources (pages of the reference set, cited by title and section):
  * "Pytorch Op for blackwell distributed gemm" (README), Usage and
    "Note on Tensor Layouts": D = alpha * (A @ B^T) + beta * C with A (M, K),
    B (N, K) row-major, C (M, N); element type float_e4m3 (Limitations).
  * "Distributed GEMM" (Hassani et al., SHI Labs, Dec 2024), Background
    (Figures 3 and 4: pipelined stages, local shard first, buffers rotate)
    and Approach (schedules AllGather1D_TilingCD_RotatingA,
    ReduceScatter1D_TilingA_RotatingC, and their column duals
    AllGather1D_TilingCD_RotatingB, ReduceScatter1D_TilingB_RotatingC).
  * The p04 problem statement ("Project objective"): "Interface, layout,
    and parameters" and "Computation and communication example" (the
    per-token-slot FFN, LayerNorm with eps 1e-5, SiLU gate, All-to-All
    dispatch/combine and its P=2 worked example).
  * "Add dist GEMM attention and FFN backend" (torchtitan PR #4044),
    Structure: AllGatherLinear / LinearReduceScatter / AllGatherLinearMulti
    for the SwiGLU w1/w3 pair; gathered rows ordered (rank, batch, seq);
    the backward of the two linears (backward.py).

Every function is pinned by a CPU test against something other than itself
(closed forms, brute-force loops, library routines, the pages' worked
example); see tests/test_oracle_*.py.

oracle.cref binds a second, independent writing of the same definitions in
plain C++17 (oracle/cpp/oracle.cpp: float64 sums, OpenMP over output rows),
checked against this one in tests/test_oracle_cpp.py and timed as the
benchmark's CPU baseline.
"""
from .formats import decode_bf16, decode_e4m3, decode
from .gemm import (ag_stage_order, rs_block_order, gemm_ag, gemm_ag_rows, gemm_rs, gemm_rs_rows,
                   gemm_ag_rotb, gemm_ag_rotb_rows, gemm_rs_tileb, gemm_rs_tileb_rows, gemm_ag_multi)
from .ffn import layer_norm, silu, ffn_slot_forward, ffn_slot_rows, ffn_slot_backward
from .swiglu import swiglu_hidden, swiglu_hidden_rows, swiglu_block
from .permute import dispatch, combine
from .backward import wgrad, wgrad_staged, wgrad_rows
