"""Float64 CPU oracle (test infrastructure only; see qmm_oracle's header)."""
from .qmm_oracle import *  # noqa: F401,F403
from .qmm_oracle import (FMT_F16, FMT_Q4_0, FMT_Q4_1, FMT_Q5_0, FMT_Q5_1, FMT_Q8_0,  # noqa: F401
                         brute_force_matmul, dequant, dequant_rows, expand_f16_ref, fp16_round,
                         gate_up_silu_ref, get_rows_ref, matmul_add_ref, matmul_ref, pack_q4_0,
                         pack_q4_1, pack_q5_0, pack_q5_1, pack_q8_0, rmsnorm_gate_up_silu_ref,
                         rmsnorm_matmul_ref, rmsnorm_ref, row_bytes, silu, tol_linear, tol_residual,
                         tol_swiglu, unpack_f16, unpack_q4_0, unpack_q4_1, unpack_q5_0, unpack_q5_1,
                         unpack_q8_0)
