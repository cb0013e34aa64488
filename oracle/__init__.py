"""CPU oracle for the capacity-padded, permute-free MoE FFN forward.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  This package is the plain, slow,
obviously-correct definition that the HIP path is checked against.  Only the
test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it; the library under ``mixture_experts_expert_amd``
never does, and the two share no code.

Pages followed (cited by title and section):

* [FC] "feat(cuda-graphs): capture fixed-capacity MoE execution"
  (NVIDIA-NeMo Automodel pull request 2932), section "Design notes":
  source capacity and per-expert drop-and-pad selection.
* [PF] "Permute-Free Grouped GEMM for MoE (bf16, gfx950)"
  (ROCm TransformerEngine pull request 694), sections 1-6: the route list,
  the sync-free align, gather-in-GEMM FC1 -> SwiGLU -> FC2 and the
  gather-combine.

Parity status per function is listed in the module docstrings of
``oracle.moe`` (forward) and ``oracle.backward`` (backward).
"""

from .moe import (  # noqa: F401
    BM_DEFAULT,
    align,
    bf16_bits_to_f64,
    capacity_select,
    dense_forward,
    dropless_align,
    dropless_bound,
    dropless_forward,
    expert_ffn,
    f32_to_bf16_bits,
    f64_to_bf16_bits,
    forward,
    gather_combine,
    grouped_ffn,
    grouped_ffn_blocks,
    padded_capacity,
    dispatch_rows,
    permuted_forward,
    route_topk,
    source_capacity,
)
from .backward import (  # noqa: F401
    backward,
    expert_backward,
    fc1_dgrad,
    fc1_preact,
    fc1_preact_slots,
    fc1_wgrad,
    fc1_wgrad_sum,
    fc2_dgrad,
    fc2_wgrad,
    fc2_wgrad_sum,
    grouped_ffn_backward,
    main_grad_accumulate,
    route_backward,
    swiglu_backward,
)
