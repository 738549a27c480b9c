"""fp64 CPU oracle for k-MIP attention (test infrastructure only; never
imported by the GPU library)."""
from .kmip_oracle import (  # noqa: F401
    bf16_bits_to_f64, graph_ranges, scores_block, select_topk_row, softmax_selected,
    kmip_forward, attend_on_sets, query_grads, kmip_backward_on_sets,
)
