"""CPU oracle for the Prox sparse SwiGLU FFN — test infrastructure only.

Only the tests, the package smoke check and the bench's CPU-baseline leg may
import this package; the product path never does."""

from .prox_oracle import (  # noqa: F401
    INT4_GROUP, Proxy, ForwardResult, TokenResult, bf16_bits_to_f64, build_proxy, dense_ffn,
    mask_diff, oracle_forward, oracle_stage2, quantize_int4_g128, quantize_int8_pc, select_topk,
    silu, stage1_batch, stage1_token, stage2_batch, stage2_token, mask_overlap, rel_l2_error,
    QWeights, build_qweights, oracle_forward_q8, quantize_rows_int8,
)
