"""CPU oracle for the denoise step, the entropy-bounded commit and the slot read.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
bench's CPU-baseline leg may import or call this package.  The HIP library
never calls it and shares no code with it.
"""
from .dg_oracle import (  # noqa: F401
    embed_input, qkv_project, prefill_kv, causal_attention, encode_prompt, window_attention,
    block_output, lm_logits,
    vocab_softmax, self_condition, denoise_canvas, denoise_step, commit_canvas,
    commit, denoise_loop, label_read, slot_read_canvas, slot_read, slot_read_staged, NearTies, argmax_near_ties,
    commit_near_ties, best_near_ties, SLOT_OK, SLOT_BAD_POS, SLOT_BAD_COUNT,
    SLOT_BAD_LABEL, SLOT_BAD_NOISE, SLOT_NOT_ASKED, MAX_LABELS, E4M3_MAX, e4m3_row_exponent, e4m3_encode,
    e4m3_decode, quantize_rows_e4m3, quantize_head_e4m3, dequantize_head_e4m3, fp8_activations,
)
