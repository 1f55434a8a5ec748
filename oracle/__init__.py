"""fp64 CPU oracle of the MSA forward path.  TEST INFRASTRUCTURE: imported only
by tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg."""
from .msa_oracle import (  # noqa: F401
    BF16, FP8, MXFP4, MXFP4_QK, E4M3FN_TABLE, E2M1_TABLE, e8m0_to_f64, mxfp4_record_rows, mxfp4_q_rows,
    dequant_proxy_q, Layout, bf16_to_f64, e4m3fn_to_f64, dequant, gather_rows,
    proxy_block_maxscore, topk_select, topk_select_row, sparse_attention, sparse_attention_backward, proxy_kl_backward, sparse_decode,
    check_selection_row,
)
