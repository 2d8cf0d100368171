"""MI355X (gfx950) sparse-verification step of long-context speculative
decoding (Dustin, arXiv 2606.24957): hybrid importance scoring, a global
TopK verification set, and attention over the selected K/V rows only.

The compute lives in libdustin.so (HIP kernels behind the C ABI of
include/dustin.h); this package only marshals torch tensors into it.
"""
from ._lib import (  # noqa: F401
    KV, DustinError, DustinKV, Workspace, lib,
    dustin_append_window_kv, dustin_arr, dustin_commit_window, dustin_score, dustin_draft_row_lse,
    dustin_sparse_verify_attn,
    dustin_sparse_verify_attn_noalloc,
    dustin_page_bounds, dustin_page_scores, dustin_policy_sweep, dustin_topk, dustin_verify_attn,
    dustin_verify_attn_append,
    dustin_window_attn, dustin_window_mean, dustin_head_scores, dustin_candidate_arr, dustin_greedy_select,
    POLICY_NAMES, dustin_probe_stream_read, dustin_probe_gather_rows,
    EXPORTS, LIB_PATH,
)
