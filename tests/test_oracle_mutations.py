"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.

Each mutation rewrites one snippet of one oracle function's source, compiles
the result into the oracle module's namespace and patches it in; then every
pin runs and at least one must fail.
"""
import inspect
import textwrap

import pytest

import oracle.layer as L
from oracle_pins import ALL_PINS

MUTATIONS = [
    # (id, function, snippet as written, planted mistake)
    ("scale_1_over_d", "attend_union", "1.0 / math.sqrt(q.shape[-1])", "1.0 / q.shape[-1]"),
    ("no_normaliser", "attend_union", "return num / den,", "return num,"),
    ("keys_as_values", "attend_union", "num += p @ np.asarray(v,", "num += p @ np.asarray(k,"),
    ("frame_off_by_one", "frame_attention", "keys = slice(f * L, (f + 1) * L)",
     "keys = slice(f * L, (f + 1) * L + 1)"),
    ("window_no_clip_rows", "window_table", "min(block * by + block, gh)", "block * by + block"),
    ("window_transposed", "window_table", "rows.append(f * L + S + r * gw + c)",
     "rows.append(f * L + S + c * gh + r)"),
    ("no_special_query_block", "query_block_table", "        if S:\n", "        if False:\n"),
    ("block_score_unscaled", "block_scores", "/ math.sqrt(d)", ""),
    ("topk_ties_high", "_topk_rows", "key=lambda j: (-row[j], j)", "key=lambda j: (-row[j], -j)"),
    ("topk_rank_order", "_topk_rows", "np.sort(np.array(order[:top_k], dtype=np.int32))",
     "np.array(order[:top_k], dtype=np.int32)"),
    ("topk_smallest", "_topk_rows", "key=lambda j: (-row[j], j)", "key=lambda j: (row[j], j)"),
    ("fine_drops_specials", "fine_attention", "if use_spec:", "if False:"),
    ("ref_specials_twice", "fine_attention", "f0 = 1 if keep_ref else 0", "f0 = 0"),
    ("ref_frame_dropped", "fine_attention", "            if keep_ref:\n", "            if False:\n"),
    ("ref_frame_patches_only", "fine_attention", "ref = np.arange(L if keep_ref else 0)",
     "ref = np.arange(geom.n_special if keep_ref else 0, L if keep_ref else 0)"),
    ("ref_rows_specials_twice", "fine_key_rows", "f0 = 1 if keep_ref else 0", "f0 = 0"),
    ("topk_first_ignored", "select_topk", "dtype=np.float64)[first:]", "dtype=np.float64)"),
    ("topk_first_local_index", "_topk_rows", "first + np.sort(", "np.sort("),
    ("gsa_ref_selects_frame0", "gsa_layer", "if keep_ref else 0\n", "if False else 0\n"),
    ("gate_swapped", "gate", "g[..., 0:1] * np.asarray(o_cmp", "g[..., 1:2] * np.asarray(o_cmp"),
    ("gate_no_bias", "gate", " + np.asarray(b, np.float64)", ""),
    ("sga_phase_1", "subsample_plan", "r % s_h == 0 and c % s_w == 0",
     "r % s_h == 1 % s_h and c % s_w == 0"),
    ("sga_mean_over_all", "sga_compact", "drop_rows = [base + p for p in dropped]",
     "drop_rows = [base + p for p in dropped + kept]"),
    ("sga_own_frame_twice", "subsampled_attention",
     "s_c[i, f * m:(f + 1) * m] = -np.inf", "pass"),
    ("sga_mean_token_dropped", "sga_compact", "        if dropped:\n", "        if False:\n"),
    ("sga_log_count_wrong", "subsampled_attention", "math.log(len(dropped))",
     "math.log(len(dropped) + 1)"),
    ("pad_ignored", "compress", "den = block * block if include_pad else len(rows)", "den = len(rows)"),
    ("pad_divides_valid_by_16", "compress", "den = block * block if include_pad else len(rows)",
     "den = block * block"),
    ("pooled_first_token", "compressed_attention_pooled",
     "o_blk = dense_attention(pooled_queries(q, geom, block, blocks=need), k_cmp, v_cmp,",
     "o_blk = dense_attention(np.stack([q[query_block_table(geom, block)[b][0]] for b in need]), k_cmp, v_cmp,"),
    ("pooled_upsample_shifted", "compressed_attention_pooled",
     "pos = np.searchsorted(need, owner[rows])",
     "pos = np.minimum(np.searchsorted(need, owner[rows]) + 1, len(need) - 1)"),
    ("diag_never_added", "_subsampled_token_diagonal", "diag = was_dropped[rows % L]",
     "diag = np.zeros(len(rows), dtype=bool)"),
    ("diag_always_added", "_subsampled_token_diagonal", "diag = was_dropped[rows % L]",
     "diag = np.ones(len(rows), dtype=bool)"),
    ("diag_no_log_count", "_subsampled_token_diagonal", "bias_c[m - 1::m] = math.log(len(dropped))",
     "pass"),
    ("prob_no_lse", "probability_block_scores", "out[h, i] = np.exp(s - lse).mean(axis=0)[first:]",
     "out[h, i] = np.exp(s).mean(axis=0)[first:]"),
    ("prob_sum_not_mean", "probability_block_scores", "out[h, i] = np.exp(s - lse).mean(axis=0)[first:]",
     "out[h, i] = np.exp(s - lse).sum(axis=0)[first:]"),
    ("prob_max_not_mean", "probability_block_scores", "out[h, i] = np.exp(s - lse).mean(axis=0)[first:]",
     "out[h, i] = np.exp(s - lse).max(axis=0)[first:]"),
    ("prob_lse_over_competing", "probability_block_scores",
     "s = (qq[qbt[bb], h, :] @ kh.T) / math.sqrt(d)",
     "s = (qq[qbt[bb], h, :] @ kh[first:].T) / math.sqrt(d); s = np.concatenate([np.full((s.shape[0], first), -np.inf), s], axis=1)"),
    ("prob_no_scale", "probability_block_scores", "s = (qq[qbt[bb], h, :] @ kh.T) / math.sqrt(d)",
     "s = (qq[qbt[bb], h, :] @ kh.T)"),
    ("prob_first_token_only", "probability_block_scores", "s = (qq[qbt[bb], h, :] @ kh.T) / math.sqrt(d)",
     "s = (qq[qbt[bb][:1], h, :] @ kh.T) / math.sqrt(d)"),
    ("prob_ranked_not_log", "select_topk_probability",
     "ranked[h] = np.where(r > 0, np.log(np.maximum(r, 0.0)), -np.inf)", "ranked[h] = r"),
    ("diag_own_frame_masked", "_subsampled_token_diagonal", "s_c = (qc @ ckh.T) * scale + bias_c",
     "s_c = (qc @ ckh.T) * scale + bias_c; s_c[:, :m] = -np.inf"),
]


def _mutant(func_name, old, new):
    src = textwrap.dedent(inspect.getsource(getattr(L, func_name)))
    assert src.count(old) >= 1, f"snippet not found in {func_name}: {old!r}"
    src = src.replace(old, new)
    ns = {}
    exec(compile(src, f"<mutant {func_name}>", "exec"), L.__dict__, ns)
    return ns[func_name]


@pytest.mark.parametrize("mid,func,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, mid, func, old, new):
    monkeypatch.setattr(L, func, _mutant(func, old, new))
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception as e:  # AssertionError, or the mutant breaking outright
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {mid}"
