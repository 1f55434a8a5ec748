"""Planted mistakes: each test breaks the oracle on the CPU in a plausible way
and checks that one of the pins catches it (so the pins are not vacuous)."""
import numpy as np
import pytest

import oracle.msa_oracle as om
from tests import test_oracle_attention as ta
from tests import test_oracle_proxy as tp
from tests import test_oracle_topk as tt


def test_off_by_one_causal_alignment_is_caught(monkeypatch):
    orig = om.Layout.pos
    monkeypatch.setattr(om.Layout, "pos", lambda self, r: orig(self, r) - 1 if orig(self, r) > 0 else 0)
    with pytest.raises(AssertionError):
        tp.test_positional_closed_form([300], [300], 16, 2)
    with pytest.raises(AssertionError):
        ta.test_all_blocks_selected_equals_dense_causal_gqa([200], [200], 32, 4, 2)


def test_wrong_kv_head_is_caught(monkeypatch):
    orig = om.gather_rows

    def bad(pages_bits, dtype, scale, kv_indices, lay, s, head, key_idx):
        return orig(pages_bits, dtype, scale, kv_indices, lay, s, (head + 1) % pages_bits.shape[1], key_idx)
    monkeypatch.setattr(om, "gather_rows", bad)
    with pytest.raises(AssertionError):
        ta.test_all_blocks_selected_equals_dense_causal_gqa([200], [200], 32, 4, 2)
    with pytest.raises(AssertionError):
        tp.test_positional_closed_form([256], [256], 128, 2)


def test_ties_to_higher_index_are_caught(monkeypatch):
    def bad(scores, local, k):
        cand = np.arange(local)
        R = min(k - 1, local)
        order = np.lexsort((-cand, -scores[:local]))
        sel = np.sort(np.concatenate([cand[order[:R]], [local]]))
        out = np.full(k, -1, np.int32)
        out[:sel.size] = sel
        return out
    monkeypatch.setattr(tt, "topk_select_row", bad)
    with pytest.raises(AssertionError):
        tt.test_hand_worked_cases()
    with pytest.raises(AssertionError):
        for seed in range(40):
            tt.test_brute_force_subsets(seed)


def test_dropping_the_local_block_is_caught(monkeypatch):
    def bad(scores, local, k):
        cand = np.arange(local + 1)
        order = np.lexsort((cand, -scores[:local + 1]))
        sel = np.sort(cand[order[:min(k, local + 1)]])
        out = np.full(k, -1, np.int32)
        out[:sel.size] = sel
        return out
    monkeypatch.setattr(tt, "topk_select_row", bad)
    with pytest.raises(AssertionError):
        tt.test_hand_worked_cases()


def test_swapped_mxfp4_nibbles_are_caught(monkeypatch):
    """Odd elements in the low nibble instead of the high one."""
    from tests import test_oracle_formats as tf
    orig = om.mxfp4_record_rows

    def bad(rec, slots):
        rec = np.asarray(rec, dtype=np.uint8)
        cb = 128 * 64
        sw = rec.copy()
        sw[:, :cb] = (rec[:, :cb] >> 4) | (rec[:, :cb] << 4)
        return orig(sw, slots)
    monkeypatch.setattr(om, "mxfp4_record_rows", bad)
    with pytest.raises(AssertionError):
        tp.test_mxfp4_proxy_k_equals_bf16_path_on_the_same_values()
    monkeypatch.setattr(tf, "mxfp4_record_rows", bad, raising=False)
    import oracle
    monkeypatch.setattr(oracle, "mxfp4_record_rows", bad)
    with pytest.raises(AssertionError):
        tf.test_mxfp4_record_layout_by_hand()


def test_mxfp4_scale_group_off_by_one_is_caught(monkeypatch):
    """Each 32-element group scaled by its neighbour's scale byte."""
    orig = om.mxfp4_record_rows

    def bad(rec, slots):
        rec = np.asarray(rec, dtype=np.uint8).copy()
        cb = 128 * 64
        sc = rec[:, cb:].reshape(rec.shape[0], 128, 4)
        rec[:, cb:] = np.roll(sc, 1, axis=2).reshape(rec.shape[0], -1)
        return orig(rec, slots)
    monkeypatch.setattr(om, "mxfp4_record_rows", bad)
    with pytest.raises(AssertionError):
        tp.test_mxfp4_proxy_k_equals_bf16_path_on_the_same_values()


def test_backward_without_the_rowsum_term_is_caught(monkeypatch):
    """ds_j = p_j dp_j (dropping the D = <dout, o> term) must fail the pins."""
    from tests import test_oracle_backward as tb
    src = om.sparse_attention_backward

    def bad(q, k_pages, v_pages, kv_indices, sel, qo_lens, kv_lens, B, scale, dout):
        zero_o = {"flag": True}
        orig_gather = om.gather_rows
        dq, dk, dv = src(q, k_pages, v_pages, kv_indices, sel, qo_lens, kv_lens, B, scale, dout)
        # recompute dq with ds = p * dp only
        lay = om.Layout(qo_lens, kv_lens, B)
        T, Hq, d = q.shape
        G = Hq // k_pages.shape[1]
        for r in range(T):
            s = lay.seq_of_row(r)
            pos = lay.pos(r)
            for g in range(k_pages.shape[1]):
                blocks = sorted(set(int(b) for b in sel[r, g] if b >= 0))
                keys = np.concatenate([np.arange(b * B, (b + 1) * B) for b in blocks])
                keys = keys[(keys <= pos) & (keys < lay.kv[s])]
                K = orig_gather(k_pages, om.BF16, None, kv_indices, lay, s, g, keys)
                V = orig_gather(v_pages, om.BF16, None, kv_indices, lay, s, g, keys)
                for h in range(g * G, (g + 1) * G):
                    sc = scale * (K @ om.bf16_to_f64(q[r, h]))
                    p = np.exp(sc - sc.max())
                    p /= p.sum()
                    dq[r, h] = scale * ((p * (V @ om.bf16_to_f64(dout[r, h]))) @ K)
        return dq, dk, dv
    monkeypatch.setattr(tb, "sparse_attention_backward", bad)
    with pytest.raises(AssertionError):
        tb.test_backward_matches_finite_differences_of_the_forward()
