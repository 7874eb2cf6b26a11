"""Plants plausible mistakes in the oracle (on the CPU, through monkeypatching) and checks
that at least one pin fails for each: the pins are able to catch a dropped term, a wrong
sign or index, a transposed operand or a flipped tie rule."""
import numpy as np
import pytest

import oracle.attention as OA
import oracle.flashblock as OF
import oracle.losa as OL
import tests.test_oracle_attention as TA
import tests.test_oracle_flashblock as TF
import tests.test_oracle_losa as TL


def _fails(fn, *args):
    try:
        fn(*args)
    except (AssertionError, ValueError, IndexError):
        return True
    return False


def test_merge_with_swapped_weights_is_caught(monkeypatch):
    def bad(a1, l1, a2, l2):
        return _orig_merge(a1, l2, a2, l1)
    _orig_merge = OA.lse_merge
    monkeypatch.setattr(TA, "lse_merge", bad)
    assert _fails(TA.test_golden_two_key_merge)


def test_attend_without_scale_is_caught(monkeypatch):
    orig = OA.attend
    monkeypatch.setattr(TA, "attend", lambda q, k, v, s: orig(q, k, v, 1.0))
    assert _fails(TA.test_attend_matches_torch_sdpa_fp64)


def test_attend_with_transposed_value_use_is_caught(monkeypatch):
    def bad(q, k, v, scale):
        a, l = OA.attend(q, v, k, scale)       # keys and values swapped
        return a, l
    monkeypatch.setattr(TA, "attend", bad)
    assert _fails(TA.test_attend_closed_forms)


def test_wrong_gqa_mapping_is_caught(monkeypatch):
    monkeypatch.setattr(OA, "_kv_head", lambda h, hq, hkv: h % hkv)
    assert _fails(TA.test_multihead_layouts_brute_force, 3, 2, 8, 2, 3, [2, 7, 4])


def test_merge_dropping_log_term_is_caught(monkeypatch):
    def bad(a1, l1, a2, l2):
        a, l = _orig(a1, l1, a2, l2)
        return a, np.maximum(l1, l2)           # forgets + log(w1 + w2)
    _orig = OA.lse_merge
    monkeypatch.setattr(TA, "lse_merge", bad)
    assert _fails(TA.test_merge_conventions)


def test_threshold_non_strict_is_caught(monkeypatch):
    monkeypatch.setattr(TF, "mask_threshold",
                        lambda m, tau, hq: np.repeat((np.asarray(m) <= tau).astype(np.uint8)[:, None], hq, 1))
    assert _fails(TF.test_golden_reuse_rules)


def test_reuse_that_rewrites_cache_is_caught(monkeypatch):
    def bad(q, k, v, cu, kb, vb, mask, ca, cl, scale):
        return OF.step(q, k, v, cu, kb, vb, np.zeros_like(mask), ca, cl, scale)
    monkeypatch.setattr(TF, "step", bad)
    assert _fails(TF.test_reuse_step_semantics)


def test_topk_tie_to_higher_index_is_caught(monkeypatch):
    def bad(S, k):
        S = np.asarray(S, dtype=np.float64)
        R, P = S.shape
        out = np.full((R, k), -1, dtype=np.int32)
        for r in range(R):
            order = np.lexsort((-np.arange(P), -S[r]))[:k]
            out[r, :order.size] = np.sort(order)
        return out
    monkeypatch.setattr(OL, "topk_pages", bad)
    assert _fails(TL.test_topk_brute_force_with_ties)


def test_quest_min_only_is_caught(monkeypatch):
    def bad(qa, kmin, kmax):
        return _orig(qa, kmin, kmin)
    _orig = OL.quest_scores
    monkeypatch.setattr(OL, "quest_scores", bad)
    assert _fails(TL.test_quest_exact_rational_and_bound)


def test_locality_wrong_sign_is_caught(monkeypatch):
    def bad(qc, qp):
        x, y = np.asarray(qc, float), np.asarray(qp, float)
        return ((x + y) ** 2).mean(axis=(2, 3))
    monkeypatch.setattr(OL, "locality_scores", bad)
    assert _fails(TL.test_golden_locality)


def test_active_set_tie_to_higher_index_is_caught(monkeypatch):
    def bad(scores, n):
        s = np.asarray(scores)
        return np.array([np.sort(sorted(range(s.shape[1]), key=lambda i: (-s[b, i], -i))[:n]) for b in range(s.shape[0])])
    monkeypatch.setattr(OL, "active_set", bad)
    assert _fails(TL.test_active_set_ties_and_order)


def test_residual_complement_off_by_one_is_caught(monkeypatch):
    """A complement that drops the last unselected page breaks the refresh = full pin."""
    import oracle.residual as OR
    import tests.test_oracle_residual as TR
    real = OR.complement_pages
    monkeypatch.setattr(OR, "complement_pages", lambda sel, n: real(sel, n)[:-1])
    assert _fails(TR.test_refresh_step_equals_full_attention)


def test_residual_merge_dropping_a_part_is_caught(monkeypatch):
    import oracle.residual as OR
    import tests.test_oracle_residual as TR
    monkeypatch.setattr(OR, "lse_merge3", lambda a1, l1, a2, l2, a3, l3: OA.lse_merge(a1, l1, a3, l3))
    assert _fails(TR.test_refresh_step_equals_full_attention)


def test_residual_reuse_that_recomputes_is_caught(monkeypatch):
    """A step that refreshes the residual whatever the mask breaks the persistence pin."""
    import oracle.residual as OR
    import tests.test_oracle_residual as TR
    real = OR.step
    monkeypatch.setattr(TR, "step", lambda *a: real(*a[:8], np.zeros_like(a[8]), *a[9:]))
    assert _fails(TR.test_stale_residual_persists_and_only_reusing_heads_keep_it)


def test_lifecycle_mask_from_previous_step_count_is_caught(monkeypatch):
    """Reading M of the previous step for the threshold decision breaks the fresh/reuse pin."""
    import oracle.lifecycle as LC
    import tests.test_oracle_lifecycle as TLC
    real = LC.block_run

    def shifted(q, k, v, cu, kb, vb, scale, rule, m_steps=None, tau=None, gamma=None):
        m2 = None if m_steps is None else np.concatenate([m_steps[:1], m_steps[:-1]])
        return real(q, k, v, cu, kb, vb, scale, rule, m_steps=m2, tau=tau, gamma=gamma)
    monkeypatch.setattr(LC, "block_run", shifted)
    assert _fails(TLC.test_threshold_run_fresh_steps_are_full_attention_and_reuse_keeps_step0)


def test_lifecycle_append_order_is_caught(monkeypatch):
    import oracle.lifecycle as LC
    import tests.test_oracle_lifecycle as TLC
    real = LC.append_block
    monkeypatch.setattr(LC, "append_block", lambda k, v, cu, kb, vb: real(k, v, cu, kb[:, ::-1], vb[:, ::-1]))
    assert _fails(TLC.test_append_tokens_by_brute_force)


def test_varlen_branch_prefix_off_by_one_is_caught(monkeypatch):
    """Reading the next branch's first prefix token (cu_k[b+1] + 1 as the end) breaks the
    brute-force pin."""
    import oracle.varlen as OV
    import tests.test_oracle_varlen as TV
    real = OV.prefix_attention_varlen

    def shifted(q, cu_q, k, v, cu_k, h_kv, scale):
        ck = np.asarray(cu_k).copy()
        ck[1:-1] += 1
        return real(q, cu_q, k, v, ck, h_kv, scale)
    monkeypatch.setattr(TV, "prefix_attention_varlen", shifted)
    assert _fails(TV.test_branches_are_independent_and_brute_force)
