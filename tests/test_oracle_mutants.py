"""Planted mistakes in (a copy of) the oracle must each fail at least one pin.

Each mutant rewrites one line of the oracle's source (a dropped term, a wrong
sign or index, a transposed operand, a wrong mask or log base), loads it as a
separate module, swaps it in, and runs the pins from ``test_oracle.py``.
"""
import inspect
import types

import numpy as np
import pytest

import oracle
from oracle import attention as A
from oracle import rope as R
from oracle import xent as X
from oracle import zigzag as Z
from tests import test_oracle as T
from tests import test_oracle_blocks as TB
from tests import test_oracle_rope as TR
from tests import test_oracle_xent as TX

MUTANTS = {
    "strict_causal": ("pos_k[None, :] <= pos_q[:, None]", "pos_k[None, :] < pos_q[:, None]"),
    "no_scale_in_scores": ("s = scale * (qb @ kc.T)", "s = (qb @ kc.T)"),
    "log2_lse": ("m + np.log(np.where(has, l, 1.0))", "m + np.log2(np.where(has, l, 1.0))"),
    "delta_sign": ("ds = p * (dp - dl[:, None])", "ds = p * (dp + dl[:, None])"),
    "dq_no_scale": ("dq[i0:i1] = scale * (ds @ kc)", "dq[i0:i1] = (ds @ kc)"),
    "dk_uses_p": ("dk[cols] += scale * (ds.T @ q[i0:i1])", "dk[cols] += scale * (p.T @ q[i0:i1])"),
    "dv_uses_ds": ("dv[cols] += p.T @ dob", "dv[cols] += ds.T @ dob"),
    "delta_from_v": ("dl = np.sum(dob * ob, axis=1)", "dl = np.sum(dob * dob, axis=1)"),
    "merge_swapped": ("w1 * o1 + w2 * o2", "w2 * o1 + w1 * o2"),
    "merge_no_log": ("lse = np.logaddexp(lse1, lse2)", "lse = np.maximum(lse1, lse2)"),
    "pv_transposed_v": ("o = p @ vc", "o = p @ vc[::-1]"),
    "sums_strict": ('side="right"', 'side="left"'),
    "sums_unsorted": ("csum[n]", "csum[np.minimum(n + 1, len(csum) - 1)]"),
    # the row-block path of the full-size comparisons
    "dk_assigned_per_block": ("dk[cols] += scale * (ds.T @ q[i0:i1])", "dk[cols] = scale * (ds.T @ q[i0:i1])"),
    "dv_assigned_per_block": ("dv[cols] += p.T @ dob", "dv[cols] = p.T @ dob"),
    "block_end_off_by_one": ("yield i0, min(sq, i0 + rows)", "yield i0, min(sq, i0 + rows - 1)"),
    "blocks_stop_one_row_early": ("for i0 in range(0, sq, rows):", "for i0 in range(0, sq - 1, rows):"),
    "useful_keys_from_block_min": ("pos_k <= pos_q_blk.max()", "pos_k <= pos_q_blk.min()"),
    # the [B, S, H, D] head wrappers
    "fwd_heads_key_head_swapped": ("attn_fwd(q[b, :, h], k[b, :, h], v[b, :, h], pos_q",
                                   "attn_fwd(q[b, :, h], k[b, :, n], v[b, :, h], pos_q"),
    "bwd_heads_value_head_swapped": ("attn_bwd(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h]",
                                     "attn_bwd(q[b, :, h], k[b, :, h], v[b, :, n], do[b, :, h]"),
    "bwd_heads_batch_slot": ("res[key][b, :, n] = val", "res[key][0, :, n] = val"),
}

# mistakes in the [B, S, H, D] wrapper of the rotary oracle
RHMUTANTS = {
    "rope_heads_key_head_swapped": ("attn_bwd_rope(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h]",
                                    "attn_bwd_rope(q[b, :, h], k[b, :, n], v[b, :, h], do[b, :, h]"),
    "rope_heads_output_slot": ("res[key][b, :, n] = r[key]", "res[key][b, :, h] = r[key]"),
}

ZMUTANTS = {
    "zigzag_wrong_partner": ("chunk_positions(2 * world - 1 - rank, C)", "chunk_positions(2 * world - 2 - rank, C)"),
    "zigzag_swapped_order": ("[chunk_positions(rank, C), chunk_positions(2 * world - 1 - rank, C)]",
                             "[chunk_positions(2 * world - 1 - rank, C), chunk_positions(rank, C)]"),
}

XMUTANTS = {
    "xent_no_onehot": ("grad[rows[keep], y[keep]] -= 1.0", "grad[rows[keep], y[keep]] -= 0.0"),
    "xent_log2_lse": ("lse = m + np.log(np.exp(x - m[:, None]).sum(axis=1))",
                      "lse = m + np.log2(np.exp(x - m[:, None]).sum(axis=1))"),
    "xent_no_scale": ("grad *= grad_scale", "grad *= 1.0"),
    "xent_ignored_kept": ("grad[~keep] = 0.0", "grad[~keep] = grad[~keep]"),
    "xent_label_off_by_one": ("picked = np.where(keep, x[rows, np.where(keep, y, 0)], 0.0)",
                              "picked = np.where(keep, x[rows, np.where(keep, (y + 1) % v, 0)], 0.0)"),
}

XPINS = [
    TX.test_golden_two_classes,
    lambda: TX.test_matches_torch_cross_entropy(0, 7, 5),
    TX.test_uniform_logits_closed_form,
    TX.test_invariants,
]

RMUTANTS = {
    "rope_sin_sign": ("return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)",
                      "return np.concatenate([a * c + b * s, b * c - a * s], axis=-1)"),
    "rope_interleaved_pairs": ("a, b = x[..., :half], x[..., half:]", "a, b = x[..., 0::2], x[..., 1::2]"),
    "rope_exponent_k_over_d": ("-2.0 * k / D", "-1.0 * k / D"),
    "rope_inverse_not_transposed": ("s = -s", "s = s"),
    "rope_position_off_by_one": ("phi = pos.astype(np.float64)[:, None]", "phi = (pos + 1).astype(np.float64)[:, None]"),
    "bf16_truncates": ("r = (bits + half_ulp + lsb) &", "r = (bits) &"),
    "rope_dq_not_rotated_back": ('out["dq"] = rope(out["dq"][:, None, :], pos_q, theta, inverse=True)[:, 0, :]',
                                 'out["dq"] = out["dq"]'),
    "rope_dk_rotated_forward": ('out["dk"] = rope(out["dk"][:, None, :], pos_k, theta, inverse=True)[:, 0, :]',
                                'out["dk"] = rope(out["dk"][:, None, :], pos_k, theta)[:, 0, :]'),
}

RPINS = [
    TR.test_golden_quarter_turn,
    TR.test_d2_is_complex_rotation,
    lambda: TR.test_matches_transformers_llama(64, 1e4),
    TR.test_orthogonal_and_inverse,
    TR.test_inv_freq_closed_form,
    TR.test_round_bf16_against_torch_and_ties,
    TR.test_attention_gradient_through_rotation,
]

PINS = [
    lambda: T.test_golden_attention("causal_two_tokens.json"),
    lambda: T.test_golden_attention("full_one_query.json"),
    T.test_golden_merge,
    lambda: T.test_bruteforce_tiny(1, True, "random"),
    lambda: T.test_torch_autograd(0, True, 4),
    T.test_zero_query_counts_and_means,
    lambda: T.test_split_merge_equals_unsplit("random", True),
    lambda: T.test_allowed_sums_match_mask(True),
    TB.test_row_blocks_partition_the_rows,
    lambda: TB.test_row_blocks_match_bruteforce(True, "zigzag", 3),
    lambda: TB.test_row_blocks_match_bruteforce(True, "random", 1),
    lambda: TB.test_head_wrappers_match_batched_torch(True, False, None),
]

ZPINS = [
    T.test_golden_zigzag,
    lambda: T.test_zigzag_reassembles_causal_attention(3, 5),
]


def _load_mutant(module, old, new):
    src = inspect.getsource(module)
    assert src.count(old) == 1, old
    mod = types.ModuleType(module.__name__ + "_mutant")
    mod.__package__ = module.__package__  # relative imports of the oracle package
    exec(compile(src.replace(old, new), "<mutant>", "exec"), mod.__dict__)
    return mod


def _fails(pins):
    failed = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed += 1
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_attention_mutant_is_caught(name, monkeypatch):
    mod = _load_mutant(A, *MUTANTS[name])
    for fn in ("allowed_mask", "allowed_sums", "attn_fwd", "attn_bwd", "lse_merge", "_block_fwd", "_row_blocks",
               "_useful_keys", "attn_fwd_heads", "attn_bwd_heads"):
        monkeypatch.setattr(A, fn, getattr(mod, fn))
    with np.errstate(all="ignore"):
        assert _fails(PINS) >= 1, f"no pin caught mutant {name}"


@pytest.mark.parametrize("name", sorted(ZMUTANTS))
def test_zigzag_mutant_is_caught(name, monkeypatch):
    mod = _load_mutant(Z, *ZMUTANTS[name])
    monkeypatch.setattr(oracle, "zigzag_positions", mod.zigzag_positions)
    assert _fails(ZPINS) >= 1, f"no pin caught mutant {name}"


@pytest.mark.parametrize("name", sorted(XMUTANTS))
def test_xent_mutant_is_caught(name, monkeypatch):
    mod = _load_mutant(X, *XMUTANTS[name])
    monkeypatch.setattr(TX, "xent_fwd_bwd", mod.xent_fwd_bwd)
    assert _fails(XPINS) >= 1, f"no pin caught mutant {name}"


@pytest.mark.parametrize("name", sorted(RMUTANTS))
def test_rope_mutant_is_caught(name, monkeypatch):
    mod = _load_mutant(R, *RMUTANTS[name])
    for fn in ("rope", "round_bf16", "attn_bwd_rope", "inv_freq"):
        monkeypatch.setattr(TR, fn, getattr(mod, fn))
    assert _fails(RPINS) >= 1, f"no pin caught mutant {name}"


@pytest.mark.parametrize("name", sorted(RHMUTANTS))
def test_rope_heads_mutant_is_caught(name, monkeypatch):
    mod = _load_mutant(R, *RHMUTANTS[name])
    monkeypatch.setattr(R, "attn_bwd_rope_heads", mod.attn_bwd_rope_heads)
    assert _fails([TB.test_rope_head_wrapper_matches_single_heads]) >= 1, f"no pin caught mutant {name}"


def test_unmutated_oracle_passes_all_pins():
    assert _fails(PINS + ZPINS + XPINS + RPINS + [TB.test_rope_head_wrapper_matches_single_heads]) == 0
