"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU) and check that
at least one pin catches it: the pins are strong enough that such a mistake cannot pass."""
import os
import types

import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "pbs_oracle.py")

MUTANTS = {
    "scores_no_scale": ("Z = scale * (Qr @", "Z = (Qr @"),
    "scores_no_causal_mask": ("Z = np.where(visible, Z, -np.inf)", "Z = Z"),
    "scores_sum_not_mean": ("(acc / (G * block))", "(acc / block)"),
    "scores_first_block_rows": ("rows = np.arange(N - block, N)", "rows = np.arange(0, block)"),
    "order_ascending": ("neg = np.where(nan, np.float32(0), -v)", "neg = np.where(nan, np.float32(0), v)"),
    "order_ties_high_index": ("(pos, neg, nan)", "(-pos, neg, nan)"),
    "order_nan_first": ("(pos, neg, nan)", "(pos, neg, ~nan)"),
    "permute_inverse_gather": ("out[b, h] = x[b, h, perm[b, h]]", "out[b, h] = x[b, h, np.argsort(perm[b, h])]"),
    "visible_inverse_perm": ("perm_row[slots].astype(np.int64)", "np.argsort(perm_row)[slots].astype(np.int64)"),
    "visible_own_excludes_t": ("own = np.arange(s0, t + 1)", "own = np.arange(s0, t)"),
    "pool_sum_not_mean": ("qbar = bf16_to_f64(q[b, g]).reshape(nb, block, d).mean(axis=1)",
                          "qbar = bf16_to_f64(q[b, g]).reshape(nb, block, d).sum(axis=1)"),
    "candidates_include_own_segment": ("n = (i // bps) * bps\n                logits",
                                       "n = min((i // bps + 1) * bps, nb)\n                logits"),
    "block_logits_no_scale": ("logits = scale * (kbar[b, h, :n] @ qbar[i])", "logits = (kbar[b, h, :n] @ qbar[i])"),
    "keep_min_zero": ("return max(1, int(math.floor(", "return max(0, int(math.floor("),
    "keep_round_up": ("int(math.floor(float(ratio) * n))", "int(math.ceil(float(ratio) * n))"),
    "coverage_strict": (">= tau          # compared in double", "> tau          # compared in double"),
    "coverage_double_sum": ("axis=-1, dtype=np.float32)   # sequential", "axis=-1, dtype=np.float64)   # sequential"),
    "attn_mask_strict": ("Z = np.where(keys[None, :] <= t[:, None], Z, -np.inf)",
                         "Z = np.where(keys[None, :] < t[:, None], Z, -np.inf)"),
    "attn_no_scale": ("Z = scale * (Qb @ Kf[keys].T)", "Z = (Qb @ Kf[keys].T)"),
    "attn_values_are_keys": ("ob = (E @ Vf[keys]) / l", "ob = (E @ Kf[keys]) / l"),
    "attn_gqa_modulo": ("        h = g // G\n        Kf, Vf = _head_kv(cache, k, v, b, h)\n        sel = None",
                        "        h = g % Hkv\n        Kf, Vf = _head_kv(cache, k, v, b, h)\n        sel = None"),
    "attn_lse_log2": ("lb = (m + np.log(l))[:, 0]", "lb = (m + np.log2(l))[:, 0]"),
    "coverage_sparse_softmax": ("cov = Pd[:, keys].sum(axis=1)",
                                "cov = Pd[:, keys].sum(axis=1) / Pd[:, keys].sum(axis=1)"),
    "coverage_no_causal_mask": ("Z = np.where(np.arange(t[-1] + 1)[None, :] <= t[:, None], Z, -np.inf)", "Z = Z"),
    "density_own_off_by_one": ("own += i - s0 + 1", "own += i - s0"),
    "keep_first_at_end": ("order = np.concatenate([np.zeros(order.shape[:-1] + (1,), order.dtype), rest], axis=-1)",
                          "order = np.concatenate([rest, np.zeros(order.shape[:-1] + (1,), order.dtype)], axis=-1)"),
    "keep_first_ignored": ("        if keep_first:\n            rest", "        if False:\n            rest"),
    "qperm_mask_on_slots": ("ob, lb = _attend_rows(Qb, Kf, Vf, keys, t, scale)     # causal test",
                            "ob, lb = _attend_rows(Qb, Kf, Vf, keys, slots, scale)     # causal test"),
    "qperm_output_not_inverted": ("o[b, g, t], lse[b, g, t] = ob, lb                 # the inverse",
                                  "o[b, g, slots], lse[b, g, slots] = ob, lb                 # the inverse"),
    "qperm_heads_modulo": ("return apply_permutation(q, np.repeat(perm, Hq // Hkv, axis=1))",
                           "return apply_permutation(q, np.tile(perm, (1, Hq // Hkv, 1)))"),
    "varlen_idx_not_shifted": ('out["idx"][:, :, i0:i1, :w] = np.where(r["idx"] >= 0, r["idx"] + i0, -1)',
                               'out["idx"][:, :, i0:i1, :w] = r["idx"]'),
    "varlen_perm_not_shifted": ('out["perm"][:, :, a:b] = r["perm"] + a', 'out["perm"][:, :, a:b] = r["perm"]'),
    "varlen_P_rows_only": ('out["P"][:, :, i0:i1, i0:i1] = r["P"]', 'out["P"][:, :, i0:i1, :i1 - i0] = r["P"]'),
    "density_perm_max_position": ("perm[b, h, j * block:(j + 1) * block].min() <= last",
                                  "perm[b, h, j * block:(j + 1) * block].max() <= last"),
    # the score softmax over the whole sequence instead of one segment at a time
    "scores_global_softmax": (
        "            for s0 in range(0, N, segment):\n"
        "                keys = np.arange(s0, s0 + segment)\n"
        "                Z = scale * (Qr @ bf16_to_f64(k[b, h, s0:s0 + segment]).T)      # [G*Bs, S]\n"
        "                visible = keys[None, :] <= t_of_row[:, None]\n"
        "                Z = np.where(visible, Z, -np.inf)\n"
        "                Z = Z - Z.max(axis=1, keepdims=True)\n"
        "                E = np.exp(Z)\n"
        "                Pm = E / E.sum(axis=1, keepdims=True)\n"
        "                acc[s0:s0 + segment] = Pm.sum(axis=0)\n",
        "            for s0 in range(0, N, N):\n"
        "                keys = np.arange(s0, s0 + N)\n"
        "                Z = scale * (Qr @ bf16_to_f64(k[b, h, s0:s0 + N]).T)      # [G*Bs, S]\n"
        "                visible = keys[None, :] <= t_of_row[:, None]\n"
        "                Z = np.where(visible, Z, -np.inf)\n"
        "                Z = Z - Z.max(axis=1, keepdims=True)\n"
        "                E = np.exp(Z)\n"
        "                Pm = E / E.sum(axis=1, keepdims=True)\n"
        "                acc[s0:s0 + N] = Pm.sum(axis=0)\n"),
    # block selection fed the unpermuted keys, or always run as keep ratio
    "prefill_unpermuted_kbar": ("P = block_probabilities(q, k_perm, block=block, segment=segment, scale=scale)",
                                "P = block_probabilities(q, k, block=block, segment=segment, scale=scale)"),
    "prefill_mode_ignored": ("counts, idx = select_blocks(P, block=block, segment=segment, mode=mode, param=param)",
                             "counts, idx = select_blocks(P, block=block, segment=segment, mode=KEEP, param=param)"),
    # attention of the pipeline in the identity order, or over the permuted copies as if unpermuted
    "prefill_attention_identity_order": ("o, lse = attention(q, k, v, block=block, segment=segment, scale=scale, perm=perm,",
                                         "o, lse = attention(q, k, v, block=block, segment=segment, scale=scale, perm=None,"),
    "prefill_attention_permuted_copies": ("o, lse = attention(q, k, v, block=block, segment=segment, scale=scale, perm=perm,",
                                          "o, lse = attention(q, k_perm, v_perm, block=block, segment=segment, scale=scale, perm=perm,"),
}


def _mutant(old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
