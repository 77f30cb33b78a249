"""CPU tests: the oracle against its pins, and planted mistakes against the pins.

The second half copies the oracle's source, plants one plausible mistake in
the copy (on the CPU, never in the product) and shows that at least one pin
rejects it.
"""
import os
import types

import pytest

import oracle
import oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "awq_oracle.py")


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.awq_oracle)


# (what is broken, text in the oracle, replacement, pins expected to catch it)
MUTATIONS = [
    ("stats without |x|", "np.abs(x).sum(axis=0)", "x.sum(axis=0)", [P.check_stats_closed_form]),
    ("stats sum, not mean", "(S / F64(T))", "(S)", [P.check_stats_closed_form]),
    ("stats over the wrong axis", "np.abs(x).sum(axis=0)", "np.abs(x).sum(axis=1)",
     [P.check_stats_closed_form]),
    ("scale not normalised", "s = p / np.sqrt(p.max() * p.min())", "s = p",
     [P.check_scale_closed_form]),
    ("scale normalised by its max", "s = p / np.sqrt(p.max() * p.min())", "s = p / p.max()",
     [P.check_scale_closed_form]),
    ("exponent applied to the reciprocal", "p = a ** F64(F32(alpha))", "p = a ** (-F64(F32(alpha)))",
     [P.check_scale_closed_form]),
    ("2^b levels instead of 2^b-1 intervals", "qmax = F32(2 ** bits - 1)\n    mx",
     "qmax = F32(2 ** bits)\n    mx", [P.check_quant_worked_examples]),
    ("zero point with the wrong sign", "np.rint((-mn) / step)", "np.rint(mn / step)",
     [P.check_quant_worked_examples]),
    ("codes truncated instead of rounded", "np.rint(wg / step[:, :, None])",
     "np.floor(wg / step[:, :, None])", [P.check_codes_nearest_bruteforce]),
    ("range not widened to contain 0", "np.maximum(wp_groups.max(axis=2), F32(0))",
     "wp_groups.max(axis=2)", [P.check_codes_nearest_bruteforce]),
    ("clip ratio applied to the max only", "mn = (r * mn).astype(F32)", "mn = mn.astype(F32)",
     [P.check_quant_worked_examples]),
    ("symmetric step over 2^(b-1)", "amax / F32(2 ** (bits - 1) - 1)", "amax / F32(2 ** (bits - 1))",
     [P.check_quant_worked_examples, P.check_codes_nearest_bruteforce]),
    ("dequantise without the zero point", "(qg - zero.astype(F64)[:, :, None])", "(qg - 0)",
     [P.check_quant_worked_examples]),
    ("fold multiplies by s", "return wp_hat / np.asarray(s32", "return wp_hat * np.asarray(s32",
     [P.check_fold_invariance, P.check_quant_worked_examples]),
    ("error of the weights, not of the output",
     "E = np.asarray(w_hat, dtype=F64) - np.asarray(w32, dtype=F64)",
     "E = np.asarray(w_hat, dtype=F64)", [P.check_output_error_bruteforce]),
    ("absolute instead of squared error", "M += (Y * Y).sum(axis=0)", "M += np.abs(Y).sum(axis=0)",
     [P.check_output_error_bruteforce]),
    ("sum over output channels instead of tokens", "M += (Y * Y).sum(axis=0)",
     "M += (Y * Y).sum(axis=1)",
     [P.check_output_error_bruteforce]),
    ("argmax instead of argmin", "best = int(np.argmin(mse))", "best = int(np.argmax(mse))",
     [P.check_search_scale_bruteforce]),
    ("curve divided by T only", "mse = row_sums.sum(axis=1) / F64(T * R)",
     "mse = row_sums.sum(axis=1) / F64(T)", [P.check_search_scale_bruteforce,
                                            P.check_monotone_and_separable]),
    ("clip picks the worst ratio", "idx = np.argmin(row_sums, axis=0)",
     "idx = np.argmax(row_sums, axis=0)", [P.check_search_clip_bruteforce]),
    ("codes packed from the top bit down", "w, b = divmod(bits * c, 32)",
     "w, b = divmod(bits * c, 32); b = 32 - bits - b if b + bits <= 32 else b",
     [P.check_pack_layout, P.check_pack_int3_layout]),
    ("codes packed along the input dim", "qweight = pack_codes(np.ascontiguousarray(q.T), bits)",
     "qweight = pack_codes(np.ascontiguousarray(q), bits)", [P.check_pack_layout]),
    ("straddling 3-bit codes lose their high bits", "        if b + bits > 32:\n",
     "        if False:\n", [P.check_pack_int3_layout]),
    ("consumer ignores the zero point", "((q - z[gidx]).astype(F64) * sc[gidx]).T",
     "((q - 0 * z[gidx]).astype(F64) * sc[gidx]).T", [P.check_w4a16_exact_layer]),
    ("consumer uses the scale of the wrong group", "gidx = np.arange(K) // group",
     "gidx = np.minimum(np.arange(K) // group + 1, K // group - 1)",
     [P.check_w4a16_exact_layer, P.check_w4a16_bruteforce]),
    ("unpacking reads codes from the top bit", "        w, b = divmod(bits * c, 32)\n        v = u",
     "        w, b = divmod(bits * c, 32)\n        b = 32 - bits - b if b + bits <= 32 else b\n        v = u",
     [P.check_w4a16_exact_layer]),
    ("consumer drops the high bits of straddling 3-bit codes",
     "        if b + bits > 32:\n            v = v | (u[:, w + 1]",
     "        if False:\n            v = v | (u[:, w + 1]", [P.check_w4a16_bruteforce]),
    ("group size ignored by the quantiser", "    G = K // group\n",
     "    group = 128\n    G = K // group\n", [P.check_codes_nearest_bruteforce]),
    ("group searched on its first layer only",
     "W = np.concatenate([np.asarray(w) for w in Ws], axis=0)", "W = np.asarray(Ws[0])",
     [P.check_search_group]),
    ("bf16 ties rounded away from zero", "((d_hi == d_lo) & ((lo & np.uint32(1)) == 1))",
     "(d_hi == d_lo)", [P.check_encode_bf16_exhaustive]),
    ("bf16 truncated", "up = finite & ((d_hi < d_lo)", "up = finite & ((d_hi < -1.0)",
     [P.check_encode_bf16_exhaustive]),
    ("fold multiplies by s", "q = decode(a, dtype) / np.asarray(d32",
     "q = decode(a, dtype) * np.asarray(d32",
     [P.check_fold_norm, P.check_fold_linear]),
    ("norm bias not folded", "b = None if beta is None else _divide_stored(beta, dtype, s)",
     "b = None if beta is None else np.asarray(beta)", [P.check_fold_norm]),
    ("previous linear folded along its input dim", "_divide_stored(W_prev, dtype, s[:, None])",
     "_divide_stored(W_prev, dtype, s[None, :])", [P.check_fold_linear]),
    ("fp16 bits read as bf16", "return np.asarray(a, dtype=np.uint16).view(np.float16).astype(F32)",
     "return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)",
     [P.check_decode_f16_exhaustive]),
    ("fp16 bit patterns converted as integers",
     "return np.asarray(a, dtype=np.uint16).view(np.float16).astype(F32)",
     "return np.asarray(a, dtype=np.uint16).astype(np.float16).astype(F32)",
     [P.check_decode_f16_exhaustive]),
    ("Gram matrix keeps only the last token block", "        G += x.T @ x", "        G = x.T @ x",
     [P.check_gram_route]),
    ("Gram route measures the candidate's weights, not its error",
     "        E = w_hat[r0:r0 + rows] - w[r0:r0 + rows]", "        E = w_hat[r0:r0 + rows]",
     [P.check_gram_route]),
    ("Gram route keeps only G's diagonal", "        M[r0:r0 + rows] = ((E @ G) * E).sum(axis=1)",
     "        M[r0:r0 + rows] = ((E * np.diag(G)) * E).sum(axis=1)", [P.check_gram_route]),
    ("Gram route from X·Xᵀ", "        G += x.T @ x", "        G += (x @ x.T)[:K, :K]",
     [P.check_gram_route]),
]


def _mutant(old, new):
    with open(ORACLE_SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mod = types.ModuleType("awq_oracle_mutant")
    exec(compile(src.replace(old, new, 1), "awq_oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("desc,old,new,checks", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(desc, old, new, checks):
    mod = _mutant(old, new)
    caught = False
    for chk in checks:
        try:
            chk(mod)
        except Exception:
            caught = True
            break
    assert caught, f"no pin caught: {desc}"
