"""Planted mistakes in copies of the oracle source, on the CPU: each
plausible slip (a dropped term, a wrong sign, index or operand) must be
caught by at least one pin. The real oracle is never modified."""
import os
import types

import pytest

import oracle
from oracle_pins import PINS, pin_rows_per_head_equals_full

SRC = os.path.join(os.path.dirname(oracle.__file__), "attn_oracle.c")

MUTANTS = {
    "scale_dropped": ("s[j] = dot * scale;", "s[j] = dot;"),
    "scores_use_v_not_k": ("dot += q[c] * Kbh[j * d + c];", "dot += q[c] * Vbh[j * dv + c];"),
    "causal_hides_diagonal": ("return j <= i;", "return j < i;"),
    "padding_off_by_one": ("return j < valid_len;", "return j <= valid_len;"),
    "exp_sign_flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "max_not_subtracted": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "not_normalised": ("for (int64_t j = 0; j < Nk; ++j) s[j] = s[j] / z;", ""),
    "value_column_reversed": ("o[c] += s[j] * Vbh[j * dv + c];", "o[c] += s[j] * Vbh[j * dv + (dv - 1 - c)];"),
    "empty_row_not_guarded": ("if (!any) {", "if (0) {"),
    "mha_k_v_blocks_swapped": ("Kh[dst] = P[src + d_model];\n                    Vh[dst] = P[src + 2 * d_model];",
                               "Kh[dst] = P[src + 2 * d_model];\n                    Vh[dst] = P[src + d_model];"),
    "mha_heads_interleaved_on_split": ("int64_t src = (b * N + t) * W3 + hh * dk + c;",
                                       "int64_t src = (b * N + t) * W3 + c * h + hh;"),
    "mha_heads_interleaved_on_concat": ("C[(b * N + t) * d_model + hh * dk + c]",
                                        "C[(b * N + t) * d_model + c * h + hh]"),
    "mha_scale_by_d_model": ("ORACLE_MASK_NONE, NULL, 1.0 / sqrt((double)dk), Oh,",
                             "ORACLE_MASK_NONE, NULL, 1.0 / sqrt((double)d_model), Oh,"),
    "cross_scale_by_d_model": ("mask_kind, valid_lens, 1.0 / sqrt((double)dk), Oh,",
                               "mask_kind, valid_lens, 1.0 / sqrt((double)d_model), Oh,"),
    "causal_padding_either_rule": ("return j <= i && j < valid_len;", "return j <= i || j < valid_len;"),
    "causal_padding_ignores_lengths": ("return mask_kind == ORACLE_MASK_PADDING || mask_kind == ORACLE_MASK_CAUSAL_PADDING;",
                                       "return mask_kind == ORACLE_MASK_PADDING;"),
    "kv_heads_interleaved": ("return (b * Hkv + h / (H / Hkv)) * n;", "return (b * Hkv + h % Hkv) * n;"),
    "lse_without_max": ("if (lse) *lse = m + log(z);", "if (lse) *lse = log(z);"),
    "lse_base_two": ("if (lse) *lse = m + log(z);", "if (lse) *lse = m + log2(z);"),
    "bwd_softmax_jacobian_without_row_term": ("const double ds = a[j] * (da[j] - dot);",
                                              "const double ds = a[j] * da[j];"),
    "bwd_dk_without_scale": ("dKbh[j * d + c] += scale * ds * q[c];", "dKbh[j * d + c] += ds * q[c];"),
    "bwd_dv_weighted_by_da": ("dVbh[j * dv + c] += a[j] * g[c];", "dVbh[j * dv + c] += da[j] * g[c];"),
    "bwd_group_first_head_only": ("for (int64_t h = hk * group; h < (hk + 1) * group; ++h) {",
                                  "for (int64_t h = hk * group; h < hk * group + 1; ++h) {"),
    "cross_queries_from_key_sequence": ("matmul_f64(Xq, Wq, Pq, Mq, d_model, d_model);",
                                        "matmul_f64(Xkv, Wq, Pq, Mq, d_model, d_model);"),
    "cross_k_v_swapped": ("Vh[((b * h + hh) * Nkv + t) * dk + c] = Pkv[(b * Nkv + t) * 2 * d_model + d_model + hh * dk + c];",
                          "Vh[((b * h + hh) * Nkv + t) * dk + c] = Pkv[(b * Nkv + t) * 2 * d_model + hh * dk + c];"),
    "cross_padding_ignored": ("oracle_attn(Qh, Kh, Vh, B, h, h, Nq, Nkv, dk, dk, mask_kind, valid_lens,",
                              "oracle_attn(Qh, Kh, Vh, B, h, h, Nq, Nkv, dk, dk, ORACLE_MASK_NONE, valid_lens,"),
    "cross_w_k_block_from_w_q": ("Wkv[r * 2 * d_model + c] = Wqkv[r * W3 + d_model + c];",
                                 "Wkv[r * 2 * d_model + c] = Wqkv[r * W3 + c];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC, encoding="utf-8").read()
    assert text.count(old) == 1, "mutation site not found exactly once: %r" % old
    src = tmp_path / ("mutant_%s.c" % name)
    src.write_text(text.replace(old, new), encoding="utf-8")
    lib = oracle.compile_source(str(src), str(tmp_path / ("libmutant_%s.so" % name)))
    caught = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "no pin caught the planted mistake %s" % name


# mistakes in the Python helper that maps flat rows of huge inputs to their heads (oracle/__init__.py)
PY_SRC = oracle.__file__
PY_MUTANTS = {
    "rows_kv_head_round_robin": ("_f64(k[b, h // grp])", "_f64(k[b, h % grp])"),
    "rows_first_batch_length_for_all": ("np.asarray([valid_lens[b]], dtype=np.int32)",
                                        "np.asarray([valid_lens[0]], dtype=np.int32)"),
    "rows_query_index_from_head": ("rows[sel] % Nq, mask=mask,", "(rows[sel] // H) % Nq, mask=mask,"),
    "rows_batch_head_swapped": ("b, h = divmod(int(bh), H)", "h, b = divmod(int(bh), B)"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_rows_helper_pin_catches_planted_mistake(name):
    old, new = PY_MUTANTS[name]
    text = open(PY_SRC, encoding="utf-8").read()
    assert text.count(old) == 1, "mutation site not found exactly once: %r" % old
    if name == "rows_batch_head_swapped":
        new = new.replace("B)", "q.shape[0])")
    mod = types.ModuleType("oracle_mutant_" + name)
    mod.__file__ = PY_SRC  # the altered helper still loads the real C oracle
    exec(compile(text.replace(old, new), PY_SRC, "exec"), mod.__dict__)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        pin_rows_per_head_equals_full(None, mod=mod)
