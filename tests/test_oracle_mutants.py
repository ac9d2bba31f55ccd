"""Planted mistakes in copies of the oracle must each fail at least one pin (CPU only).

Each mutant is oracle.c with one plausible slip (a dropped term, a wrong sign or index,
a transposed operand), compiled to a temporary library and run through every check in
tests/_pins.py.  A mutant that passes them all would mean the pins cannot see that
class of mistake.
"""
import os

import pytest

import oracle as O
from oracle.build import SRC, build_oracle
from tests import _pins

MUTANTS = {
    "gqa_interleaved_heads": ("int kvh = h / group;", "int kvh = h % A->hkv;"),
    "scale_dropped": ("J->scores[t] = J->scale * dot;", "J->scores[t] = dot;"),
    "v_read_token_major": (
        "size_t idx = ((phys * P->hkv + P->kv_head) * P->d + e) * ORACLE_BLOCK + off;",
        "size_t idx = ((phys * P->hkv + P->kv_head) * ORACLE_BLOCK + off) * P->d + e;"),
    "k_row_off_by_one": (
        "size_t off = (size_t)(t % ORACLE_BLOCK);\n    size_t idx = ((phys * P->hkv + P->kv_head) * ORACLE_BLOCK",
        "size_t off = (size_t)((t + 1) % ORACLE_BLOCK);\n    size_t idx = ((phys * P->hkv + P->kv_head) * ORACLE_BLOCK"),
    "exp_sign_flipped": ("J->scores[t] = exp(J->scores[t] - m);",
                         "J->scores[t] = exp(m - J->scores[t]);"),
    "final_divide_dropped": ("out[e] = acc / z;", "out[e] = acc;"),
    "block_index_uses_offset": (
        "size_t phys = (size_t)P->table_row[t / ORACLE_BLOCK];\n    size_t off = (size_t)(t % ORACLE_BLOCK);\n    size_t idx = ((phys * P->hkv + P->kv_head) * P->d",
        "size_t phys = (size_t)P->table_row[t % P->hkv];\n    size_t off = (size_t)(t % ORACLE_BLOCK);\n    size_t idx = ((phys * P->hkv + P->kv_head) * P->d"),
    "f16_exponent_bias": ("v = ldexp((double)(frac | 0x400), expo - 25);",
                          "v = ldexp((double)(frac | 0x400), expo - 24);"),
    "bf16_shift": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    "append_row_col_swapped": (
        "size_t vdst = ((blk * num_kv_heads + h) * head_dim + e) * ORACLE_BLOCK + off;",
        "size_t vdst = ((blk * num_kv_heads + h) * ORACLE_BLOCK + off) * head_dim + e;"),
    "kv_size_factor_dropped": ("return 2ull * layers * kv_heads", "return layers * kv_heads"),
    "max_over_first_token_only": ("if (J->scores[t] > m)", "if (t == 0)"),
    "weight_sum_unnormalised": ("s += J->scores[t] / z;", "s += J->scores[t];"),
    "e4m3_exponent_bias": ("v = ldexp((double)(frac | 0x8), expo - 10);",
                           "v = ldexp((double)(frac | 0x8), expo - 9);"),
    "e4m3_subnormal_step": ("v = ldexp((double)frac, -9);", "v = ldexp((double)frac, -8);"),
    "e4m3_encode_truncates": ("float steps = rintf(ldexpf(a, 3 - k));",
                              "float steps = floorf(ldexpf(a, 3 - k));"),
    "e4m3_encode_no_saturation": ("if (a >= 448.0f)\n        return sign | 0x7e;",
                                  "if (a >= 448.0f)\n        return sign | 0x7f;"),
    "fp8_k_scale_dropped": ("return widen_at(P->k_pool, idx, P->dtype) * P->k_scale;",
                            "return widen_at(P->k_pool, idx, P->dtype);"),
    "fp8_append_scale_multiplied": ("encode_e4m3(vx / vs)", "encode_e4m3(vx * vs)"),
    "fp8_head_scale_of_first_head": (
        "double ks = A->k_head_scales ? (double)A->k_head_scales[kvh] : A->k_scale;",
        "double ks = A->k_head_scales ? (double)A->k_head_scales[0] : A->k_scale;"),
    "fp8_v_head_scale_from_k": (
        "double vs = A->v_head_scales ? (double)A->v_head_scales[kvh] : A->v_scale;",
        "double vs = A->v_head_scales ? (double)A->k_head_scales[kvh] : A->v_scale;"),
    "fp8_append_head_scale_of_next_head": (
        "float ks = k_head_scales ? k_head_scales[h] : k_scale;",
        "float ks = k_head_scales ? k_head_scales[(h + 1) % num_kv_heads] : k_scale;"),
    "fp8_bad_head_scale_not_poisoned": ("if (!scale_ok(ks) || !scale_ok(vs)) {", "if (0) {"),
    "prefill_causal_mask_dropped": ("n = pos < 0 ? 0 : pos + 1;", "n = pos < 0 ? 0 : n;"),
    "prefill_own_token_excluded": ("n = pos < 0 ? 0 : pos + 1;", "n = pos < 0 ? 0 : pos;"),
    "prefill_upper_left_alignment": ("int pos = n - q_len + (r - A->q_start[b]);",
                                     "int pos = r - A->q_start[b];"),
    "prefill_q_row_of_sequence": ("J.q_row = (const char *)A->q + ((size_t)r * A->hq + h)",
                                  "J.q_row = (const char *)A->q + ((size_t)b * A->hq + h)"),
    "prefill_owner_off_by_one": ("if (q_start[mid] <= tok)", "if (q_start[mid] < tok)"),
    "copy_v_block_skipped": (
        "        memmove((char *)v_pool + (size_t)dst * bytes, (const char *)v_pool + (size_t)src * bytes,\n                bytes);\n",
        ""),
    "copy_to_source": ("memmove((char *)k_pool + (size_t)dst * bytes, (const char *)k_pool + (size_t)src * bytes,",
                       "memmove((char *)k_pool + (size_t)src * bytes, (const char *)k_pool + (size_t)dst * bytes,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in oracle.c"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib_path = build_oracle(str(mutated), str(tmp_path / f"lib_{name}.so"))
    lib = O.load(lib_path)
    failures = []
    for check in _pins.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, ValueError) as exc:
            failures.append(check.__name__)
    assert failures, f"mutant {name} passed every pin"
