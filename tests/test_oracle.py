"""The fp64 oracle against its pins, and the pins against planted mistakes (CPU only)."""
import os
import shutil

import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.default())


# Plausible mistakes planted in a copy of the oracle source: (name, original text, replacement).
# Each must make at least one pin fail; none reads or writes out of bounds.
MUTATIONS = [
    ("dropped_scale", "p[j] = c->scale * dot_bf16(", "p[j] = dot_bf16("),
    ("causal_sees_next_key", "static int last_key(const ctx_t* c, int i) { return c->causal ? i : c->S - 1; }",
     "static int last_key(const ctx_t* c, int i) { return c->causal ? (i + 1 < c->S ? i + 1 : i) : c->S - 1; }"),
    ("window_one_too_wide", "return (c->window > 0 && i - c->window + 1 > 0) ? i - c->window + 1 : 0;",
     "return (c->window > 0 && i - c->window > 0) ? i - c->window : 0;"),
    ("window_key_side_one_too_wide", "return (c->window > 0 && j + c->window - 1 < c->S - 1) ? j + c->window - 1 : c->S - 1;",
     "return (c->window > 0 && j + c->window < c->S - 1) ? j + c->window : c->S - 1;"),
    ("gqa_interleaved_map", "j1 = last_key(c, i), hkv = hq / c->G;", "j1 = last_key(c, i), hkv = hq % c->Hkv;"),
    ("lse_log2", "if (lse_out) *lse_out = m + log(l);\n    if (o_out) {\n        for (int d",
     "if (lse_out) *lse_out = m + log2(l);\n    if (o_out) {\n        for (int d"),
    ("unnormalised_p", "for (int j = j0; j <= j1; ++j) p[j] /= l;", ""),
    ("ds_sign_flipped", "const double ds = p[j] * (dp[j] - delta);",
     "const double ds = p[j] * (delta - dp[j]);"),
    ("dp_uses_k_not_v", "dp[j] = dot_bf16(doi, c->v + kvrow_off", "dp[j] = dot_bf16(doi, c->k + kvrow_off"),
    ("dq_missing_scale", "kvrow_off(c, b, hkv, j, D);\n                for (int d = 0; d < D; ++d) dq_out[d] += c->scale",
     "kvrow_off(c, b, hkv, j, D);\n                for (int d = 0; d < D; ++d) dq_out[d] += 1.0"),
    ("dk_missing_scale", "for (int d = 0; d < D; ++d) dk_out[d] += c->scale * ds * widen(qi[d]);",
     "for (int d = 0; d < D; ++d) dk_out[d] += ds * widen(qi[d]);"),
    ("dk_dv_first_head_only", "    for (int g = 0; g < c->G; ++g) {\n        const int hq = hkv * c->G + g;\n        for (int i",
     "    for (int g = 0; g < 1; ++g) {\n        const int hq = hkv * c->G + g;\n        for (int i"),
    ("dv_weighted_by_ds", "for (int d = 0; d < Dv; ++d) dv_out[d] += pij * widen(doi[d]);",
     "for (int d = 0; d < Dv; ++d) dv_out[d] += ds * widen(doi[d]);"),
    ("delta_missing_p", "delta += p[j] * dp[j];", "delta += dp[j];"),
    # value width d_v != d: each of these stays in bounds while Dv > D, and the
    # d_v pin runs all its Dv > D cases before any Dv < D one
    ("o_uses_d_columns", "for (int d = 0; d < Dv; ++d) o_out[d] += p[j] * widen(vj[d]);",
     "for (int d = 0; d < D; ++d) o_out[d] += p[j] * widen(vj[d]);"),
    ("v_row_stride_d", "dp[j] = dot_bf16(doi, c->v + kvrow_off(c, b, hkv, j, Dv), Dv);",
     "dp[j] = dot_bf16(doi, c->v + kvrow_off(c, b, hkv, j, D), Dv);"),
    ("dv_uses_d_columns", "for (int d = 0; d < Dv; ++d) dv_out[d] += pij * widen(doi[d]);",
     "for (int d = 0; d < D; ++d) dv_out[d] += pij * widen(doi[d]);"),
    ("dp_dot_over_d", "const double dpij = dot_bf16(doi, vj, Dv);", "const double dpij = dot_bf16(doi, vj, D);"),
    # sparse (index-list) attention
    ("sparse_gqa_interleaved_map", "const int D = c->D, hkv = hq / c->G;", "const int D = c->D, hkv = hq % c->Hkv;"),
    ("sparse_empty_slot_is_row_0", "return (j >= 0 && j < c->N) ? (int)j : -1;",
     "return j < c->N ? (j < 0 ? 0 : (int)j) : -1;"),
    ("sparse_lse_without_max", "if (lse_out) *lse_out = m + log(l);\n    if (o_out) {\n        for (int s",
     "if (lse_out) *lse_out = log(l);\n    if (o_out) {\n        for (int s"),
    ("sparse_inverse_map_first_entry_only", "for (int64_t e = 0; e < ne; ++e) {",
     "for (int64_t e = 0; e < (ne > 0 ? 1 : 0); ++e) {"),
    ("sparse_dk_dv_first_head_only", "        for (int g = 0; g < c->G; ++g) {\n            const int hq = hkv * c->G + g;\n            const size_t r",
     "        for (int g = 0; g < 1; ++g) {\n            const int hq = hkv * c->G + g;\n            const size_t r"),
    ("sparse_dv_weighted_by_ds", "                dv_out[d] += pij * widen(doi[d]);", "                dv_out[d] += ds * widen(doi[d]);"),
    ("sparse_dq_missing_scale", "skv_row(c, c->k, b, hkv, j);\n                for (int d = 0; d < D; ++d) dq_out[d] += c->scale",
     "skv_row(c, c->k, b, hkv, j);\n                for (int d = 0; d < D; ++d) dq_out[d] += 1.0"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    mutated = tmp_path / ("oracle_%s.c" % name)
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(src=str(mutated), out=str(tmp_path / ("liboracle_%s.so" % name)))
    broken = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(broken)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "planted mistake %s passed every pin" % name
