"""The pins are strong enough: a plausible mistake planted anywhere in the
oracle (a swapped nibble, a dropped clamp, a wrong bias, a transposed index)
makes at least one pin fail.

Each case copies ``oracle/oracle.c``, replaces one exact source fragment,
builds the copy with gcc into a temporary directory, points the oracle
binding at it and runs every pin. CPU only; nothing here touches the GPU.
"""
import os
import tempfile

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, fragment in oracle.c, planted replacement) or (name, [(fragment, replacement), ...])
MUTATIONS = [
    ("nibble_order_decode", "int c = (k & 1) ? (byte >> 4) : (byte & 15);",
     "int c = (k & 1) ? (byte & 15) : (byte >> 4);"),
    ("nibble_order_w13", "int cg = (k & 1) ? (bg >> 4) : (bg & 15);",
     "int cg = (k & 1) ? (bg & 15) : (bg >> 4);"),
    ("nibble_order_w2", "int c = (i & 1) ? (b >> 4) : (b & 15);",
     "int c = (i & 1) ? (b & 15) : (b >> 4);"),
    ("e2m1_exponent_bias", "(1.0 + 0.5 * m) * (double)(1 << (e - 1))", "(1.0 + 0.5 * m) * (double)(1 << e)"),
    ("e2m1_subnormal", "(e == 0) ? 0.5 * m", "(e == 0) ? 1.0 * m"),
    ("e8m0_bias", "ldexp(1.0, b - 127)", "ldexp(1.0, b - 128)"),
    ("scale_group_index", "double sg = or_e8m0(s13[(int64_t)i * (H / 32) + k0 / 32]);",
     "double sg = or_e8m0(s13[(int64_t)i * (H / 32) + ((k0 / 32) ^ 1)]);"),
    ("gate_up_swapped", "g += or_e2m1(cg) * sg * xd[k];\n        u += or_e2m1(cu) * su * xd[k];",
     "u += or_e2m1(cg) * sg * xd[k];\n        g += or_e2m1(cu) * su * xd[k];"),
    ("gate_not_clamped", "double gc = g < limit ? g : limit;", "double gc = g;"),
    ("gate_clamped_below", "double gc = g < limit ? g : limit;",
     "double gc = g < -limit ? -limit : (g < limit ? g : limit);"),
    ("up_not_clamped", "double uc = u < -limit ? -limit : (u > limit ? limit : u);", "double uc = u;"),
    ("silu_sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("score_no_sqrt", "return sqrt(or_softplus(logit));", "return or_softplus(logit);"),
    ("softplus_sign", "log1p(exp(-fabs(z)))", "log1p(exp(fabs(z)))"),
    ("bias_in_weights", "for (int j = 0; j < k; ++j) w[j] = scale * s[ids[j]] / sum;",
     "for (int j = 0; j < k; ++j) w[j] = scale * (s[ids[j]] + bias[ids[j]]) / sum;"),
    ("no_routed_scale", "for (int j = 0; j < k; ++j) w[j] = scale * s[ids[j]] / sum;",
     "for (int j = 0; j < k; ++j) w[j] = s[ids[j]] / sum;"),
    ("bias_ignored", "b[e] = (float)(s[e] + (double)bias[e]);", "b[e] = (float)s[e];"),
    ("topk_tie_to_higher_id", "if (best < 0 || b[e] > b[best]) best = e;",
     "if (best < 0 || b[e] >= b[best]) best = e;"),
    ("topk_ascending", "if (best < 0 || b[e] > b[best]) best = e;",
     "if (best < 0 || b[e] < b[best]) best = e;"),
    ("decision_in_fp64", [("float b[4096];", "double b[4096];"),
                          ("b[e] = (float)(s[e] + (double)bias[e]);", "b[e] = s[e] + (double)bias[e];"),
                          ("static int topk_desc(const float* b", "static int topk_desc(const double* b")]),
    ("offset_ignored", "if (offset) l += (double)offset[e];", "(void)offset;"),
    ("hash_uses_wrong_row", "tid2eid + (int64_t)tids[t] * k, scale,\n                     ids",
     "tid2eid + (int64_t)(tids[t] + 1) % V * k, scale,\n                     ids"),
    ("shared_up_scale_row", "u *= (double)s13[I + i];", "u *= (double)s13[i];"),
    ("shared_not_added", "out[(int64_t)r * H + n] += z[n];", "out[(int64_t)r * H + n] += 0.0 * z[n];"),
    ("shared_w2_transposed", "acc += (double)q2[(int64_t)n * I + i] * hbuf[i];",
     "acc += (double)q2[(int64_t)i * H + n % I] * hbuf[i];"),
    ("h_not_rounded", "hbuf[i] = round_h ? or_round_bf16(h) : h;", "hbuf[i] = h;"),
    ("bf16_round_truncates", "double q = nearbyint(ldexp(v, 8 - e));", "double q = trunc(ldexp(v, 8 - e));"),
    ("routed_weight_dropped", "for (int n = 0; n < H; ++n) out[n] += w[j] * y[n];",
     "for (int n = 0; n < H; ++n) out[n] += y[n];"),
    ("permute_unstable", "int32_t p = cursor[ids[i]]++;", "int32_t p = cursor[ids[i]]++; p = p;"
     " if (i % 2) { int32_t q = offsets[ids[i] + 1] - 1 - (p - offsets[ids[i]]); p = q; }"),
    ("block_bytes_no_scale", "return ((int64_t)bits * group + scale_bits) / 8;",
     "return ((int64_t)bits * group) / 8;"),
    ("force_ids_ignored", "for (int j = 0; j < k; ++j) ids[j] = force_ids[j];",
     "nxt = topk_desc(b, E, k, ids);"),
    ("force_weights_from_topk", "for (int j = 0; j < k; ++j) ids[j] = force_ids[j];",
     "int32_t tk[64]; topk_desc(b, E, k, tk); double st[64];"
     " for (int j = 0; j < k; ++j) st[j] = s[tk[j]];"
     " for (int j = 0; j < k; ++j) { ids[j] = force_ids[j]; s[ids[j]] = st[j]; }"),
    ("force_row_of_token", "force_ids ? force_ids + (int64_t)r * k : NULL",
     "force_ids ? force_ids + (int64_t)(t % n_rows) * k : NULL"),
    ("forward_hash_wrong_row", "tid2eid + (int64_t)tids[t] * k, scale, idr, wr);",
     "tid2eid + (int64_t)((tids[t] + 1) % V) * k, scale, idr, wr);"),
    ("forward_hash_row_of_output", "tid2eid + (int64_t)tids[t] * k, scale, idr, wr);",
     "tid2eid + (int64_t)tids[r] * k, scale, idr, wr);"),
    ("forward_hash_uses_bias", "tid2eid + (int64_t)tids[t] * k, scale, idr, wr);",
     "tid2eid + (int64_t)tids[t] * k, scale, idr, wr);"
     " for (int j = 0; j < k; ++j) wr[j] *= 1.0 + 0.5 * (double)bias[idr[j]];"),
    ("linear_input_group", "const uint16_t* xt = x + ((int64_t)t * groups + g) * K;",
     "const uint16_t* xt = x + (int64_t)t * groups * K;"),
    ("linear_weight_group", "const int8_t* row = q + ((int64_t)g * N + n) * K;",
     "const int8_t* row = q + (int64_t)n * K;"),
    ("fp16_exponent_bias", "else mag = ldexp(1.0 + f / 1024.0, e - 15);",
     "else mag = ldexp(1.0 + f / 1024.0, e - 16);"),
    ("fp16_subnormal", "else if (e == 0) mag = ldexp((double)f, -24);",
     "else if (e == 0) mag = ldexp((double)f, -25);"),
    ("q3_code_half_shift", "int shift = (i % 8 < 4) ? 0 : 3;", "int shift = (i % 8 < 4) ? 3 : 0;"),
    ("q3_code_byte", "int byte = 4 * (i / 8) + i % 4;", "int byte = 4 * (i / 8) + (i % 8) / 2;"),
    ("q3_top_codes_swapped", "if (i < 28) return ((b[j] >> 6) & 3)",
     "if (i >= 28) return ((b[j] >> 6) & 3)"),
    ("q3_high_bit", "if (i < 28) return ((b[j] >> 6) & 3) | (((b[8 + j] >> 6) & 1) << 2);",
     "if (i < 28) return ((b[j] >> 6) & 3) | (((b[8 + j] >> 7) & 1) << 2);"),
    ("q3_uniform_offset", "return levels ? (double)levels[c] : (double)(c - 4);",
     "return levels ? (double)levels[c] : (double)(c - 3);"),
    ("q3_table_not_per_expert", "a->w2lv ? a->w2lv + (int64_t)e * 8 : NULL", "a->w2lv ? a->w2lv : NULL"),
    ("q3_scale_of_block", "double d = or_fp16_value(s2q3[(int64_t)n * (I / 32) + i0 / 32]);",
     "double d = or_fp16_value(s2q3[(int64_t)n * (I / 32) + (i0 / 32) / 2 * 2]);"),
    ("q3_expert_stride", "a->w2c + (int64_t)e * H * (I / 32) * 12, NULL",
     "a->w2c + (int64_t)e * H * (I / 2), NULL"),
    ("q3_weight_row_stride", "const uint8_t* blk = codes + (n * (K / 32) + k / 32) * 12;",
     "const uint8_t* blk = codes + (n * (K / 32) + k / 32) * 12 + (n > 0 ? 12 : 0);"),
    ("linear_scale_row", "out[((int64_t)t * groups + g) * N + n] = (double)s[(int64_t)g * N + n] * acc;",
     "out[((int64_t)t * groups + g) * N + n] = (double)s[n] * acc;"),
]


def _edits(m):
    return m[1] if isinstance(m[1], list) else [(m[1], m[2])]


def test_every_fragment_exists():
    src = open(SRC).read()
    for m in MUTATIONS:
        for old, _new in _edits(m):
            assert src.count(old) >= 1, f"{m[0]}: fragment not found in oracle.c"


@pytest.mark.parametrize("m", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(m, tmp_path):
    name = m[0]
    src = open(SRC).read()
    mutated = src
    for old, new in _edits(m):
        mutated = mutated.replace(old, new, 1)
    assert mutated != src
    csrc = tmp_path / "oracle_mut.c"
    csrc.write_text(mutated)
    so = str(tmp_path / "liboracle_mut.so")
    oracle.build(src=str(csrc), out=so)
    failed = []
    try:
        oracle.use_library(so)
        for check in oracle_pins.ALL_CHECKS:
            try:
                check()
            except (AssertionError, ValueError, IndexError):
                failed.append(check.__name__)
    finally:
        oracle.use_library(None)
    assert failed, f"planted mistake {name!r} passed every pin"
