"""Plant plausible mistakes in a copy of the oracle (on the CPU) and require
that at least one pin in oracle_pins.py catches each of them.

The oracle source itself is never modified: each mutant is a text substitution
applied to a temporary copy, built with the same gcc command into a temporary
library and swapped in for the duration of the checks.
"""
import shutil

import pytest

import oracle
import oracle_pins

# (name, exact text in attn_oracle.c, replacement)
MUTANTS = [
    ("dropped_scale", "S[i * nk + j] = scale * acc;", "S[i * nk + j] = acc;"),
    ("mask_off_by_one", "int64_t lim = nk - nq + i + 1;", "int64_t lim = nk - nq + i;"),
    ("top_left_causal", "int64_t lim = nk - nq + i + 1;", "int64_t lim = i + 1;"),
    ("wrong_k_channel", "acc += Q[i * d + c] * K[j * d + c];", "acc += Q[i * d + c] * K[j * d + (d - 1 - c)];"),
    ("softmax_sign", "P[i * nk + j] = exp(S[i * nk + j] - m) / l;", "P[i * nk + j] = exp(m - S[i * nk + j]) / l;"),
    ("no_normalisation", "P[i * nk + j] = exp(S[i * nk + j] - m) / l;", "P[i * nk + j] = exp(S[i * nk + j] - m);"),
    ("lse_without_max", "if (LSE) LSE[i] = m + log(l);", "if (LSE) LSE[i] = log(l);"),
    ("pv_wrong_row", "acc += P[i * nk + j] * V[j * d + c];", "acc += P[i * nk + j] * V[(nk - 1 - j) * d + c];"),
    ("gather_k_reads_v", "K[t * d + c] = elem(pool, dtype, pool_index(pb, 0, h, off, c, H, bs, d));",
     "K[t * d + c] = elem(pool, dtype, pool_index(pb, 1, h, off, c, H, bs, d));"),
    ("gather_wrong_offset", "int off = (int)(t % bs);\n        if (lb >= maxb) return ORACLE_ERR_TABLE;\n        int64_t pb = table[(int64_t)r * maxb + lb];\n        if (pb < 0 || pb >= num_blocks) return ORACLE_ERR_TABLE;\n        for (int c = 0; c < d; ++c) {",
     "int off = (int)((bs - 1 - t % bs));\n        if (lb >= maxb) return ORACLE_ERR_TABLE;\n        int64_t pb = table[(int64_t)r * maxb + lb];\n        if (pb < 0 || pb >= num_blocks) return ORACLE_ERR_TABLE;\n        for (int c = 0; c < d; ++c) {"),
    ("pool_layout_head_major", "return (((pb * 2 + kv) * H + h) * bs + off) * (int64_t)d + c;",
     "return (((pb * H + h) * 2 + kv) * bs + off) * (int64_t)d + c;"),
    ("tiled_no_rescale", "for (int c = 0; c < d; ++c) o[i * d + c] *= alpha;", ""),
    ("tiled_sum_not_rescaled", "l[i] = alpha * l[i] + psum;", "l[i] = l[i] + psum;"),
    ("merge_uses_max", "acc += exp(lse_parts[s] - L) * o_parts[(int64_t)s * d + c];",
     "acc += exp(lse_parts[s] - M) * o_parts[(int64_t)s * d + c];"),
    ("bf16_low_half", "uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]) << 16;",
     "uint32_t bits = ((uint32_t)((const uint16_t*)base)[idx]);"),
    ("prefix_skips_request", "for (int i = 0; i < r; ++i) s += q_lens[i];", "for (int i = 1; i < r; ++i) s += q_lens[i];"),
    ("gqa_strided_groups", "static int kv_head(int h, int H, int Hkv) { return h / (H / Hkv); }",
     "static int kv_head(int h, int H, int Hkv) { return h % Hkv; }"),
    # backward
    ("bwd_dq_unscaled", "dQ[c] = scale * acc;", "dQ[c] = acc;"),
    ("bwd_ds_sign", "for (int64_t j = 0; j < nk; ++j) ds[j] = p[j] * (ds[j] - D);",
     "for (int64_t j = 0; j < nk; ++j) ds[j] = p[j] * (D - ds[j]);"),
    ("bwd_ds_without_row_term", "for (int64_t j = 0; j < nk; ++j) ds[j] = p[j] * (ds[j] - D);",
     "for (int64_t j = 0; j < nk; ++j) ds[j] = p[j] * ds[j];"),
    ("bwd_dp_reads_k", "for (int c = 0; c < d; ++c) acc += doi[c] * V[j * d + c];",
     "for (int c = 0; c < d; ++c) acc += doi[c] * K[j * d + c];"),
    ("bwd_dv_uses_ds", "dV[j * d + c] += p[j] * doi[c];", "dV[j * d + c] += ds[j] * doi[c];"),
    ("bwd_dk_wrong_operand", "dK[j * d + c] += scale * ds[j] * qi[c];", "dK[j * d + c] += scale * ds[j] * doi[c];"),
    ("bwd_dk_unscaled", "dK[j * d + c] += scale * ds[j] * qi[c];", "dK[j * d + c] += ds[j] * qi[c];"),
    ("bwd_dq_transposed", "for (int64_t j = 0; j < Nk; ++j) acc += ds[j] * K[j * d + c];\n                        dQ[c]",
     "for (int64_t j = 0; j < Nk; ++j) acc += ds[j] * V[j * d + c];\n                        dQ[c]"),
    ("bwd_group_strided", "const int64_t bh = b * H + hk * G + gh;", "const int64_t bh = b * H + gh * Hkv + hk;"),
    ("bwd_group_not_summed", "for (int gh = 0; gh < G; ++gh) {\n                const int64_t bh = b * H",
     "for (int gh = 0; gh < G; ++gh) {\n                for (int64_t x = 0; x < (int64_t)Nk * d; ++x) "
     "dK[x] = dV[x] = 0.0;\n                const int64_t bh = b * H"),
    ("bwd_rows_dq_unscaled", "dq_rows[(int64_t)s * d + c] = scale * acc;", "dq_rows[(int64_t)s * d + c] = acc;"),
    ("bwd_rows_dv_operand", "acc_v[c] += p[j] * doi[c];", "acc_v[c] += p[j] * qi[c];"),
    ("bwd_rows_wrong_group_head", "const int64_t bh = (int64_t)kb[s] * H + (int64_t)khk[s] * G + gh;",
     "const int64_t bh = (int64_t)kb[s] * H + (int64_t)khk[s] + gh;"),
    ("bwd_rows_last_thread_dropped", "for (int t = 0; t < nthr; ++t) {\n                sk",
     "for (int t = 0; t + 1 < nthr; ++t) {\n                sk"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = oracle._SRC.read_text()
    assert src.count(old) == 1, "mutation anchor for %s not unique/present" % name
    mutated = tmp_path / "attn_oracle_mutant.c"
    mutated.write_text(src.replace(old, new))
    lib_path = oracle.build(src=mutated, out=tmp_path / "liboracle_mutant.so")
    saved = oracle._lib
    oracle._lib = oracle.load(lib_path)
    caught = []
    try:
        for check in oracle_pins.ALL_CHECKS:
            try:
                check()
            except (AssertionError, RuntimeError) as e:  # a pin fired
                caught.append(check.__name__)
    finally:
        oracle._lib = saved
        shutil.rmtree(tmp_path, ignore_errors=True)
    assert caught, "mutant %s survived every pin" % name
