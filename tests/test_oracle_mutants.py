"""Plant plausible mistakes in copies of the oracle and check that the pins catch each one.

Each mutant is oracle.c with one textual change (a dropped term, a wrong sign or index, a
transposed operand, a wrong tie-break or rounding).  It is compiled to a private library and the
pin suite (tests/test_oracle_pins.py) runs against it in a subprocess; the suite must fail.
CPU only; nothing here touches the product path.
"""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "route_tie_to_higher_id": ("v[e] > v[best]) best = e;", "v[e] >= v[best]) best = e;"),
    "route_softmax_drops_last_term": ("        sum += z[k];", "        if (k + 1 < R) sum += z[k];"),
    "route_bias_sign": ("l + bias[e]", "l - bias[e]"),
    "send_scan_not_cumulative": ("off[d + 1] = off[d] + n;", "off[d + 1] = n;"),
    "send_owner_modulo": ("int d = e / L;\n                long pos", "int d = e % N;\n                long pos"),
    "send_meta_drops_slot": ("meta[0] = (int32_t)((long)e * TR + i);", "meta[0] = (int32_t)((long)e * TR + t * R);"),
    "send_meta_rank_off_by_one": ("meta[1] = seen[e];", "meta[1] = seen[e] + 1;"),
    "net_offsets_transposed": ("roff[s + 1] = roff[s] + (soff[d + 1] - soff[d]);",
                               "roff[s + 1] = roff[s] + (soff[s + 1] - soff[s]);"),
    "recv_src_uses_dest_rank": ("expert_src[rrow0(sh, d) + q] = (int32_t)((long)s * TR + i);",
                                "expert_src[rrow0(sh, d) + q] = (int32_t)((long)d * TR + i);"),
    "recv_expert_off_not_scanned": ("eoff[j + 1] = eoff[j] + c;", "eoff[j + 1] = c;"),
    "expert_tag_local_id": ("(double)(64 + e % 64) / 64.0", "(double)(64 + j % 64) / 64.0"),
    "combine_shuffle_inverted": (
        "memcpy(cs_buf + (rrow0(sh, d) + r) * H, expert_y + (rrow0(sh, d) + q) * H, 2L * H);",
        "memcpy(cs_buf + (rrow0(sh, d) + q) * H, expert_y + (rrow0(sh, d) + r) * H, 2L * H);"),
    "combine_net_offsets_transposed": ("long src = rrow0(sh, d) + recv_off[(long)d * (N + 1) + s];",
                                       "long src = rrow0(sh, d) + recv_off[(long)s * (N + 1) + d];"),
    "combine_weight_of_slot0": ("acc += (double)topk_w[base + k] * y;", "acc += (double)topk_w[base] * y;"),
    "combine_drops_last_slot": ("for (int k = 0; k < R; ++k) {\n                    long row",
                                "for (int k = 0; k < R - 1; ++k) {\n                    long row"),
    "acc_sums_every_slot": ("                    if (!is_first) continue;\n", ""),
    "acc_group_weight_of_first_row": ("if (mode == 0) acc += (double)topk_w[si] * y;\n                    else accf = fmaf(topk_w[si], (float)y, accf);",
                                      "if (mode == 0) acc += (double)topk_w[si - i] * y;\n                    else accf = fmaf(topk_w[si - i], (float)y, accf);"),
    "acc_rows_never_grouped": ("while (r + c < total && expert_src[rrow0(sh, d) + qof[r + c]] / R == tok) ++c;",
                               "while (0) ++c;"),
    "acc_net_sends_other_rows": ("if (!first[d][r0 + i]) continue;", "if (first[d][r0 + i] && i > 0) continue;"),
    "bf16_truncates": ("double q = nearbyint(ldexp(a, -ulp_exp));", "double q = floor(ldexp(a, -ulp_exp));"),
    "bf16_one_bit_short": ("int ulp_exp = ex - 8;", "int ulp_exp = ex - 7;"),
    "e4m3_wrong_bias": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 9)"),
    "quant_scale_fnuz_max": ("amax / 448.0f", "amax / 240.0f"),
    "quant_ties_away_from_zero": ("double r = ldexp(nearbyint(ldexp(a, -sp)), sp);",
                                  "double r = ldexp(round(ldexp(a, -sp)), sp);"),
    "quant_truncates": ("double r = ldexp(nearbyint(ldexp(a, -sp)), sp);",
                        "double r = ldexp(floor(ldexp(a, -sp)), sp);"),
    "quant_no_saturation": ("if (r > 448.0) r = 448.0;", ""),
    "quant_subnormal_spacing": ("? ex - 1 - 3 : -9;", "? ex - 1 - 3 : -10;"),
    "quant_two_mantissa_bits": ("? ex - 1 - 3 : -9;", "? ex - 1 - 2 : -9;"),
    "quant_amax_signed": ("float a = fabsf((float)oracle_bf16_to_double(xb[i]));",
                          "float a = (float)oracle_bf16_to_double(xb[i]);"),
    "send_counts_absent_tokens": ("for (long i = 0; i < (long)Ts * R; ++i) {",
                                  "for (long i = 0; i < TR; ++i) {"),
    "send_packs_absent_tokens": ("for (int t = 0; t < Ts; ++t) {", "for (int t = 0; t < T; ++t) {"),
    "prefill_src_transposed": ("expert_src[row] = t * R + k;", "expert_src[row] = k * T + t;"),
    "prefill_owner_modulo": ("if (topk_idx[i] / L != d) continue;", "if (topk_idx[i] % N != d) continue;"),
    "prefill_local_ignores_weight": ("else accf = fmaf(topk_w[i], (float)y, accf);",
                                     "else accf = fmaf(1.0f, (float)y, accf);"),
    "prefill_allreduce_reversed": ("for (int d = 0; d < N; ++d) s = s + partial",
                                   "for (int d = N - 1; d >= 0; --d) s = s + partial"),
    "prefill_allreduce_drops_rank": ("for (int d = 0; d < N; ++d) s = s + partial",
                                     "for (int d = 1; d < N; ++d) s = s + partial"),
    "prefill_sum_weight_of_slot0": ("                    acc += (double)topk_w[i] *\n",
                                    "                    acc += (double)topk_w[(long)t * R] *\n"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not unique"
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "oracle.c")
        with open(c, "w") as f:
            f.write(src.replace(before, after))
        with open(os.path.join(tmp, "oracle.h"), "w") as f:
            f.write(open(os.path.join(ROOT, "oracle", "oracle.h")).read())
        so = os.path.join(tmp, "liboracle.so")
        subprocess.check_call(["gcc", *oracle.CFLAGS, c, "-o", so, "-lm"])
        env = dict(os.environ, MOE_ORACLE_LIB=so)
        p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            "-k", "not groupgemm and not qwen_prefill and not receive_bound",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
        assert p.returncode != 0, f"mutant {name} survived the pins:\n{p.stdout[-2000:]}"
