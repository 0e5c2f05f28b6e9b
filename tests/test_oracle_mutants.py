"""Do the oracle's pins catch plausible mistakes?  Each case plants one
mistake in a temporary copy of oracle.c (never in the file itself), builds
it, and runs the pin suite against it: the suite must fail.

Opt-in (about five minutes on 8 cores): set SPA_ORACLE_MUTANTS=1."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "gqa_mapping": ("int kvh = h / (a->Hq / a->Hkv);\n    double acc = 0.0;",
                    "int kvh = h % a->Hkv;\n    double acc = 0.0;"),
    "dropped_scale": ("return a->scale * acc;", "return acc;"),
    "row_off_by_one": ("int64_t row = page * a->P + (t % a->P);",
                       "int64_t row = page * a->P + ((t + 1) % a->P);"),
    "page_index": ("a->page_table_stride + t / a->P];", "a->page_table_stride + (t + 1) / a->P];"),
    "lse_base2": ("lse[bh] = m + log(l);", "lse[bh] = m + log2(l);"),
    "mask_off_by_one": ("attend_range(&a, b, h, 0, seq_lens[b], &m, &l, o);",
                        "attend_range(&a, b, h, 0, seq_lens[b] + 1, &m, &l, o);"),
    "merge_weight_sign": ("double w = exp(mj[j] - M);", "double w = exp(M - mj[j]);"),
    "split_bound": ("int p0 = j * pps, p1 = (j + 1) * pps;",
                    "int p0 = j * pps, p1 = (j + 1) * pps + 1;"),
    "truncating_division": ("if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;", ""),
    "cu_seqlens_k0": ("cu_seqlens_k[0] = 0;", ""),
    "kv_index": ("int64_t idx = (row * a->Hkv + kvh) * a->D + d;",
                 "int64_t idx = (row * a->Hkv + (kvh + d) % a->Hkv) * a->D + (d + kvh) % a->D;"),
    "int8_value_scale": ("const float *sc = which ? a->v_scales : a->k_scales;",
                         "const float *sc = a->k_scales;"),
    "dropped_offset": ("(uint32_t)seq_lens[i] + (uint32_t)seqlen_offset", "(uint32_t)seq_lens[i]"),
    "strided_q_from_zero": ("(uint64_t)(i + 1) * (uint64_t)(uint32_t)q_stride",
                            "(uint64_t)i * (uint64_t)(uint32_t)q_stride"),
    "cumsum_q_exclusive": ("run += (uint32_t)qlens[i];\n            cu_seqlens_q[i + 1] = (int32_t)run;",
                           "cu_seqlens_q[i + 1] = (int32_t)run;\n            run += (uint32_t)qlens[i];"),
    "swa_no_sentinel": ("(int32_t)(v < 0 ? -1 : floor_div(v, page_size));",
                        "(int32_t)floor_div(v, page_size);"),
    "swa_padding_minus_one": ("swa_out_cache_loc[k] = 0;", "swa_out_cache_loc[k] = -1;"),
    "swa_out_untranslated": ("swa_out_cache_loc[k] = loc < 0 ? -1 : swa[loc];",
                             "swa_out_cache_loc[k] = loc;"),
    "fp8_exponent_bias": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "fp8_subnormal_as_normal": ("e == 0 ? ldexp(m / 8.0, -6)", "e == 0 ? ldexp(1.0 + m / 8.0, -7)"),
    "fp8_sign_dropped": ("return sign ? -v : v;", "return v;"),
    "fp8_scale_dropped": ("return e4m3_to_double(base[idx]) * sigma;",
                          "return e4m3_to_double(base[idx]);"),
    "verify_causal_off_by_one": ("visible = seq_lens[b] - nq + i + 1;",
                                 "visible = seq_lens[b] - nq + i;"),
    "verify_not_causal": ("visible = seq_lens[b] - nq + i + 1;", "visible = seq_lens[b];"),
    "verify_query_row": ("a.q_row = row;", "a.q_row = cu_seqlens_q[b < 0 ? 0 : b];"),
    "swa_num_out_max": ("n_out_cache_loc < swa_out_len ? n_out_cache_loc : swa_out_len",
                        "n_out_cache_loc > swa_out_len ? swa_out_len : swa_out_len"),
}

pytestmark = pytest.mark.skipif(os.environ.get("SPA_ORACLE_MUTANTS") != "1",
                                reason="opt-in: SPA_ORACLE_MUTANTS=1")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_fail_on_planted_mistake(name, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    a, b = MUTANTS[name]
    assert a in src, "mutation anchor no longer in oracle.c"
    mut_c = tmp_path / "oracle_mut.c"
    mut_c.write_text(src.replace(a, b))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", str(lib),
                    str(mut_c), "-lm"], check=True)
    env = dict(os.environ, SPA_ORACLE_LIB=str(lib))
    env.pop("SPA_ORACLE_MUTANTS", None)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    assert r.returncode != 0, f"pins did not catch mutant {name}"
