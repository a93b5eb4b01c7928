"""The oracle's pins catch plausible slips: each mutant fails at least one pin.

Every case below plants one mistake in a temporary copy of ``fa_oracle.c``
(on the CPU, never on a GPU), builds it, and runs ``test_oracle_pins.py``
against that build.  A mutant that passes every pin would mean the pins leave
that part of the oracle unchecked.
"""
import os
import shutil
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
SRC = ROOT / "oracle" / "fa_oracle.c"

MUTANTS = {
    "causal_off_by_one": ("J->causal ? i + 1 + (Nk - Nq) : Nk", "J->causal ? i + (Nk - Nq) : Nk"),
    "causal_offset_sign": ("J->causal ? i + 1 + (Nk - Nq) : Nk",
                           "J->causal ? i + 1 - (Nk - Nq) : Nk"),
    "dropped_scale": ("s[j] = J->scale * dot;", "s[j] = dot;"),
    "key_row_index": ("qi[c] * load_elem(J->k, J->dtype, kvhead + j * d + c)",
                      "qi[c] * load_elem(J->k, J->dtype, kvhead + i * d + c)"),
    "value_row_index": ("o_out[c] += p * load_elem(J->v, J->dtype, kvhead + j * d + c)",
                        "o_out[c] += p * load_elem(J->v, J->dtype, kvhead + i * d + c)"),
    "transposed_query": ("(c = 0; c < d; ++c) qi[c] = load_elem(J->q, J->dtype, qhead + i * d + c)",
                         "(c = 0; c < d; ++c) qi[c] = load_elem(J->q, J->dtype, qhead + c * Nq + i)"),
    "dropped_normalisation": ("double p = exp(s[j] - m) / l;", "double p = exp(s[j] - m);"),
    "lse_sign": ("*lse_out = m + log(l);", "*lse_out = m - log(l);"),
    "lse_dropped_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "head_offset": ("const int64_t qhead = bh * Nq * d;", "const int64_t qhead = bh * d;"),
    "kv_head_offset": ("(b * J->Hkv + kvh) * Nk * d;", "(b * J->Hkv + kvh) * d;"),
    "grouped_head_map": ("const int64_t kvh = h / (J->H / J->Hkv);",
                         "const int64_t kvh = h % J->Hkv;"),
    "max_not_subtracted_in_sum": ("l += exp(s[j] - m);", "l += exp(s[j]);"),
    "f16_bias": ("expo - 15);", "expo - 16);"),
    "f16_subnormal": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "bf16_shift": ("(uint32_t)bits << 16;", "(uint32_t)bits << 15;"),
    "max_uses_min": ("if (s[j] > m) m = s[j];", "if (s[j] < m || m == -INFINITY) m = s[j];"),
    "combine_max_uses_min": ("const double m_new = mt > m ? mt : m;",
                             "const double m_new = mt < m ? mt : m;"),
    "combine_weight_sign": ("a_new = lt * exp(mt - m_new)", "a_new = lt * exp(m_new - mt)"),
    "combine_dropped_old_scale": ("(a_old * out[c] + a_new * ot[c]) / l_new",
                                  "(out[c] + a_new * ot[c]) / l_new"),
    "combine_lse_sign": ("lse[r] = l > 0.0 ? m + log(l)", "lse[r] = l > 0.0 ? m - log(l)"),
    "bwd_dropped_row_dot": ("ds[j] = p[j] * (dp - D);", "ds[j] = p[j] * dp;"),
    "bwd_dk_from_keys": ("dk[j * d + c] += J->scale * ds[j] * qi[c];",
                         "dk[j * d + c] += J->scale * ds[j] * load_elem(J->k, J->dtype, kvhead + j * d + c);"),
    "bwd_dv_from_ds": ("dv[j * d + c] += p[j] * gi[c];", "dv[j * d + c] += ds[j] * gi[c];"),
    "bwd_dq_dropped_scale": ("dq[i * d + c] += J->scale * ds[j] *", "dq[i * d + c] += ds[j] *"),
    "bwd_causal_bound": ("const int64_t nvis = causal ? i + 1 + (Nk - Nq) : Nk;",
                         "const int64_t nvis = causal ? i + (Nk - Nq) : Nk;"),
    "bwd_causal_offset_sign": ("const int64_t nvis = causal ? i + 1 + (Nk - Nq) : Nk;",
                               "const int64_t nvis = causal ? i + 1 - (Nk - Nq) : Nk;"),
    "bwd_rows_dropped_row_dot": ("const double ds = p[j] * (dp - D);",
                                 "const double ds = p[j] * dp;"),
    "bwd_row_dot_from_v": ("D += gi[c] * o[c];",
                           "D += load_elem(J->v, J->dtype, qhead + i * d + c) * o[c];"),
    "bwd_group_member": ("const int64_t h = g * grp + hh;", "const int64_t h = hh * J->Hkv + g;"),
    "bwd_group_sum_dropped": (
        "for (int64_t e = 0; e < Nk * d; ++e) dk[e] = dv[e] = 0.0;\n"
        "    for (int64_t hh = 0; hh < grp; ++hh) {",
        "for (int64_t hh = 0; hh < grp; ++hh) {\n"
        "      for (int64_t e = 0; e < Nk * d; ++e) dk[e] = dv[e] = 0.0;"),
    "bwd_rows_kv_map": ("kvhead = (b * Hkv + h / (H / Hkv)) * Nk * d;",
                        "kvhead = (b * Hkv + h % Hkv) * Nk * d;"),
    "bwd_row_parts_overwrite": ("hk[e] += jobs[t].pdk[e];", "hk[e] = jobs[t].pdk[e];"),
    "f16_table_index": ("f16_table[((const uint16_t*)base)[idx]]",
                        "f16_table[((const uint16_t*)base)[idx] ^ 1u]"),
}


def _run_mutant(name, workdir):
    old, new = MUTANTS[name]
    text = SRC.read_text()
    if text.count(old) != 1:
        return name, None, f"mutation anchor for {name} not found exactly once"
    src = workdir / f"fa_oracle_{name}.c"
    src.write_text(text.replace(old, new))
    lib = workdir / f"liboracle_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-pthread", "-o",
                    str(lib), str(src), "-lm"], check=True)
    env = dict(os.environ, FA_ORACLE_LIB=str(lib), OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        str(ROOT / "tests" / "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return name, r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    """Run every mutant's pin suite, several at a time (each is one process)."""
    from concurrent.futures import ThreadPoolExecutor
    workdir = tmp_path_factory.mktemp("mutants")
    workers = max(1, min(6, (os.cpu_count() or 2) - 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(lambda n: _run_mutant(n, workdir), sorted(MUTANTS)))
    return {name: (rc, out) for name, rc, out in results}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(mutant_results, name):
    rc, out = mutant_results[name]
    assert rc is not None, out
    assert rc != 0, f"mutant {name} passed every pin:\n{out}"
