"""The oracle's pins have teeth: each plausible one-line mistake planted in a
copy of oracle/oracle.c (a dropped term, a wrong sign, base or index, a
transposed store, the wrong rank, a wrong decoder) must fail at least one of
the pins in test_oracle.py.

Each mutant is compiled to its own library in a temporary directory and
checked in a child process (a mutant that crashes cannot take the test run
down; a crash counts as caught). The real oracle is never modified.

Two single-line changes are left out on purpose because they are equivalent
(no input can tell them apart): dropping the reset of an all -inf maximum to 0,
and dropping the NaN-weight guard. Either one alone still gives a zero output
and a -inf LSE for an all -inf row, because the other step covers that case
(the page's function has both).
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement, occurrence: None = every one)
MUTANTS = [
    ("sanitise_keeps_inf", "(isnan(v) || isinf(v))", "isnan(v)", None),
    ("base2_uses_exp", "pow(2.0, l[n] - m)", "exp(l[n] - m)", None),
    ("weight_sign", ": exp(l[n] - m)", ": exp(m - l[n])", None),
    ("no_clamp", "double denom = s < 1e-10 ? 1e-10 : s;", "double denom = s;", None),
    ("no_normalisation", "wn[n] = w[n] / denom;", "wn[n] = w[n];", None),
    ("sum_skips_first_shard", "for (int64_t n = 0; n < N; ++n) s += w[n];",
     "for (int64_t n = 1; n < N; ++n) s += w[n];", None),
    ("lse_without_max", "if (L) L[r] = (base2 ? log2(s) : log(s)) + m;",
     "if (L) L[r] = (base2 ? log2(s) : log(s));", 0),
    ("lse_wrong_base", "if (L) L[r] = (base2 ? log2(s) : log(s)) + m;",
     "if (L) L[r] = log(s) + m;", 0),
    ("output_index_transposed", "acc += o[(n * R + r) * D + d] * wn[n];",
     "acc += o[(r * N + n) * D + d] * wn[n];", None),
    ("bf16_shift", "uint32_t x = (uint32_t)h << 16;", "uint32_t x = (uint32_t)h << 15;", None),
    ("f16_bias", "e - 25);", "e - 24);", None),
    ("f32_not_reinterpreted", "memcpy(&f, &u, 4);\n    return (double)f;",
     "memcpy(&f, &u, 4);\n    return (double)u;", None),
    ("pack_plane_mapping", "const int64_t src = b * H + r * Hl + h;",
     "const int64_t src = b * H + h * N + r;", None),
    ("pack_tail_at_row_start", "memcpy(dst + D * E, &lse[src], 4);",
     "memcpy(dst, &lse[src], 4);", None),
    ("unpack_combine_tail_off_by_one", "memcpy(&lf, src + D * E, 4);",
     "memcpy(&lf, src + (D - 1) * E, 4);", None),
    ("merge_not_transposed", "token_dim == 1 ? r : c * A + a", "token_dim == 1 ? r : a * C + c",
     None),
    ("correct_wrong_rank", "if (n == rank) wr = w;", "if (n == 0) wr = w;", None),
    ("correct_lse_without_max", "if (L) L[r] = (base2 ? log2(s) : log(s)) + m;",
     "if (L) L[r] = (base2 ? log2(s) : log(s));", 1),
    ("valid_reads_previous_entry", "int64_t t = query_start_loc[num_reqs];",
     "int64_t t = query_start_loc[num_reqs > 0 ? num_reqs - 1 : 0];", None),
    ("valid_reads_next_entry", "int64_t t = query_start_loc[num_reqs];",
     "int64_t t = query_start_loc[num_reqs + 1];", None),
    ("valid_reads_first_entry", "int64_t t = query_start_loc[num_reqs];",
     "int64_t t = query_start_loc[0];", None),
    ("valid_no_capacity_clamp", "    if (t > capacity) t = capacity;\n", "", None),
    ("valid_no_negative_clamp", "    if (t < 0) t = 0;\n", "", None),
    ("valid_takes_the_last_tokens", "n * plane + r", "n * plane + (T - Tv) * H + r", None),
    ("valid_plane_stride_of_valid_tokens", "const int64_t plane = T * H;",
     "const int64_t plane = Tv * H;", None),
]

RUNNER = textwrap.dedent("""
    import importlib.util, os, sys
    root, lib = sys.argv[1], sys.argv[2]
    sys.path.insert(0, os.path.join(root, "tests"))
    sys.path.insert(0, root)
    spec = importlib.util.spec_from_file_location(
        "oracle_mutant", os.path.join(root, "oracle", "__init__.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    m._LIB = lib
    m._load()
    import synth
    synth._load()
    import test_oracle as t
    pins = [
        ("bf16 decoding", lambda: t.test_bf16_decoding_all_patterns(m)),
        ("f16 decoding", lambda: t.test_f16_decoding_all_patterns(m)),
        ("f32 decoding", lambda: t.test_f32_decoding(m)),
        ("brute force base e", lambda: t.test_brute_force_sharded_attention(m, "contiguous", False, 5)),
        ("brute force base 2, empty shards",
         lambda: t.test_brute_force_sharded_attention(m, "with_empty", True, 5)),
        ("brute force fp32 storage", lambda: t.test_brute_force_fp32_storage(m, 2)),
        ("logsumexp base e", lambda: t.test_global_lse_is_logsumexp(m, False)),
        ("logsumexp base 2", lambda: t.test_global_lse_is_logsumexp(m, True)),
        ("softmax formulation", lambda: t.test_agrees_with_softmax_formulation(m, synth)),
        ("invariants", lambda: t.test_invariants(m)),
        ("pack layout", lambda: t.test_pack_layout_and_round_trip(m, synth)),
        ("pack layout fp32", lambda: t.test_pack_layout_f32(m, synth)),
        ("simulated all-to-all", lambda: t.test_simulated_all_to_all(m, synth, "bf16", False)),
        ("merge layout", lambda: t.test_merge_matches_page2_layout(m, synth, 2, "bf16")),
        ("corrected partials", lambda: t.test_corrected_partials_sum_to_the_combine(m, synth, True, "bf16")),
        ("corrected partial closed form", lambda: t.test_corrected_partial_closed_form(m)),
        ("valid tokens: padded step of requests",
         lambda: t.test_valid_combine_is_attention_of_the_real_tokens(m, [3, 0, 4], 10, 3)),
        ("valid tokens: entry num_reqs", lambda: t.test_valid_combine_counts_entry_num_reqs(m, synth)),
    ]
    pins += [("closed form " + c["name"], (lambda c=c: t.test_closed_forms(m, c)))
             for c in t._golden_cases()]
    pins += [("valid tokens " + c["name"], (lambda c=c: t.test_valid_tokens_hand_derived(m, c)))
             for c in t._valid_cases()]
    failed = []
    for name, fn in pins:
        try:
            fn()
        except BaseException as e:  # an assertion, a library error: the pin caught it
            failed.append(name)
    print("FAILED PINS: " + "; ".join(failed))
""")


def _mutate(text, old, new, occurrence):
    assert old in text, f"mutation site not found: {old!r}"
    if occurrence is None:
        return text.replace(old, new)
    parts = text.split(old)
    assert occurrence < len(parts) - 1, f"occurrence {occurrence} of {old!r} not found"
    return old.join(parts[:occurrence + 1]) + new + old.join(parts[occurrence + 1:])


@pytest.mark.parametrize("name,old,new,occurrence", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, occurrence):
    import oracle
    oracle._load()  # the real oracle builds first if it has not been built
    src = _mutate(open(SRC).read(), old, new, occurrence)
    csrc = tmp_path / "oracle_mutant.c"
    csrc.write_text(src)
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", str(lib), str(csrc), "-lm"],
                   check=True)
    res = subprocess.run([sys.executable, "-c", RUNNER, ROOT, str(lib)], capture_output=True,
                         text=True, timeout=300)
    if res.returncode != 0:  # the mutant crashed the process: caught
        return
    line = [ln for ln in res.stdout.splitlines() if ln.startswith("FAILED PINS:")]
    assert line, res.stdout + res.stderr
    caught = line[0][len("FAILED PINS:"):].strip()
    print(f"{name}: caught by {caught}")
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_every_pin(tmp_path):
    """The runner itself reports no failure on the real oracle's source."""
    import oracle
    oracle._load()
    lib = tmp_path / "liboracle_copy.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", str(lib), SRC, "-lm"],
                   check=True)
    res = subprocess.run([sys.executable, "-c", RUNNER, ROOT, str(lib)], capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr
    line = [ln for ln in res.stdout.splitlines() if ln.startswith("FAILED PINS:")]
    assert line and not line[0][len("FAILED PINS:"):].strip(), res.stdout
