"""Mutation check of the oracle's pins (CPU).

Each mutant plants one plausible mistake in a copy of oracle/oracle.c -- a
flipped sign, a dropped term, a transposed index, a tie rule or an order
reversed, an off-by-one at the capacity -- is compiled on its own and loaded
by tests/test_oracle_pins.py in a fresh process; every mutant must make at
least one pin fail, and the unchanged copy must pass them all.  This is the
evidence that the pins tie the oracle to the pages and the mathematics
rather than to itself.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# name -> (text in oracle.c, its replacement); each text occurs once
MUTANTS = {
    "unchanged": ("", ""),
    "silu_sign": ("double silu = a / (1.0 + exp(-a));", "double silu = a / (1.0 + exp(a));"),
    "gate_up_swapped": ("double silu = a / (1.0 + exp(-a));\n    h[f] = silu * bb;",
                        "double silu = bb / (1.0 + exp(-bb));\n    h[f] = silu * a;"),
    "w_down_transposed": ("elem_f(wd, dtype, wd_off + i * d_ff + f)",
                          "elem_f(wd, dtype, wd_off + f * d + i)"),
    "router_bias_dropped": ("if (b) acc = acc + b[e];", "(void)b;"),
    "r64_granule_of_one": ("const int l = (int)((i / 8) % 64);", "const int l = (int)(i % 64);"),
    "topk_ties_highest": ("if (best < 0 || l[e] > l[best]) best = e;\n      }\n      taken[best] = 1;",
                          "if (best < 0 || l[e] >= l[best]) best = e;\n      }\n      taken[best] = 1;"),
    "renorm_over_all_e": ("if (renorm) {", "if (0) {"),
    "capacity_floor": ("double c = ceil(phi * (double)(T * k) / (double)E);",
                       "double c = floor(phi * (double)(T * k) / (double)E);"),
    "keeps_c_plus_one": ("if (C < 0 || slot[r] < C) {", "if (C < 0 || slot[r] <= C) {"),
    "last_arrivals_kept": ("for (int64_t r = 0; r < R; r++) {\n    int32_t e = expert_ids[r];\n    slot[r] = counts[e];",
                           "for (int64_t r = R - 1; r >= 0; r--) {\n    int32_t e = expert_ids[r];\n    slot[r] = counts[e];"),
    "combine_ignores_gates": ("acc += (double)gates[t * k + j] *", "acc += 1.0 *"),
    "shared_expert_lost": ("if (y_shared) acc += elem_d(y_shared, ypdtype, t * d + i);",
                           "(void)y_shared;"),
    "padded_slot_major": ("pad_pos[r] = (int32_t)(e * C + slot);",
                          "pad_pos[r] = (int32_t)(slot * E + e);"),
    "reroute_ties_highest": ("if (best < 0 || l[e] > l[best]) best = e; /* strict >",
                             "if (best < 0 || l[e] >= l[best]) best = e; /* strict >"),
    "queue_after_batch": ("for (int64_t a = 0; a < Q; a++) seq[a] = q_ids[a];\n  for (int64_t r = 0; r < T * k; r++) seq[Q + r] = ids[r];",
                          "for (int64_t a = 0; a < Q; a++) seq[T * k + a] = q_ids[a];\n  for (int64_t r = 0; r < T * k; r++) seq[r] = ids[r];"),
    "choice_ties_highest_token": ("return x->t < y->t ? -1 : (x->t > y->t ? 1 : 0);",
                                  "return x->t > y->t ? -1 : (x->t < y->t ? 1 : 0);"),
    "aux_loss_without_e": ("out[0] = alpha * (double)E * aux;", "out[0] = alpha * aux;"),
    "entropy_unnormalised": ("sum_entropy += h / log((double)k);", "sum_entropy += h;"),
    "confidence_bins_ceil": ("int32_t b = (int32_t)floor(conf * (double)n_bins);",
                             "int32_t b = (int32_t)ceil(conf * (double)n_bins);"),
    "js_natural_log": ("js += 0.5 * share[e] * log2(share[e] / mid);",
                       "js += 0.5 * share[e] * log(share[e] / mid);"),
}


def _run(name, old, new, tmp):
    src = open(SRC).read()
    if old:
        assert src.count(old) == 1, f"{name}: the mutated text must occur exactly once"
        src = src.replace(old, new)
    mdir = os.path.join(tmp, name)
    os.makedirs(mdir)
    c = os.path.join(mdir, "oracle.c")
    with open(c, "w") as f:
        f.write(src)
    so = os.path.join(mdir, "liboracle.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", "-I", os.path.join(ROOT, "oracle"), "-o", so, c, "-lm"],
                   check=True, capture_output=True)
    env = dict(os.environ, MOE_ORACLE_LIB=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", PINS], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_every_mutant_fails_a_pin(tmp_path):
    with cf.ThreadPoolExecutor(4) as ex:
        futs = {n: ex.submit(_run, n, o, m, str(tmp_path)) for n, (o, m) in MUTANTS.items()}
        res = {n: f.result() for n, f in futs.items()}
    rc, out = res.pop("unchanged")
    assert rc == 0, f"the unchanged oracle fails its pins:\n{out}"
    # pytest exits with 1 when a test failed; a crash or a collection error
    # would not show that a pin caught the mutant
    survivors = {n: rc for n, (rc, _) in res.items() if rc != 1}
    assert not survivors, f"mutants no pin caught (exit code): {survivors}"
