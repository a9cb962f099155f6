"""The pins must be able to fail: each plausible mistake below is applied to a
copy of the oracle's source, built into a library of its own, and the pin suite
(tests/test_oracle_pins.py, without the exponential scans, which no mutant
touches) is run against it; at least one pin must fail per mutant. The
unmodified copy passes every pin run here.

Known silent mistake: the Gumbel argmax tie-break (two kept ids with equal
double scores e / q do not occur with a 52-bit stream)."""
import ctypes
import inspect
import os
import subprocess

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.cpp")

MUTANTS = {
    "score_times_q": ("const double score = static_cast<double>(e[j]) / q;",
                      "const double score = static_cast<double>(e[j]) * q;"),
    "topp_strictly_greater": ("if (static_cast<double>(cum) >= thr) break;",
                              "if (static_cast<double>(cum) > thr) break;"),
    "sample_ties_to_highest_id": ("    if (s[a] != s[b]) return s[a] > s[b];\n    return a < b;",
                                  "    if (s[a] != s[b]) return s[a] > s[b];\n    return a > b;"),
    "repetition_branches_swapped": ("float y = (x >= 0.0f) ? x / rep : x * rep;",
                                    "float y = (x >= 0.0f) ? x * rep : x / rep;"),
    "presence_times_count": ("          y = y - pres;",
                             "          y = y - pres * static_cast<float>(pcount[j]);"),
    "temperature_multiplies": ("for (int j = 0; j < V; ++j) s[j] = x[j] / T;",
                               "for (int j = 0; j < V; ++j) s[j] = x[j] * T;"),
    "min_p_dropped": ("if (e[j] >= mp) S.push_back(j);", "S.push_back(j);"),
    "top_k_dropped": ("const int n0 = (keff > 0) ? keff : V;", "const int n0 = V;"),
    "ignored_prompt_skips_repetition": ("        ++count[t];\n        if (i - off[r] >= skip) ++pcount[t];",
                                        "        if (i - off[r] >= skip) ++count[t];\n        if (i - off[r] >= skip) ++pcount[t];"),
    "ignore_length_ignored": ("if (i - off[r] >= skip) ++pcount[t];", "++pcount[t];"),
    "decay_reset_ignored": ("      top_p[r] = p0;  // the reset id was sampled",
                            "      top_p[r] = top_p[r] * d;  // the reset id was sampled"),
    "decay_floor_dropped": ("top_p[r] = p > lo ? p : lo;", "top_p[r] = p;"),
    "seed_step_of_one": ("seeds[r] += 0x9E3779B97F4A7C15ull;", "seeds[r] += 1ull;"),
    "logsoftmax_sign": ("auto lp = [&](int j) { return (z[j] - M) - logS; };",
                        "auto lp = [&](int j) { return (z[j] - M) + logS; };"),
    "slot_remap_scatters": ("    std::memcpy(static_cast<char*>(dst) + static_cast<int64_t>(i) * elem_bytes,\n"
                            "                static_cast<const char*>(src) + static_cast<int64_t>(j) * elem_bytes, elem_bytes);",
                            "    std::memcpy(static_cast<char*>(dst) + static_cast<int64_t>(j) * elem_bytes,\n"
                            "                static_cast<const char*>(src) + static_cast<int64_t>(i) * elem_bytes, elem_bytes);"),
    "logprob_temperature_multiplies": ("const float s = (T == 1.0f) ? x : x / T;",
                                       "const float s = (T == 1.0f) ? x : x * T;"),
    "top2_second_not_demoted": ("      g2 = g1;\n      g1 = score;", "      g1 = score;"),
    "top2_second_from_best_only": ("    } else if (score > g2) {", "    } else if (score > g1) {"),
    "unset_parameters_not_greedy": ("(unset ? 0.0f : 1.0f)", "1.0f"),
    "logprob_ties_to_highest_id": ("        if (z[a] != z[b]) return z[a] > z[b];\n        return a < b;",
                                   "        if (z[a] != z[b]) return z[a] > z[b];\n        return a > b;"),
}


def _pins():
    import test_oracle_pins as pins
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_") or "exp_" in name:
            continue
        params = list(inspect.signature(fn).parameters)
        if params == ["orc"]:
            out.append((name, fn, {}))
        elif params == ["orc", "kind"]:
            mark = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
            for kind in mark[0].args[1]:
                out.append((f"{name}[{kind}]", fn, {"kind": kind}))
    return out


def _build(tmp_path, mutant):
    src = open(SRC).read()
    if mutant is not None:
        a, b = MUTANTS[mutant]
        assert src.count(a) == 1, mutant
        src = src.replace(a, b)
    d = tmp_path / (mutant or "plain")
    d.mkdir()
    (d / "oracle.cpp").write_text(src)
    (d / "oracle.h").write_text(open(os.path.join(ROOT, "oracle", "oracle.h")).read())
    lib = d / "liboracle.so"
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", str(d / "oracle.cpp"), "-o", str(lib)], check=True)
    return str(lib)


def _failing_pins(lib_path):
    saved = oracle._lib
    oracle._lib = oracle._configure(ctypes.CDLL(lib_path))
    failed = []
    try:
        for name, fn, kw in _pins():
            try:
                fn(oracle, **kw)
            except AssertionError:
                failed.append(name)
    finally:
        oracle._lib = saved
    return failed


def test_unmodified_copy_passes(tmp_path):
    assert _failing_pins(_build(tmp_path, None)) == []


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, mutant):
    failed = _failing_pins(_build(tmp_path, mutant))
    assert failed, f"no pin catches {mutant}"
