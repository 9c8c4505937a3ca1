"""The pins of the oracle catch plausible mistakes in it (no GPU needed).

Each case plants one mistake (a dropped term, a wrong sign, index or constant, a swapped operand)
in a copy of ``oracle/skv_oracle.c``, compiles the copy, and runs the pins of
``tests/test_oracle_pins.py`` against it in a child process (``SKV_ORACLE_LIB`` names the copy).
The pins must fail for every mutant, and pass for an unmodified copy built the same way.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "skv_oracle.c")

# name -> list of (exact text in the source, replacement); each text occurs exactly once
MUTANTS = {
    "bf16 rounding ties away from zero": [
        ("y = ldexp(nearbyint(ldexp(x, 8 - e)), e - 8);", "y = ldexp(round(ldexp(x, 8 - e)), e - 8);")],
    "box minimum skips the last token": [
        ("          for (int32_t t = 0; t < n; ++t) {\n            double x = orc_decode(c->k, orc_kv_at(c, phys, g, t, j), c->dtype);\n            if (x < lo) lo = x;",
         "          for (int32_t t = 0; t < n; ++t) {\n            double x = orc_decode(c->k, orc_kv_at(c, phys, g, t, j), c->dtype);\n            if (x < lo && t + 1 < n) lo = x;")],
    "sample instead of population variance": [
        ("var[o] = ss / n;", "var[o] = ss / (n > 1 ? n - 1 : 1);")],
    "mean over the page size instead of the valid tokens": [
        ("double mu = sum / n;", "double mu = sum / c->S;")],
    "pooled mean over the sub-block size instead of its valid tokens": [
        ("(float)(sum / (t1 - t0));", "(float)(sum / pb);")],
    "projected key rounded through float32": [
        ("kproj[(((size_t)phys * c->Hkv + g) * c->S + t) * r + i] = orc_round_bf16(acc);",
         "kproj[(((size_t)phys * c->Hkv + g) * c->S + t) * r + i] = orc_round_bf16((float)acc);")],
    "box bound takes the smaller product": [
        ("U += (a > e ? a : e);", "U += (a < e ? a : e);")],
    "box key of the first query head only": [
        ("          if (U > best) best = U;", "          if (h == g * G) best = U;")],
    "gaussian spread with q instead of q squared": [
        ("sv += qj * qj * var[mo + j];", "sv += qj * var[mo + j];")],
    "gaussian spread without the square root": [
        ("s[o] = scale * sqrt(sv);", "s[o] = scale * sv;")],
    "estimated maximum with sqrt(ln n)": [
        ("sqrt(2.0 * log((double)n))", "sqrt(log((double)n))")],
    "estimated maximum with log2": [
        ("sqrt(2.0 * log((double)n))", "sqrt(2.0 * log2((double)n))")],
    "estimated maximum at the page size instead of the valid tokens": [
        ("shat[o] = m[o] + s[o] * fac[n];", "shat[o] = m[o] + s[o] * fac[c->S];")],
    "pooled key of the first query head only": [
        ("u += orc_q(c, b, g * G + hh, i) * (double)mv[i];", "u += orc_q(c, b, g * G, i) * (double)mv[i];")],
    "projected key with the first head's query": [
        ("u += (double)qt[hh * r + i] * orc_decode(kr, (size_t)i, ORC_BF16);",
         "u += (double)qt[i] * orc_decode(kr, (size_t)i, ORC_BF16);")],
    "soft hash without the factor 2": [
        ("sp[i] = 1.0 / (1.0 + exp(-((2.0 * z) / tau)));", "sp[i] = 1.0 / (1.0 + exp(-(z / tau)));"),
        ("sn[i] = 1.0 / (1.0 + exp(-((-2.0 * z) / tau)));", "sn[i] = 1.0 / (1.0 + exp(-(-z / tau)));")],
    "bucket bit set on the negative side": [
        ("if (dot > 0.0) id |= 1u << i;", "if (dot < 0.0) id |= 1u << i;")],
    "soft-collision sum over heads instead of the maximum": [
        ("          if (sum > best) best = sum;", "          best += sum;")],
    "top-k ties go to the higher index": [
        ("return (x->idx > y->idx) - (x->idx < y->idx);", "return (x->idx < y->idx) - (x->idx > y->idx);")],
    "budget rounds down": [
        ("int64_t k = ((int64_t)pct * P_b + 99) / 100;", "int64_t k = ((int64_t)pct * P_b) / 100;")],
    "second partial moment without the variance term": [
        ("return (mu * mu + sd_x * sd_x) * orc_Phi(a) + mu * sd_x * orc_phi(a);",
         "return (mu * mu) * orc_Phi(a) + mu * sd_x * orc_phi(a);")],
    "first partial moment without the density term": [
        ("if (alpha == 2.0) return mu * orc_Phi(a) + sd_x * orc_phi(a);", "if (alpha == 2.0) return mu * orc_Phi(a);")],
    "normalisation equation without the token counts": [
        ("if (n[p] > 0) f += n[p] * orc_gauss_partial_moment(", "if (n[p] > 0) f += orc_gauss_partial_moment(")],
    "truncated power moment with the wrong normal constant": [
        ("return orc_tanh_sinh(a, k, L0, U) / sqrt(2.0 * acos(-1.0));", "return orc_tanh_sinh(a, k, L0, U) / sqrt(acos(-1.0));")],
    "tanh-sinh weight without the cosh t factor": [
        ("const double wt = hw * 0.5 * acos(-1.0) * cosh(t) / (ch * ch);", "const double wt = hw * 0.5 * acos(-1.0) / (ch * ch);")],
    "tanh-sinh node distance from its end halved": [
        ("const double d = 2.0 * hw / (1.0 + exp(2.0 * fabs(x)));", "const double d = hw / (1.0 + exp(2.0 * fabs(x)));")],
    "threshold margin added instead of subtracted": [
        ("> tau_hat[hh] - delta) keep = 1;", "> tau_hat[hh] + delta) keep = 1;")],
    "box threshold against the largest head threshold": [
        ("if (tau_hat[hh] < tmin) tmin = tau_hat[hh];", "if (tau_hat[hh] < tmin || tmin < tau_hat[hh]) tmin = tau_hat[hh];")],
    "softmax of z / 2": [
        ("for (int32_t t = 0; t < n; ++t) sum += exp(z[t] - mx);", "for (int32_t t = 0; t < n; ++t) sum += exp(0.5 * (z[t] - mx));"),
        ("for (int32_t t = 0; t < n; ++t) p[t] = exp(z[t] - mx) / sum;", "for (int32_t t = 0; t < n; ++t) p[t] = exp(0.5 * (z[t] - mx)) / sum;")],
    "sparsemax threshold with the wrong sign": [
        ("if (1.0 + k * zs[k - 1] > cum) tau = (cum - 1.0) / k;", "if (1.0 + k * zs[k - 1] > cum) tau = (cum + 1.0) / k;")],
    "1.5-entmax without the (alpha - 1) scaling": [
        ("for (int32_t t = 0; t < n; ++t) zs[t] = 0.5 * z[t];", "for (int32_t t = 0; t < n; ++t) zs[t] = z[t];"),
        ("double x = 0.5 * z[t] - tau;", "double x = z[t] - tau;")],
    "1.5-entmax weights not squared": [
        ("p[t] = x > 0 ? x * x : 0.0;", "p[t] = x > 0 ? x : 0.0;")],
    "bisection entmax with power alpha - 1": [
        ("if (x > 0) sum += pow(x, 1.0 / am1);", "if (x > 0) sum += pow(x, am1);"),
        ("p[t] = x > 0 ? pow(x, 1.0 / am1) : 0.0;", "p[t] = x > 0 ? pow(x, am1) : 0.0;")],
    "logits without the scale": [
        ("z[i] = scale * acc;", "z[i] = acc;")],
    "attention sums keys instead of values": [
        ("orc_row(c, c->v, b, g, tok[i], row);", "orc_row(c, c->k, b, g, tok[i], row);")],
    "selected page expands to all its slots, not its valid tokens": [
        ("for (int32_t t = 0; t < np; ++t) tok[n++] = (int64_t)sel[i] * c->S + t;",
         "for (int32_t t = 0; t < c->S; ++t) tok[n++] = (int64_t)sel[i] * c->S + t;")],
}


def _mutate(text: str, edits) -> str:
    for old, new in edits:
        assert text.count(old) == 1, f"mutation anchor not unique or missing: {old[:60]!r}"
        text = text.replace(old, new)
    return text


def _run_pins(lib_path: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, SKV_ORACLE_LIB=lib_path, PYTHONDONTWRITEBYTECODE="1")
    return subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                           "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=600)


def test_every_planted_mistake_is_caught(tmp_path):
    src = open(SRC).read()
    jobs = {"(unmodified)": src}
    for name, edits in MUTANTS.items():
        jobs[name] = _mutate(src, edits)
        assert jobs[name] != src, name

    def one(item):
        i, (name, text) = item
        c_path = tmp_path / f"m{i}.c"
        c_path.write_text(text)
        lib = oracle.compile_source(str(c_path), str(tmp_path / f"m{i}.so"), extra=["-w"])
        r = _run_pins(lib)
        return name, r.returncode, (r.stdout[-600:] + r.stderr[-300:])

    workers = max(1, min(8, len(os.sched_getaffinity(0))))
    with cf.ThreadPoolExecutor(workers) as ex:
        results = list(ex.map(one, enumerate(jobs.items())))
    control = [r for r in results if r[0] == "(unmodified)"][0]
    assert control[1] == 0, f"the pins fail on an unmodified copy:\n{control[2]}"
    missed = [(n, rc) for n, rc, _ in results if n != "(unmodified)" and rc != 1]
    assert not missed, f"mutants not caught by a failing pin (rc 1): {missed}"
