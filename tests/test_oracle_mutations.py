"""The pins have teeth: plant plausible mistakes in a private copy of the
oracle's C source (a dropped term, a wrong sign, a wrong decay power, a
swapped operand), rebuild it in a temporary folder, and check that the pin
checks below reject every variant.  The real oracle is never modified.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "G decays by g instead of g^2": ("Gi[j] = g2 * Gi[j] + gk * r[j]", "Gi[j] = g * Gi[j] + gk * r[j]"),
    "cross term loses its g": ("const double gk = g * k[i];", "const double gk = k[i];"),
    "cross term sign": ("Gi[j] = g2 * Gi[j] + gk * r[j]", "Gi[j] = g2 * Gi[j] - gk * r[j]"),
    "h decays by g": ("h[i] = g2 * h[i] + gk * s;", "h[i] = g * h[i] + gk * s;"),
    "ridge dropped": ("a[i] = acc + lam * q[i];", "a[i] = acc;"),
    "G added instead of removed": ("num[j] += ai * Ci[j] - qi * Gi[j];", "num[j] += ai * Ci[j] + qi * Gi[j];"),
    "h added in den": ("dn += ai * m[i] - qi * h[i];", "dn += ai * m[i] + qi * h[i];"),
    "m not decayed": ("m[i] = g * m[i] + q[i];", "m[i] = m[i] + q[i];"),
    "S delta uses q": ("Si[j] = g * Si[j] + k[i] * k[j];", "Si[j] = g * Si[j] + k[i] * q[j];"),
    "C delta transposed roles": ("Ci[j] = g * Ci[j] + q[i] * v[j];", "Ci[j] = g * Ci[j] + k[i] * v[j];"),
    "rho not advanced": ("rho *= g;", "rho *= 1.0;"),
    "compose G decays once": ("rb * rb * Ga[", "rb * Ga["),
    "compose cross uses earlier S": ("cross += Sb[i * d + l] * Ca[", "cross += Sa[i * d + l] * Ca["),
    "compose h cross dropped": ("h[i] = rb * rb * ha[i] + hb[i] + rb * cross;", "h[i] = rb * rb * ha[i] + hb[i];"),
    "r read after the delta (inclusive C)": (
        "    /* cross summaries: G, h */",
        "    for (i = 0; i < d; ++i) for (j = 0; j < dv; ++j) r[j] += k[i] * q[i] * v[j];\n"
        "    /* cross summaries: G, h */"),
}

CHECKS = textwrap.dedent(r'''
    import sys, numpy as np
    sys.path.insert(0, sys.argv[1])
    import oracle
    from oracle import brute
    oracle.build(force=True)
    r = np.random.default_rng(1)
    fails = []
    def rel(a, b):
        return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))
    # brute force, with decay and ridge, d != dv
    q, k, v = (r.standard_normal((1, 1, 13, 3)), r.standard_normal((1, 1, 13, 3)),
               r.standard_normal((1, 1, 13, 4)))
    out, den, st = oracle.forward(q, k, v, gamma=[0.9], lam=0.3)
    nr, dr = brute.masked(q[0, 0], k[0, 0], v[0, 0], 0.9, 0.3)
    if rel(out[0, 0], nr) > 1e-10: fails.append("num")
    if rel(den[0, 0], dr) > 1e-10: fails.append("den")
    S, C, m = brute.prefix_moments(q[0, 0], k[0, 0], v[0, 0], 12, 0.9)
    G, h = brute.future_pairs(q[0, 0], k[0, 0], v[0, 0], 12, 0.9)
    for name, a, b in (("S", st.S[0], S), ("C", st.C[0], C), ("m", st.m[0], m),
                       ("G", st.G[0], G), ("h", st.h[0], h)):
        if rel(a, b) > 1e-10: fails.append(name)
    if abs(st.rho[0] - 0.9 ** 13) > 1e-14: fails.append("rho")
    # compose of two segments == serial
    _, _, sa = oracle.forward(q[:, :, :6], k[:, :, :6], v[:, :, :6], gamma=[0.9])
    _, _, sb = oracle.forward(q[:, :, 6:], k[:, :, 6:], v[:, :, 6:], gamma=[0.9])
    _, _, sf = oracle.forward(q, k, v, gamma=[0.9])
    c = oracle.compose(sa, sb)
    for name in ("S", "C", "m", "G", "h", "rho"):
        if rel(getattr(c, name), getattr(sf, name)) > 1e-10: fails.append("compose-" + name)
    print("CAUGHT" if fails else "MISSED", fails)
''')


@pytest.fixture(scope="module")
def pristine_src():
    with open(os.path.join(ROOT, "oracle", "hla_oracle.c")) as f:
        return f.read()


def _run_variant(tmp_path, src):
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    for name in ("__init__.py", "brute.py", "higher.py", "higher_oracle.c"):
        shutil.copy(os.path.join(ROOT, "oracle", name), pkg / name)
    (pkg / "hla_oracle.c").write_text(src)
    (tmp_path / "checks.py").write_text(CHECKS)
    r = subprocess.run([sys.executable, str(tmp_path / "checks.py"), str(tmp_path)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    return r.stdout


def test_unmutated_copy_passes(tmp_path, pristine_src):
    assert "MISSED []" in _run_variant(tmp_path, pristine_src)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, pristine_src, name):
    old, new = MUTATIONS[name]
    assert pristine_src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    out = _run_variant(tmp_path, pristine_src.replace(old, new))
    assert "CAUGHT" in out, f"{name}: {out}"
