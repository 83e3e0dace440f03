"""The AHLA and third-order pins have teeth: plant plausible mistakes in a
private copy of oracle/higher_oracle.c (a state read before its token delta,
a wrong decay, a dropped or misplaced composition term, a swapped operand),
rebuild the oracle from that copy in a temporary folder, and check that the
pin checks below reject every variant.  The real oracle is never modified.
"""
import os
import shutil
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    # AHLA
    "AHLA y read before the P delta (strict inner mask)": (
        "    for (j = 0; j < dv; ++j) y[j] = 0.0;\n    for (i = 0; i < d; ++i) {\n        const double *Pi = P + (size_t)i * dv;\n        for (j = 0; j < dv; ++j) y[j] += q[i] * Pi[j];",
        "    for (j = 0; j < dv; ++j) y[j] = 0.0;\n    for (i = 0; i < d; ++i) {\n        const double *Pi = P + (size_t)i * dv;\n        for (j = 0; j < dv; ++j) y[j] += q[i] * (Pi[j] - k[i] * v[j]);"),
    "AHLA E decays by g^2": ("Ei[j] = g * Ei[j] + k[i] * y[j];", "Ei[j] = g * g * Ei[j] + k[i] * y[j];"),
    "AHLA E delta uses q": ("Ei[j] = g * Ei[j] + k[i] * y[j];", "Ei[j] = g * Ei[j] + q[i] * y[j];"),
    "AHLA n uses the wrong mass": ("yd += q[i] * m[i];\n    }\n    for (i = 0; i < d; ++i) {\n        double *Ei",
                                   "yd += k[i] * m[i];\n    }\n    for (i = 0; i < d; ++i) {\n        double *Ei"),
    "AHLA P delta transposed roles": ("Pi[j] = g * Pi[j] + k[i] * v[j];", "Pi[j] = g * Pi[j] + q[i] * v[j];"),
    "AHLA R sums q k^T": ("R[(size_t)i * d + j] += k[i] * q[j];", "R[(size_t)i * d + j] += q[i] * k[j];"),
    "AHLA compose cross drops rho_b": (
        "Eb[s * sc + (size_t)i * dv + j] + rb * cross;", "Eb[s * sc + (size_t)i * dv + j] + cross;"),
    "AHLA compose cross uses the earlier R": (
        "cross += Rb[s * sd + (size_t)i * d + l] * Pa[", "cross += Ra[s * sd + (size_t)i * d + l] * Pa["),
    # third order
    "third a read before the S delta": (
        "        for (j = 0; j < d; ++j) acc += Si[j] * q[j];",
        "        for (j = 0; j < d; ++j) acc += (Si[j] - k[i] * k[j]) * q[j];"),
    "third F delta uses q instead of S q": ("for (j = 0; j < dv; ++j) Fi[j] += a[i] * y[j];",
                                            "for (j = 0; j < dv; ++j) Fi[j] += q[i] * y[j];"),
    "third Fd uses y of the value": ("Fd[i] += yd * a[i];", "Fd[i] += yd * q[i];"),
    "third M sums q q^T": ("M[(size_t)i * d + j] += a[i] * q[j];", "M[(size_t)i * d + j] += q[i] * q[j];"),
    "third compose drops S_a N_b": ("        mat_acc(d, dv, sa, Nb + s * sc, F + s * sc);\n", ""),
    "third compose M without the cross": ("M[s * sd + e] = Ma[s * sd + e] + mbb[e] + T[e];",
                                          "M[s * sd + e] = Ma[s * sd + e] + mbb[e];"),
    "third compose N cross from the earlier SQ": ("        mat_acc(d, dv, sqb, pa, Nn + s * sc);",
                                                  "        mat_acc(d, dv, SQa + s * sd, pa, Nn + s * sc);"),
}

CHECKS = textwrap.dedent(r'''
    import sys, numpy as np
    sys.path.insert(0, sys.argv[1])
    import oracle
    from oracle import brute, higher
    oracle.build(force=True)
    r = np.random.default_rng(3)
    fails = []
    def rel(a, b):
        return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))
    q, k, v = (r.standard_normal((1, 2, 11, 3)), r.standard_normal((1, 2, 11, 3)), r.standard_normal((1, 2, 11, 2)))
    # AHLA: brute force with decay, composition == serial (R included)
    out, den, st = higher.ahla_forward(q, k, v, gamma=[0.9, 0.7])
    for h, g in ((0, 0.9), (1, 0.7)):
        nr, dr = brute.ahla(q[0, h], k[0, h], v[0, h], g)
        if rel(out[0, h], nr) > 1e-10: fails.append("ahla-num")
        if rel(den[0, h], dr) > 1e-10: fails.append("ahla-den")
    _, _, sa = higher.ahla_forward(q[:, :, :5], k[:, :, :5], v[:, :, :5], gamma=[0.9, 0.7])
    _, _, sb = higher.ahla_forward(q[:, :, 5:], k[:, :, 5:], v[:, :, 5:], gamma=[0.9, 0.7])
    c = higher.ahla_compose(sa, sb)
    for name in ("P", "m", "E", "n", "R", "rho"):
        if rel(getattr(c, name), getattr(st, name)) > 1e-10: fails.append("ahla-compose-" + name)
    R = np.einsum("bhtd,bhte->bhde", k, q).reshape(2, 3, 3)
    if rel(st.R, R) > 1e-10: fails.append("ahla-R")
    # third order: brute force, composition == serial (all nine parts)
    o3, d3, s3 = higher.third_forward(q, k, v)
    for h in range(2):
        nr, dr = brute.third(q[0, h], k[0, h], v[0, h])
        if rel(o3[0, h], nr) > 1e-10: fails.append("third-num")
        if rel(d3[0, h], dr) > 1e-10: fails.append("third-den")
    _, _, ta = higher.third_forward(q[:, :, :4], k[:, :, :4], v[:, :, :4])
    _, _, tb = higher.third_forward(q[:, :, 4:], k[:, :, 4:], v[:, :, 4:])
    ct = higher.third_compose(ta, tb)
    for name in ("S", "P", "m", "F", "Fd", "SQ", "M", "Nq", "Nd"):
        if rel(getattr(ct, name), getattr(s3, name)) > 1e-10: fails.append("third-compose-" + name)
    print("CAUGHT" if fails else "MISSED", fails)
''')


@pytest.fixture(scope="module")
def pristine_src():
    with open(os.path.join(ROOT, "oracle", "higher_oracle.c")) as f:
        return f.read()


def _run_variant(tmp_path, src):
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    for name in ("__init__.py", "brute.py", "higher.py", "hla_oracle.c"):
        shutil.copy(os.path.join(ROOT, "oracle", name), pkg / name)
    (pkg / "higher_oracle.c").write_text(src)
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
