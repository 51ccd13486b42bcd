"""CPU tests of the oracle: every pin in oracle_pins.py against the oracle,
and planted mistakes in copies of the oracle that some pin must catch."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import oracle_pins
from oracle_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name, oracle_lib):
    PINS[name](oracle_lib)


def test_parent_logit_recovery_exact():
    oracle_pins.pin_parent_logit_recovery()


# (what the mistake is, exact source text, replacement)
MUTANTS = [
    ("correction sign flipped",
     "exp(s[c] - m) - exp(sp - m) : 0.0;", "exp(sp - m) - exp(s[c] - m) : 0.0;"),
    ("parent logit is not the mean of all children", "sp /= C;", "sp /= (C + 1);"),
    ("child comparison not strict", "if (dc < dchild) { dchild = dc; cstar = c0 + c; }",
     "if (dc <= dchild) { dchild = dc; cstar = c0 + c; }"),
    ("move on a tie with the parent", "(C > 0 && dchild < dbest)", "(C > 0 && dchild <= dbest)"),
    ("last minimum among parents", "if (dm < dbest) { dbest = dm; a = m; }", "if (dm <= dbest) { dbest = dm; a = m; }"),
    ("children of the wrong parent", "int64_t c0 = M0 + (int64_t)a * C;", "int64_t c0 = M0 + (int64_t)((a + 1) % M0) * C;"),
    ("denominator without counts", "z += A * n[j];", "z += A;"),
    ("empty children not masked", "double dA = n[c0 + c] > 0 ? exp(s[c] - m) - exp(sp - m) : 0.0;",
     "double dA = exp(s[c] - m) - exp(sp - m);"),
    ("running max over empty children", "if (n[c0 + c] > 0 && s[c] > mnew) mnew = s[c];", "if (s[c] > mnew) mnew = s[c];"),
    ("importance without counts", "if (n[j] > 0) w[j] += exp(s[j] - m) * n[j] / Z;",
     "if (n[j] > 0) w[j] += exp(s[j] - m) / Z;"),
    ("importance without the logit scale", "s[j] = scale * dotd(q, cbh + (int64_t)j * d, d);\n            if (n[j] > 0 && s[j] > m) m = s[j];\n        }\n        double Z",
     "s[j] = dotd(q, cbh + (int64_t)j * d, d);\n            if (n[j] > 0 && s[j] > m) m = s[j];\n        }\n        double Z"),
    ("top-P ties to the higher index", "if (wr[jj] > wr[j] || (wr[jj] == wr[j] && jj < j)) ++ahead;",
     "if (wr[jj] > wr[j] || (wr[jj] == wr[j] && jj > j)) ++ahead;"),
    ("parent rows miss the moved keys", "ct[a] += 1;", "ct[a] += (r == a);"),
    ("no residual for a refined parent", "nn[a] -= n[c0 + c];", ";"),
    ("brute force ignores the selection", "int32_t khat = (r != a && in_sel(S, P, a)) ? r : a;",
     "int32_t khat = r;"),
    ("tiled denominator not extrapolated", "const double zt = ntot / nseen * zacc;", "const double zt = zacc;"),
    ("tiled denominator not rescaled with the stabiliser", "zacc = m == -INFINITY ? 0.0 : zacc * exp(m - mt);",
     "zacc = m == -INFINITY ? 0.0 : zacc;"),
    ("keys of a tile's first parent not seen", "                        nseen += n[j];",
     "                        nseen += (j > j0) ? n[j] : 0;"),
    ("harmonic weight sums the masses", "if (n > 0.0) sigma += 1.0 / n; else ++zeros;",
     "if (n > 0.0) sigma += n; else ++zeros;"),
    ("residual without the child count", "delta[t] = sm - (double)C * cbh[(int64_t)p * d + t];",
     "delta[t] = sm - cbh[(int64_t)p * d + t];"),
    ("EMA weights swapped", "Sh[x * d + t] = decay * Sh[x * d + t] + (1.0 - decay) * kb[t];",
     "Sh[x * d + t] = (1.0 - decay) * Sh[x * d + t] + decay * kb[t];"),
    ("unweighted projection", "if (zeros == 0) share = 1.0 / (n * sigma);", "if (zeros == 0) share = 1.0 / C;"),
    ("massless children keep their place", "else share = n > 0.0 ? 0.0 : 1.0 / zeros;", "else share = 0.0;"),
    ("parent choice in single precision", "if (dm < dbest) { dbest = dm; a = m; }",
     "if ((float)dm < (float)dbest) { dbest = dm; a = m; }"),
    ("move decision in single precision", "(C > 0 && dchild < dbest)", "(C > 0 && (float)dchild < (float)dbest)"),
    ("selection in single precision", "if (wr[jj] > wr[j] || (wr[jj] == wr[j] && jj < j)) ++ahead;",
     "if ((float)wr[jj] > (float)wr[j] || ((float)wr[jj] == (float)wr[j] && jj < j)) ++ahead;"),
    ("count EMA uses the old count twice", "Nh[x] = decay * Nh[x] + (1.0 - decay) * cnt;", "Nh[x] = decay * Nh[x] + (1.0 - decay) * Nh[x];"),
]


@pytest.mark.parametrize("what,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(what, old, new, tmp_path):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old}"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    oracle.build(str(mpath), so)
    lib = oracle.load(so)
    failed = []
    for name, pin in PINS.items():
        try:
            pin(lib)
        except AssertionError:
            failed.append(name)
    assert failed, f"no pin catches: {what}"


# planted mistakes in the ordering step of the oracle (Python), each of which
# some pin must catch
_real_ordered = oracle.Oracle.ordered


def _gather_by_inverse(self, Q, order):
    order = np.asarray(order)
    if np.array_equal(np.sort(order), np.arange(order.size)):
        order = np.argsort(order)
    return _real_ordered(self, Q, order)


def _left_in_tile_order(self, Yo, rows):
    Y = np.full((self.B * self.H, self.N, self.d), np.nan)
    Y[:, :len(rows)] = Yo
    return Y


def _empty_reads_row_zero(self, Q, order):
    order = np.asarray(order, np.int64)
    rows = np.where((order >= 0) & (order < self.N), order, 0)
    return oracle.Oracle(self.B, self.H, self.N, self.d, self.M0, self.C, lib=self.lib), np.asarray(Q)[:, rows], rows


ORDER_MUTANTS = [
    ("queries gathered by the inverse order", "ordered", _gather_by_inverse),
    ("outputs left in tile order", "scatter_rows", _left_in_tile_order),
    ("empty positions read row 0", "ordered", _empty_reads_row_zero),
]


@pytest.mark.parametrize("what,attr,fn", ORDER_MUTANTS, ids=[m[0] for m in ORDER_MUTANTS])
def test_order_mutant_is_caught(what, attr, fn, oracle_lib, monkeypatch):
    monkeypatch.setattr(oracle.Oracle, attr, fn)
    failed = []
    for name, pin in PINS.items():
        if name.startswith("order_"):
            try:
                pin(oracle_lib)
            except AssertionError:
                failed.append(name)
    assert failed, f"no pin catches: {what}"
