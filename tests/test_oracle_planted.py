"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake into a copy of the oracle's source (a wrong
sign of the causal offset, a wrong GQA head map, a log base, a dropped max
subtraction, a window off by one, a dropped scale, a missing
normalisation, and a few in the next-row features), installs the copy as
``oracle`` in a fresh interpreter and runs the pins of
``tests/test_oracle.py`` against it: at least one pin must fail.  The
unpatched source passes the same run (checked first), so a failure means
the pins saw the mistake.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "attention.py")

# (name, text in the oracle, replacement)
MISTAKES = [
    ("causal offset sign", "    pos = i + (Lk - Lq)\n    vis = (i < Lq) & (j < Lk)",
     "    pos = i - (Lk - Lq)\n    vis = (i < Lq) & (j < Lk)"),
    ("GQA head map", "kvh = h // group", "kvh = h % Hkv"),
    ("log base of LSE", "lse = m_safe + np.log(l)", "lse = m_safe + np.log2(l)"),
    ("no max subtraction", "p = np.exp(s - m_safe[:, None])", "p = np.exp(s)"),
    ("window off by one", "vis &= j > pos - window_left", "vis &= j >= pos - window_left"),
    ("dropped scale", "s = scale * (q_rows @ k.T)", "s = (q_rows @ k.T)"),
    ("no normalisation", "o = (p[:, cols] @ v[cols]) / l[:, None]", "o = (p[:, cols] @ v[cols])"),
    ("ALiBi sign", "return -float(slope) * np.abs(pos - j)", "return float(slope) * np.abs(pos - j)"),
    ("RoPE rotation sign", "round_to_dtype(a * s + b * c, store)", "round_to_dtype(-a * s + b * c, store)"),
    ("E4M3 exponent bias", "np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    ("decode query position", "qb = rope_rotate(qb, np.full(qb.shape[0], L - 1), *rope_q)",
     "qb = rope_rotate(qb, np.full(qb.shape[0], max(L - 2, 0)), *rope_q)"),
    ("paged row index", "rows = [pool[int(table_row[j // P]), j % P] for j in range(L)]",
     "rows = [pool[int(table_row[j % P]), j // P] for j in range(L)]"),
]

BOOT = r"""
import sys, types
src = open({src!r}).read()
old, new = {old!r}, {new!r}
if old:
    assert src.count(old) == 1, "the planted text must occur once"
    src = src.replace(old, new)
pkg = types.ModuleType("oracle")
pkg.__path__ = []
sub = types.ModuleType("oracle.attention")
exec(compile(src, "planted_oracle", "exec"), sub.__dict__)
for k, v in sub.__dict__.items():
    if not k.startswith("__"):
        setattr(pkg, k, v)
pkg.attention_module = sub
sys.modules["oracle"] = pkg
sys.modules["oracle.attention"] = sub
import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                      {tests!r}]))
"""


def _run_pins(old, new):
    code = BOOT.format(src=SRC, old=old, new=new, tests=os.path.join(ROOT, "tests", "test_oracle.py"))
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                          timeout=600)


def test_pins_pass_on_the_unpatched_copy():
    r = _run_pins("", "")
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new", MISTAKES, ids=[m[0] for m in MISTAKES])
def test_planted_mistake_fails_a_pin(name, old, new):
    assert open(SRC).read().count(old) == 1, f"{name}: text to patch not found once"
    r = _run_pins(old, new)
    assert r.returncode == 1, f"{name}: no pin failed\n" + r.stdout[-2000:] + r.stderr[-2000:]
