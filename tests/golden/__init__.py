"""Reader for the hand-worked fixtures in this folder."""
import os
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))


def _parse_value(text):
    rows = [r.split() for r in text.split(";")]
    vals = [[Fraction(x) for x in r] for r in rows]
    if len(vals) == 1:
        return vals[0] if len(vals[0]) > 1 else vals[0][0]
    return vals


def load_cases(name="worked_steps.txt"):
    """{case name: {key: Fraction | list | list of lists}} from a fixture file."""
    cases = {}
    cur = None
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = [s.strip() for s in line.split(":", 1)]
            if key == "case":
                cur = cases.setdefault(val, {})
                continue
            cur[key] = _parse_value(val)
    return cases
