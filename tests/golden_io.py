"""Reader for the small text fixtures under tests/golden/.

Format: blocks separated by blank lines; each line is ``key: value`` where the
value is a word or a whitespace-separated list of numbers (a single number
becomes a scalar); ``#`` starts a comment.
"""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _num(tok):
    t = tok.strip()
    if t.lower() == "nan":
        return float("nan")
    if t.lower().startswith("0x"):
        return int(t, 16)
    try:
        return int(t)
    except ValueError:
        return float(t)


def load_golden(name):
    cases, cur = [], {}
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                if cur:
                    cases.append(cur)
                    cur = {}
                continue
            key, val = line.split(":", 1)
            toks = val.split()
            try:
                nums = [_num(t) for t in toks]
                cur[key.strip()] = nums if key.strip() in _LIST_KEYS or len(nums) != 1 else nums[0]
            except ValueError:
                cur[key.strip()] = val.strip()
    if cur:
        cases.append(cur)
    return cases


_LIST_KEYS = {"x", "q", "codes", "values", "w", "wq", "widths", "scales", "s_rows",
              "xq", "s_x", "s_w", "acc", "c", "y", "y_sym", "y_asym"}
