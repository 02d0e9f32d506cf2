"""Reader for the small ``key = value`` fixtures in this folder."""
import os

HERE = os.path.dirname(__file__)


def load(name: str) -> dict:
    out = {}
    with open(os.path.join(HERE, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            nums = [float(t) if "." in t else int(t) for t in val.split()]
            out[key] = nums[0] if len(nums) == 1 else nums
    return out
