"""The key-range split count block_causal_attn picks (host logic, no GPU),
through tests/c_abi/split_choice, which runs the library's own host code.
Each expected count is the one measured fastest on MI355X over whole calls
with 1 .. 8 splits (or, where noted, the rule's own choice within a flat
optimum): a pin of the scheduler model against measurement."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROG = os.path.join(ROOT, "tests", "c_abi", "split_choice")
F32, BF16, FP8 = 0, 1, 2

CASES = [
    # H, D, page, dtype, n_q, q_pos0, block, n_kv, splits, what
    (5, 128, 256, BF16, 3712, 118784, 3712, 122496, 7,
     "one GPU's 5-head share of the v0.2 call: 7 measured fastest (1.074 ms; 3: 1.181, 8: 1.203)"),
    (24, 128, 256, BF16, 1024, 65536, 1024, 66560, 3,
     "v0.1 unit: 3 measured fastest (0.811 ms; 8: 0.853)"),
    (40, 128, 256, BF16, 3712, 118784, 3712, 122496, 8,
     "v0.2 unit: 8 measured fastest (caps of 4 and 6 slower)"),
    (40, 128, 256, BF16, 29696, 92800, 3712, 122496, 4,
     "8-unit catch-up, 4640 pairs: wave-count rule, 4 (52.93 ms; 3: 52.77, 8: 53.67)"),
    (40, 128, 256, FP8, 3712, 2784000, 3712, 2787712, 8, "long fp8 history"),
    (4, 128, 256, BF16, 100, 0, 16, 100, 1, "two key tiles: fewer than 4 per split, no split"),
    (4, 64, 256, F32, 100, 0, 100, 100, 1, "the fp32 path never splits"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[-1].split(":")[0] for c in CASES])
def test_split_count(case):
    if not os.path.exists(PROG):
        pytest.skip("tests/c_abi/split_choice is built by __graft_entry__.build()")
    *shape, want, what = case
    r = subprocess.run([PROG, *map(str, shape)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    assert int(r.stdout) == want, what
