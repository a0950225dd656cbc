"""CPU checks of the inputs that drive the GPU online-softmax tests
(tests/test_gpu_online_softmax.py; inputs and replay in tests/softmax_cases.py).

* Every call's ``spike`` and ``ramp`` inputs make every query row take at least
  one rescale of its running maximum (the replay of the kernels' rule: a
  step's largest logit beats the running maximum by more than 8 log2 units,
  after the wave's first step), under the wave arrangement the library picks
  for that call; ``wide`` inputs make at least 90 % of the rows take one.
* Those inputs catch a mistake in the rescale: streaming the softmax with the
  kernels' raise rule in exact arithmetic matches the oracle, while the same
  stream with the rescale factor left at 1, or the running sum or the
  accumulators not rescaled, breaks the parity bounds the GPU tests apply;
  with ``spike`` inputs (the mass before the rise is comparable to the mass
  after it) so does e^-dm in place of 2^-dm.  (The online softmax is exact: §4.2 of the
  ialgorithm.me page.)
"""
import numpy as np
import pytest

import oracle
import softmax_cases as sc
from parity_bounds import violations


@pytest.mark.parametrize("name", [c.name for c in sc.CASES])
def test_rescale_patterns_force_a_rescale(name):
    c = sc.CASE_BY_NAME[name]
    for pattern in (p for p in sc.RESCALE_PATTERNS if p in sc.patterns_for(c.kind)):
        inp = sc.build(c, pattern, 4000 + sc.CASES.index(c))
        n = sc.rescales(inp)
        if pattern == "wide":
            assert (n >= 1).mean() >= 0.9, f"{name} wide: {(n == 0).mean():.3f} of rows without"
        else:
            assert n.min() >= 1, f"{name} {pattern}: a row takes no rescale"


def stream_rows(inp, mistake):
    """The streamed softmax of every (sequence, draft token, head) row, one
    wave walking every step of the context in order."""
    c, w = inp.case, inp.w
    B, T, Hq, d = inp.q.shape
    G = c.group
    out = np.zeros((B, T, Hq, d))
    for s in range(B):
        L = int(w.context_lens[s])
        for g in range(c.num_kv_heads):
            K = sc.key_rows(inp, s, g, L)
            V = oracle.widen(oracle.v_rows(w.v_pool, w.block_tables[s], L, g), c.dtype)
            for i in range(T):
                lim = sc.visible(L, T, i)
                q = oracle.widen(inp.q[s, i, g * G:(g + 1) * G], c.dtype)
                x = float(np.float32(inp.scale)) * sc.LOG2E * (q @ K[:lim].T)
                out[s, i, g * G:(g + 1) * G] = sc.stream_softmax(x, V[:lim], mistake)
    return out


MISTAKES = ("alpha_one", "sum_not_rescaled", "acc_not_rescaled", "alpha_natural")


@pytest.mark.parametrize("name,pattern", [("bf16-reg4-gqa8", "spike"), ("f16-reg8-mha", "spike"),
                                          ("f32-reg4-mha-d64", "spike"),
                                          ("k8-bf16-reg4", "spike"), ("k2-f16-reg4", "spike"),
                                          ("bf16-reg4-gqa8", "ramp")])
def test_rescale_mistakes_break_the_bounds(name, pattern):
    c = sc.CASE_BY_NAME[name]
    inp = sc.build(c, pattern, 4000 + sc.CASES.index(c))
    want = sc.oracle_out(inp)
    right = stream_rows(inp, None)
    assert np.abs(right - want).max() < 1e-9, "the exact stream is the oracle's result"
    for mistake in MISTAKES if pattern == "spike" else MISTAKES[:3]:
        got = stream_rows(inp, mistake)
        n_bad, max_abs, _ = violations(got, want, c.dtype)
        print(f"{name} {pattern} {mistake}: max-abs {max_abs:.3e}, {n_bad} elements outside")
        assert n_bad > 0, f"{mistake} passes the bounds on {name} {pattern}"
