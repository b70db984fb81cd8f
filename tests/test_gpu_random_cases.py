"""Seeded random combinations of the layer's options, prefill and decode,
against the fp64 oracle on every value head: sequence counts and lengths
around the chunk boundaries, head groupings, fp32 or bf16 I/O, conv and gate
on or off, seeded or zero initial and conv states, either launch form (and,
for decode, either state dtype).  Each case draws its options from its own
seed, so a failure names a reproducible case."""
import numpy as np
import pytest

import gdn_synth as gs
from helpers import check_prefill, say
from test_gpu_decode import check_decode

pytestmark = pytest.mark.gpu

# lengths near the chunk grid's edges, and a few longer ones
_LENS = [0, 1, 2, 3, 5, 63, 64, 65, 127, 128, 129, 191, 250, 333]


def _prefill_case(seed):
    rng = np.random.default_rng(seed)
    io = gs.F32 if rng.random() < 0.25 else gs.BF16
    Hk = int(rng.choice([1, 2, 3, 4]))
    Hv = Hk * int(rng.choice([1, 2]))
    lens = [int(rng.choice(_LENS)) for _ in range(int(rng.integers(1, 5)))]
    l2 = bool(rng.random() < 0.8)
    p = gs.Problem(f"random-prefill-{seed}", lens, Hk=Hk, Hv=Hv, io=io,
                   conv=bool(rng.random() < 0.75), gate=bool(rng.random() < 0.75),
                   l2norm=l2, prenormalize_qk=not l2,
                   init_state_std=0.01 if rng.random() < 0.6 else None,
                   conv_state_std=0.01 if rng.random() < 0.5 else None,
                   seed=seed)
    separate = bool(rng.random() < 0.3)
    return p, separate


@pytest.mark.parametrize("seed", range(7100, 7112))
def test_random_prefill(seed):
    p, separate = _prefill_case(seed)
    say(f"seed {seed}: separate launches {separate}")
    rep = check_prefill(p, gs.generate(p), separate_launches=separate)
    say(f"  {rep}")


def _decode_case(seed):
    rng = np.random.default_rng(seed)
    Hk = int(rng.choice([1, 2, 4]))
    Hv = Hk * int(rng.choice([1, 2]))
    N = int(rng.integers(1, 40))
    return gs.Problem(f"random-decode-{seed}", [1] * N, Hk=Hk, Hv=Hv,
                      state_dtype=gs.BF16 if rng.random() < 0.5 else gs.F32,
                      conv=bool(rng.random() < 0.5), gate=bool(rng.random() < 0.5),
                      init_state_std=0.01, conv_state_std=0.01, seed=seed, decode=True)


@pytest.mark.parametrize("seed", range(7200, 7206))
def test_random_decode(seed):
    p = _decode_case(seed)
    e_out, e_st = check_decode(p, gs.generate(p))
    say(f"seed {seed}: conv {p.conv} gate {p.gate} state {p.state_dtype}: out {e_out:.2e} state {e_st:.2e}")
