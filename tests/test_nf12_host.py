"""Host-side checks of the NF12 part of libdf11.so (no GPU needed): the
multi-threaded encoder writes exactly the NF12 oracle's bytes, and the
validator accepts the oracle's containers and rejects broken ones."""
import numpy as np
import pytest

from oracle import nf12 as nf12_oracle
import lossless_bf16_weight_amd as df11
from lossless_bf16_weight_amd import workloads as W


@pytest.mark.parametrize("n", [0, 1, 7, 8, 9, 63, 64, 65, 511, 512, 513, 4096 + 3, 100003])
def test_encoder_matches_oracle_bytes(n):
    w = W.normal_bf16((n,), seed=n)
    w[::37] = 0                     # some outlier groups
    a = df11.nf12_encode(w, threads=4)
    b = nf12_oracle.encode(w)
    assert a.size == b.size and (a == b).all()
    assert df11.nf12_validate(a) == n


def test_encoder_on_special_tensors_and_thread_counts():
    cases = [W.exhaustive_words(), W.heavy_tail_bf16((300001,), seed=2),
             np.full(1000, 0x3F80, np.uint16), np.zeros(1001, np.uint16)]
    for w in cases:
        want = nf12_oracle.encode(w)
        for t in (1, 3, 8):
            got = df11.nf12_encode(w, threads=t)
            assert got.size == want.size and (got == want).all()


def test_bound_holds():
    for n in (0, 1, 8, 9, 1000, 65536):
        w = np.zeros(n, np.uint16)       # every group an outlier: the largest container
        assert df11.nf12_encode(w).size <= df11.lib().df11_nf12_bound(n)


def test_validate_rejects_broken_containers():
    w = W.normal_bf16((8 * 1000 + 5,), seed=9)
    w[::101] = 0
    c = nf12_oracle.encode(w)
    h = nf12_oracle.header(c)
    assert df11.nf12_validate(c) == w.size and h["n_escaped"] > 0

    def status(mut, cut=None):
        x = c.copy()
        mut(x)
        if cut is not None:
            x = x[:cut]
        return df11.lib().df11_nf12_validate(x.ctypes.data, x.size, None)

    E_FORMAT, E_UNSUPPORTED = 2, 3
    assert status(lambda x: x.__setitem__(0, ord("X"))) == E_FORMAT
    assert status(lambda x: x.__setitem__(8, 2)) == E_UNSUPPORTED
    assert status(lambda x: x.__setitem__(12, 1)) == E_UNSUPPORTED
    assert status(lambda x: x.__setitem__(32, x[32] + 1)) == E_FORMAT        # outlier count vs layout
    assert status(lambda x: x.__setitem__(120, 1)) == E_FORMAT                # reserved header byte
    assert status(lambda x: x.__setitem__(h["off_flags"], x[h["off_flags"]] ^ 2)) == E_FORMAT
    assert status(lambda x: x.__setitem__(h["off_prefix"] + 4, x[h["off_prefix"] + 4] ^ 1)) == E_FORMAT
    pad = h["off_slots"] + 12 * h["n_groups"]          # the first padding byte after the slots
    assert pad < h["off_flags"]
    assert status(lambda x: x.__setitem__(pad, 7)) == E_FORMAT
    # header-only validation: the layout is checked, the sections are not
    assert status(lambda x: x.__setitem__(h["off_prefix"] + 4, x[h["off_prefix"] + 4] ^ 1), cut=256) == 0
    assert status(lambda x: x.__setitem__(24, x[24] ^ 1), cut=256) == E_FORMAT
    assert status(lambda x: None, cut=255) == E_FORMAT


def test_encoder_matches_oracle_on_random_distributions():
    """60 seeded random exponent distributions (random sizes, random
    exponent sets, so that anything from no group to every group escapes):
    the product encoder's bytes equal the NF12 oracle's."""
    from exponent_mixes import random_exponent_case
    for seed in range(60):
        w = random_exponent_case(seed, 120_000)
        a = df11.nf12_encode(w, threads=4)
        b = nf12_oracle.encode(w)
        assert a.size == b.size and (a == b).all(), seed
        assert df11.nf12_validate(a) == w.size
