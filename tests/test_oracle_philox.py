"""Oracle Philox4x32 pinned to rocRAND's independent Philox4x32-10.

The stochastic-rounding key mapping (seed -> key, coordinates -> counter) is
the library's own reading; the generator itself is the published
Philox4x32-R of Salmon, Moraes, Dror and Shaw (SC'11).  rocRAND ships a
separate implementation of the 10-round variant; it is compiled here on the
host and called on the same (counter, key) pairs.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROCRAND_INC = "/opt/rocm/include"


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    if not os.path.exists(os.path.join(ROCRAND_INC, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.fail("rocRAND headers are missing; the Philox pin needs them")
    exe = str(tmp_path_factory.mktemp("philox") / "rocrand_philox_ref")
    cxx = shutil.which("g++")
    subprocess.check_call([cxx, "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + ROCRAND_INC,
                           os.path.join(HERE, "pins", "rocrand_philox_ref.cpp"), "-o", exe])

    def run(rows, rounds=10):
        text = "".join("%08x %08x %08x %08x %08x %08x %d\n" % (tuple(int(v) for v in r) + (rounds,)) for r in rows)
        out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
        return np.array([[int(w, 16) for w in line.split()] for line in out.strip().splitlines()], np.uint64)
    return run


def test_philox10_matches_rocrand(orc, rocrand_ref):
    rng = np.random.default_rng(7)
    rows = rng.integers(0, 2**32, size=(500, 6), dtype=np.uint64)
    # plus edge words: all zero, all ones, small counters like the SR mapping uses
    rows = np.vstack([rows, [[0] * 6, [0xFFFFFFFF] * 6, [1, 2, 3, 4, 1234, 0], [31, 127, 255, 47, 1234, 0]]])
    ref = rocrand_ref(rows)
    got = np.array([orc.philox4x32(r[:4], r[4:], 10) for r in rows], np.uint64)
    np.testing.assert_array_equal(got, ref)


@pytest.mark.parametrize("rounds", [1, 2, 3, 7, 12])
def test_philox_other_round_counts_match_rocrand_rounds(orc, rocrand_ref, rounds):
    """Round counts other than 10: rocRAND's own single round and key bump,
    applied `rounds` times (the published R-round construction)."""
    rng = np.random.default_rng(100 + rounds)
    rows = rng.integers(0, 2**32, size=(200, 6), dtype=np.uint64)
    rows = np.vstack([rows, [[0] * 6, [0xFFFFFFFF] * 6, [31, 127, 255, 47, 1234, 0]]])
    ref = rocrand_ref(rows, rounds)
    got = np.array([orc.philox4x32(r[:4], r[4:], rounds) for r in rows], np.uint64)
    np.testing.assert_array_equal(got, ref)


def test_rocrand_round_composition_equals_its_ten_round_block(rocrand_ref):
    """The pin program's composition of rocRAND's single round and key bump,
    run for 10 rounds, reproduces rocRAND's shipped ten-round block: the
    composition used for the other round counts is the generator's own."""
    rng = np.random.default_rng(99)
    rows = rng.integers(0, 2**32, size=(100, 6), dtype=np.uint64)
    np.testing.assert_array_equal(rocrand_ref(rows, -10), rocrand_ref(rows, 10))
    assert not np.array_equal(rocrand_ref(rows, 11), rocrand_ref(rows, 10))


def test_philox_zero_rounds_is_identity(orc):
    assert list(orc.philox4x32([1, 2, 3, 4], [5, 6], 0)) == [1, 2, 3, 4]


def test_philox_rounds_change_output(orc):
    a = orc.philox4x32([9, 8, 7, 6], [5, 4], 7)
    b = orc.philox4x32([9, 8, 7, 6], [5, 4], 10)
    assert list(a) != list(b)


def test_philox_output_is_uniform(orc):
    # 32-bit words over many counters: mean of u/2^32 near 1/2, each bit ~ 1/2.
    words = np.concatenate([orc.philox4x32([i, 0, 0, 0], [1234, 0], 10) for i in range(2000)]).astype(np.float64)
    u = words / 2.0**32
    assert abs(u.mean() - 0.5) < 4 * np.sqrt(1 / 12 / u.size)


@pytest.mark.parametrize("state", ["bf16", "i8"])
def test_sr_word_of_each_element_is_the_mapped_rocrand_word(orc, rocrand_ref, state):
    """Which random word each element's stochastic rounding uses (the
    library's reading of the pages' "Philox seed derivation"): counter
    ((r * dstate + c) / 4, head, request, layer), key (low, high) 32-bit words
    of the seed, output word c mod 4.  Every element sits exactly halfway
    between two codes, so it rounds up iff its word is below 2^31; the words
    come from rocRAND's generator with that mapping written out here, not
    from the oracle.  A wrong counter word, a swapped key or counter pair, or
    another output word each flip about half the elements."""
    import rssm_inputs as ri
    seed = 0x0123456789ABCDEF
    ds = 16
    spec = ri.with_(ri.CONFIGS["tiny_f32"], dstate=ds, state_dtype=state, philox_rounds=10, rand_seed=seed)
    if state == "bf16":
        row = np.full(ds, 1.0 + 2.0 ** -8, np.float32)     # halfway between bf16 1 and 1 + 2^-7
        lo, hi = 0x3F80, 0x3F81
    else:
        row = np.full(ds, 10.5, np.float32)                # row max 127: t = v, halfway between 10 and 11
        row[0] = 127.0
        lo, hi = 10, 11
    coords = [(l, b, h, r) for l in (0, 5) for b in (0, 3, 200) for h in (0, 7) for r in (0, 1, 13)]
    rows, want = [], []
    for (l, b, h, r) in coords:
        for c in range(ds):
            rows.append([(r * ds + c) // 4, h, b, l, seed & 0xFFFFFFFF, seed >> 32])
    words = rocrand_ref(np.array(rows, np.uint64))
    n_up = 0
    for i, (l, b, h, r) in enumerate(coords):
        codes, _ = orc.encode_row(spec, row, l, b, h, r)
        codes = np.asarray(codes).view(np.uint16 if state == "bf16" else np.int8).astype(np.int64)
        for c in range(ds):
            if state == "i8" and c == 0:
                continue                                   # exact 127
            u = int(words[i * ds + c][c % 4])
            expect = hi if u < 2 ** 31 else lo
            assert codes[c] == expect, f"layer {l} request {b} head {h} row {r} col {c}: code {codes[c]}, word {u:#x}"
            n_up += expect == hi
    total = len(coords) * (ds - (1 if state == "i8" else 0))
    assert 0.35 * total < n_up < 0.65 * total              # both directions occur
