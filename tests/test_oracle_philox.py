"""Pins of the oracle's noise: Philox4x32-10 against rocRAND, and the
uniform, Gumbel and logistic maps against closed forms and statistics."""

import math
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROCRAND_HDR = "/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    """Host build of rocRAND's Philox4x32-10 engine (independent library)."""
    if not os.path.exists(ROCRAND_HDR) or shutil.which("g++") is None:
        pytest.skip("rocRAND header or g++ not available")
    exe = str(tmp_path_factory.mktemp("rr") / "rocrand_philox_ref")
    subprocess.run(["g++", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                    os.path.join(HERE, "helpers", "rocrand_philox_ref.cpp"), "-o", exe],
                   check=True, capture_output=True)

    def run(seed, subsequence, offset, count):
        out = subprocess.run([exe, str(seed), str(subsequence), str(offset), str(count)],
                             check=True, capture_output=True, text=True).stdout
        return np.array([int(x) for x in out.split()], dtype=np.uint32)

    return run


@pytest.mark.parametrize("seed,stream,step,first,count", [
    (0, 0, 0, 0, 64),
    (0, 0, 0, 3, 17),                       # starts mid-block
    (0x0123456789ABCDEF, 7, 199, 1000, 40),  # both key words in use
    (42, 0xFFFFFFFF, 0xFFFFFFFF, 0, 12),     # all-ones counter high words
    (1, 2, 3, (1 << 34) + 5, 23),            # block index above 2**32
    (2**64 - 1, 0, 5, (1 << 36) - 8, 16),
])
def test_noise_stream_matches_rocrand(rocrand_ref, seed, stream, step, first, count):
    # Element e of (seed, stream, step) is rocRAND's engine(seed,
    # subsequence=(stream << 32) | step, offset=e).next().
    ref = rocrand_ref(seed, (stream << 32) | step, first, count)
    got = oracle.noise_words(seed, stream, step, np.arange(first, first + count, dtype=np.uint64))
    np.testing.assert_array_equal(got, ref)


def test_block_function_zero_key_counter(rocrand_ref):
    words = oracle.philox4x32_10(0, 0, 0, 0, 0, 0)
    np.testing.assert_array_equal(np.array([int(w) for w in words], dtype=np.uint32),
                                  rocrand_ref(0, 0, 0, 4))


def test_uniform_closed_form():
    x = np.array([0, 0xFF, 0x100, 0xFFFFFFFF, 0x80000000, 0x7FFFFFFF], dtype=np.uint32)
    u = oracle.uniform_from_word(x)
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24
    assert u[3] == 1.0 - 2.0 ** -24
    assert u[4] == (2 ** 23 + 1) * 2.0 ** -24
    # Odd multiples of 2**-24, exact in fp32, never 0 or 1.
    allx = np.arange(0, 2 ** 32, 2 ** 8 * 997, dtype=np.uint64).astype(np.uint32)
    ua = oracle.uniform_from_word(allx)
    k = ua * 2 ** 24
    assert np.all(k == np.round(k)) and np.all(k.astype(np.int64) % 2 == 1)
    assert np.all(ua.astype(np.float32).astype(np.float64) == ua)
    assert np.all((1.0 - ua).astype(np.float32).astype(np.float64) == 1.0 - ua)
    assert ua.min() > 0 and ua.max() < 1


def test_uniform_of_low_words():
    # 0x100 >> 8 = 1 is already odd -> 2**-24; 0x200 >> 8 = 2 -> 3 * 2**-24;
    # 0x300 >> 8 = 3 -> 3 * 2**-24 (words differing in the low bit collide).
    u = oracle.uniform_from_word(np.array([0x100, 0x200, 0x300], dtype=np.uint32))
    np.testing.assert_array_equal(u * 2 ** 24, [1, 3, 3])


@pytest.fixture(scope="module")
def million_uniforms():
    return oracle.uniform_from_word(oracle.noise_words(0, 3, 11, np.arange(1_000_000)))


def test_uniform_statistics(million_uniforms):
    u = million_uniforms
    assert stats.kstest(u, "uniform").pvalue > 1e-4


def test_gumbel_moments(million_uniforms):
    g = oracle.gumbel(million_uniforms)
    n = g.size
    euler_gamma = 0.5772156649015329
    var = math.pi ** 2 / 6
    assert abs(g.mean() - euler_gamma) < 4 * math.sqrt(var / n)
    # Var of the sample variance of a Gumbel: (mu4 - sigma^4)/n, mu4 = 27/5 sigma^4.
    assert abs(g.var() - var) < 4 * math.sqrt((27 / 5 - 1) * var ** 2 / n)
    # Largest value reachable: -ln(-ln(1 - 2**-24)).
    assert g.max() <= -math.log(-math.log1p(-2.0 ** -24)) + 1e-9


def test_logistic_moments(million_uniforms):
    n_ = oracle.logistic(million_uniforms)
    n = n_.size
    var = math.pi ** 2 / 3
    assert abs(n_.mean()) < 4 * math.sqrt(var / n)
    # Logistic kurtosis: mu4 = 21/5 sigma^4.
    assert abs(n_.var() - var) < 4 * math.sqrt((21 / 5 - 1) * var ** 2 / n)
    # Antisymmetry of the map: logistic(1 - u) = -logistic(u), exactly.
    u = million_uniforms[:1000]
    np.testing.assert_array_equal(oracle.logistic(1.0 - u), -oracle.logistic(u))


def test_gumbel_max_trick():
    # argmax_k (l_k + g_k) is distributed as softmax(l): the identity that makes
    # the Gumbel-Softmax a relaxation of sampling from the logits.
    l = np.array([0.3, -1.0, 1.2, 0.0])
    n = 200_000
    e = np.arange(n * 4, dtype=np.int64).reshape(n, 4)
    g = oracle.gumbel(oracle.uniform_from_word(oracle.noise_words(5, 0, 0, e)))
    counts = np.bincount(np.argmax(l[None] + g, axis=1), minlength=4)
    p = np.exp(l) / np.exp(l).sum()
    assert stats.chisquare(counts, n * p).pvalue > 1e-4


def test_logistic_threshold_is_sigmoid():
    # P(l + n > 0) = sigmoid(l): the binary Gumbel-Softmax used for the ternary
    # mask and sign has the right hard limit.
    n = 400_000
    x = oracle.logistic(oracle.uniform_from_word(oracle.noise_words(9, 1, 2, np.arange(n))))
    for l in (-1.5, 0.0, 0.7):
        p = 1 / (1 + math.exp(-l))
        frac = np.mean(l + x > 0)
        assert abs(frac - p) < 4 * math.sqrt(p * (1 - p) / n)
