"""Plain CPU oracle of the sampled selection (temperature and top-p) that
replaces the greedy argmax at the end of a window step.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It shares no code with
the HIP path and imports nothing from it.

The RK3588 page ("LocateAnything-3B for RK3588 (RKLLM + RKNN)", section
"Usage (on the board)", and its "Evaluation" section) runs the model with the
original sampling defaults, temperature 0.7, top-p 0.9 and repetition penalty
1.1, and warns that greedy decoding rarely terminates; the Jetson page (Part 1
section 1.4) notes that the model's sampler falls back to greedy selection
when the temperature is not positive.  The pages fix no formula, so this is the
plain one (standard nucleus sampling), in float64:

1. z_v: the row's logits (after the repetition penalty, when one is used);
2. p_v proportional to exp(z_v / T), T > 0 the temperature;
3. the nucleus: order the vocabulary by z descending, equal logits by lower
   id first, and keep the shortest prefix whose probability reaches top_p
   (never fewer than one token);
4. the draw: one uniform u in [0, 1) per row; among the kept ids in ascending
   id order, the first whose running kept probability exceeds u times the
   kept probability is selected.
T <= 0 selects the argmax (lowest id on a tie).

Random numbers: u comes from Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC 2011), a counter-based
generator written here from its published definition: ten rounds, each
multiplying two of the four 32-bit counter words by 0xD2511F53 and 0xCD9E8D57
and mixing the high halves with the other two words and the key, the key
advanced by 0x9E3779B9 and 0xBB67AE85 between rounds.  Row t of a step with
seed s and offset o draws from counter (t, o mod 2^32, o div 2^32, 0) and key
(s mod 2^32, s div 2^32); u is the top 24 bits of the first output word
times 2^-24.

Pins (tests/test_oracle_pins.py): the generator's known-answer vectors of the
Random123 distribution; a hand-worked nucleus and draw; ties at the nucleus
boundary; T -> 0 equals the argmax; top_p = 1 and top_p -> 0 limits; the
empirical frequencies of many draws against the renormalised nucleus.
"""
from __future__ import annotations

import numpy as np

__all__ = ["philox4x32_10", "philox_uniform", "nucleus", "sample_row", "sample_rows"]

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """Philox4x32 with 10 rounds: counter (4 uint32), key (2 uint32) -> 4 uint32."""
    c = [int(x) & _MASK for x in counter]
    k = [int(x) & _MASK for x in key]
    for r in range(10):
        if r:
            k = [(k[0] + _W0) & _MASK, (k[1] + _W1) & _MASK]
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        c = [(p1 >> 32) ^ c[1] ^ k[0], p1 & _MASK, (p0 >> 32) ^ c[3] ^ k[1], p0 & _MASK]
    return c


def philox_uniform(row, seed, offset):
    """The uniform draw of window row ``row`` for (seed, offset): top 24 bits of
    the first Philox output word, times 2^-24 (exact in float32 and float64)."""
    x = philox4x32_10([row, offset & _MASK, (offset >> 32) & _MASK, 0], [seed & _MASK, (seed >> 32) & _MASK])
    return (x[0] >> 8) * 2.0 ** -24


def nucleus(z, temperature, top_p):
    """(kept ids in ascending order, their probabilities p_v (unnormalised
    exp((z_v - max z) / T)), total probability of all ids) of one row."""
    z = np.asarray(z, dtype=np.float64)
    p = np.exp((z - z.max()) / float(temperature))
    total = p.sum()
    order = np.lexsort((np.arange(z.size), -z))   # z descending, lower id first on ties
    cum = np.cumsum(p[order])
    n = int(np.searchsorted(cum, float(top_p) * total, side="left")) + 1
    n = min(max(n, 1), z.size)
    kept = np.sort(order[:n])
    return kept, p[kept], total


def sample_row(z, temperature, top_p, u):
    """The selected id of one row of logits for the uniform draw u."""
    z = np.asarray(z, dtype=np.float64)
    if not temperature > 0:
        return int(np.argmax(z))
    kept, pk, _ = nucleus(z, temperature, top_p)
    cum = np.cumsum(pk)
    i = int(np.searchsorted(cum, u * cum[-1], side="right"))
    return int(kept[min(i, kept.size - 1)])


def sample_rows(logits, temperature, top_p, seed, offset):
    """Selected ids of every row of ``logits`` [T, V] (row t draws with row index t)."""
    logits = np.asarray(logits)
    return np.array([sample_row(logits[t], temperature, top_p, philox_uniform(t, seed, offset))
                     for t in range(logits.shape[0])], dtype=np.int64)
