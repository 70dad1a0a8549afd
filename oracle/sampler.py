"""CPU oracle of the sampling suffix of the decode step.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the tests and the smoke check may use it; it shares
nothing with the HIP path.

Source: "Models, Registry and the Driver" page, section "The Driver", item "The sampling suffix", and the
"Backends" page, section "ROCm (AMD)". The rules named there -- greedy and temperature draws with top-k, top-p and
min-p cuts, the repetition, presence and frequency penalties with a logit bias taken from each sequence's token
history (kept on the device and grown by each drawn token), and the top-n logprobs -- come without formulas, so
each rule below is the plainest reading of its name, and the kernel follows the same readings:

* adjusted logits, per token v with history count c_v and bias b_v:
  z_v = r(l_v) - presence * [c_v > 0] - frequency * c_v + b_v, where r(x) = x / rep if x > 0 else x * rep when
  c_v > 0 (the repetition penalty shrinks a seen token's logit toward zero from either side), r(x) = x otherwise.
  A NaN logit counts as -inf (never drawn);
* temperature 0: greedy, the first index of the largest z;
* temperature T > 0: s = z / T; tokens ranked by (s descending, index ascending); top-k keeps the k best ranked
  (k = 0: all); their probabilities q = softmax(s) over the kept tokens; top-p keeps the shortest ranked prefix
  whose cumulative q reaches p (p = 1: all); min-p keeps the tokens with q >= min_p * q_max (min_p = 0: all);
* the draw: u in [0, 1); the kept tokens in INDEX order, weights q; the token is the first whose running weight
  exceeds u times the kept total (an inverse CDF; the order of the walk does not change the distribution);
* u: the d-th output of SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
  2014) seeded with the row's seed, d = the row's draw count; its top 24 bits, times 2^-24;
* logprobs: log-softmax of s over every token (T = 1 for greedy), the top-n by rank, and the drawn token's.
"""
from __future__ import annotations

import numpy as np

__all__ = ["splitmix64", "uniform", "adjust", "keep_set", "draw", "sample", "logprobs"]

_M64 = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def splitmix64(seed: int, d: int) -> int:
    """Output d (0-based) of the SplitMix64 sequence whose state starts at `seed`: the state advances by the golden
    gamma before each output, and each output is the state through the generator's two xor-shift-multiply rounds
    and a final xor-shift."""
    z = (seed + (d + 1) * _GAMMA) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def uniform(seed: int, d: int) -> float:
    """The draw's u: the top 24 bits of output d, times 2^-24 (exactly representable in float32)."""
    return (splitmix64(seed, d) >> 40) * 2.0 ** -24


def adjust(logits, counts, bias, rep: float = 1.0, presence: float = 0.0, frequency: float = 0.0) -> np.ndarray:
    """Adjusted logits z (float64): penalties from the history counts, then the bias; NaN -> -inf."""
    l = np.asarray(logits, np.float64).copy()
    l[np.isnan(l)] = -np.inf
    c = np.asarray(counts, np.float64)
    seen = c > 0
    r = np.where(l > 0, l / rep, l * rep)
    z = np.where(seen, r, l) - presence * seen - frequency * c
    return z + (np.asarray(bias, np.float64) if bias is not None else 0.0)


def _ranked(s: np.ndarray) -> np.ndarray:
    """Token indices by (s descending, index ascending)."""
    return np.lexsort((np.arange(s.size), -s))


def keep_set(z: np.ndarray, temperature: float, top_k: int = 0, top_p: float = 1.0, min_p: float = 0.0):
    """The tokens a temperature draw may pick and their (unnormalized) weights: (indices ascending, weights)."""
    s = z / temperature
    order = _ranked(s)
    if top_k > 0:
        order = order[:top_k]
    finite = np.isfinite(s[order])
    order = order[finite] if finite.any() else order[:1]
    q = np.exp(s[order] - s[order[0]])
    q /= q.sum()
    if top_p < 1.0:
        m = int(np.searchsorted(np.cumsum(q), top_p))   # first ranked prefix whose cumulative q >= top_p
        order, q = order[:m + 1], q[:m + 1]
    if min_p > 0.0:
        keep = q >= min_p * q[0]
        order, q = order[keep], q[keep]
    by_index = np.argsort(order, kind="stable")
    return order[by_index], q[by_index]


def draw(kept: np.ndarray, weights: np.ndarray, u: float) -> int:
    """Inverse CDF in index order: the first kept token whose running weight exceeds u * total."""
    run = np.cumsum(weights)
    i = int(np.searchsorted(run, u * run[-1], side="right"))
    return int(kept[min(i, kept.size - 1)])


def sample(logits, counts, bias, *, temperature=0.0, top_k=0, top_p=1.0, min_p=0.0, rep=1.0, presence=0.0,
           frequency=0.0, seed=0, d=0) -> int:
    """The token the suffix picks for one row (greedy at temperature 0)."""
    z = adjust(logits, counts, bias, rep, presence, frequency)
    if temperature == 0.0:
        if not np.isfinite(z).any() and np.isnan(z).all():
            return 0
        return int(np.argmax(z))
    kept, w = keep_set(z, temperature, top_k, top_p, min_p)
    return draw(kept, w, uniform(seed, d))


def logprobs(z: np.ndarray, temperature: float, n: int, token: int):
    """(top-n token ids by rank, their logprobs, the drawn token's logprob) of log-softmax(z / T) (T = 1 when 0)."""
    t = temperature if temperature > 0.0 else 1.0
    s = z / t
    m = np.max(s)
    lse = m + np.log(np.sum(np.exp(s - m)))
    lp = s - lse
    top = _ranked(s)[:n]
    return top, lp[top], float(lp[token])
