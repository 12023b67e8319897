"""Speculative-round accounting (test infrastructure only).

Closed forms from the speculative-decoding e-book; used to pin the acceptance
stage (Monte Carlo against the expected-tokens formula) and to read measured
costs.  Float64 throughout.
"""
from __future__ import annotations

__all__ = ["expected_tokens", "speedup", "best_gamma", "rounds_from_flags"]


def expected_tokens(alpha: float, gamma: int) -> float:
    """Expected tokens per round with independent acceptance probability alpha
    per drafted position: sum_{i=0..gamma} alpha^i = (1 - alpha^(gamma+1)) /
    (1 - alpha); at alpha = 1 the closed form is 0/0 and the value is gamma+1
    [SD-E]."""
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def speedup(alpha: float, gamma: int, c_draft: float, c_verify: float) -> float:
    """Tokens per round divided by the cost of a round, gamma draft passes plus
    one verify pass, in units of one target pass [SD-default]."""
    return expected_tokens(alpha, gamma) / (gamma * c_draft + c_verify)


def best_gamma(alpha: float, c_draft: float, c_verify: float, gmax: int = 32) -> int:
    """The gamma in 0..gmax with the largest modelled speedup [SD-gamma],
    [SD-peak]."""
    return max(range(gmax + 1), key=lambda g: (speedup(alpha, g, c_draft, c_verify), -g))


def rounds_from_flags(flags: str, gamma: int):
    """Split an acceptance-flag string into rounds: each round reads flags until
    a 0 or until gamma flags were read [SD-flags].  Returns the accepted count
    of each round."""
    out, i = [], 0
    while i < len(flags):
        a = 0
        while a < gamma and i < len(flags):
            f = flags[i]
            i += 1
            if f == "1":
                a += 1
            else:
                break
        out.append(a)
    return out
