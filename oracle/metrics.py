"""Reported-metric identities (oracle; test infrastructure only).

Speedup = acceleration rate / overhead, where the acceleration rate is the
average number of tokens committed per decoding step and the overhead is the
per-step latency relative to one vanilla decoding step (Medusa paper digest,
Results, app. B.1; wq-win lecture note, section 四, evidence 1).  With times,
speedup = A * T_base / T_tree (zwxr blog, section 3.1): tokens per round
times the vanilla time per token over the time of one tree round.
"""
from __future__ import annotations


def speedup(tokens_per_step: float, overhead: float) -> float:
    return tokens_per_step / overhead


def overhead(t_step: float, t_vanilla: float) -> float:
    return t_step / t_vanilla
