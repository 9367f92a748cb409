"""Cumulative attention score (test-only).

At every decode step each cached position i gains the attention weight it
received, averaged over the query heads of a layer and then over the layers
(gist.science summary of "Not all thinking needs HBM", methodology 2,
importance scoring).  Readings: H is the number of query heads (a softmax, and
so a weight, exists per query head) and the layer average runs over the
layers of the step; positions are logical token indices of the sequence.
Because each head's weights sum to one, one step adds exactly 1 to the sum of
a sequence's scores.
"""
from __future__ import annotations

import numpy as np


def step_increment(alphas) -> np.ndarray:
    """Score increment of one sequence for one step.

    ``alphas``: list over layers of ``[n_q][s]`` attention weights.
    Returns (1/L) * sum_l (1/n_q) * sum_h alpha_{l,h}.
    """
    L = len(alphas)
    acc = np.zeros(alphas[0].shape[1])
    for a in alphas:
        acc += a.sum(axis=0) / a.shape[0]
    return acc / L


def layer_increment(alpha: np.ndarray, weight: float) -> np.ndarray:
    """One layer call's share: weight * (1/n_q) * sum_h alpha_h (weight = 1/L)."""
    return weight * alpha.sum(axis=0) / alpha.shape[0]
