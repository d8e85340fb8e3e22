"""Seeded operation traces for the block manager: branch trees of parallel sampling and beam
search, and a request stream for continuous batching.

Pages cited:
  P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html (explainer, sections 1-9)
  P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html (article, sections 1-5)

A trace says which sequences start, fork, finish and take a token at each step. It decides
nothing that depends on a block manager's state and holds none of the paging arithmetic
(slots, blocks, copies): both the C++ manager and the reference model replay the same trace.

Trees (P2 §2.2: branches share their parent's blocks until one writes into a shared block):
  - parallel sampling: one prompt, n branches forked from it; every branch takes one token per
    step until it stops (each step it stops with probability stop_prob, or at max_new);
  - beam search: `width` beams; each step every live beam proposes `width` continuations whose
    scores add an independent log-uniform increment to the beam's score; the `width` best of
    all proposals survive. A beam with no surviving continuation finishes (its sequence is
    freed); one with c > 0 survivors continues as the first and forks c - 1 children; then
    every surviving beam takes one token.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass
class TreeStep:
    frees: list = field(default_factory=list)      # sequences finished before the forks
    forks: list = field(default_factory=list)      # (parent, child), in order
    appends: list = field(default_factory=list)    # sequences that take one token, in order


@dataclass
class TreeTrace:
    kind: str
    prompt_len: int
    root: int
    steps: list                                   # [TreeStep]


def parallel_sampling_trace(rng: np.random.Generator, prompt_len: int, branches: int,
                            max_new: int, stop_prob: float = 0.0, root: int = 0) -> TreeTrace:
    steps = []
    first = TreeStep(forks=[(root, root + i) for i in range(1, branches)])
    live = list(range(root, root + branches))
    produced = 0
    while live and produced < max_new:
        st = first if produced == 0 else TreeStep()
        if produced > 0:
            stopped = [s for s in live if rng.random() < stop_prob]
            st.frees = stopped
            live = [s for s in live if s not in stopped]
        st.appends = list(live)
        steps.append(st)
        produced += 1
    steps.append(TreeStep(frees=list(live)))
    return TreeTrace("parallel_sampling", prompt_len, root, steps)


def beam_search_trace(rng: np.random.Generator, prompt_len: int, width: int, steps: int,
                      root: int = 0) -> TreeTrace:
    beams = [root]
    score = {root: 0.0}
    next_id = root + 1
    out = []
    for _ in range(steps):
        cand = []                                 # (score, parent, rank within parent)
        for b in beams:
            inc = np.log(rng.random(width))
            for r in range(width):
                cand.append((score[b] + float(inc[r]), b, r))
        cand.sort(key=lambda c: (-c[0], c[1], c[2]))
        kept = cand[:width]
        st = TreeStep()
        children = {b: [c for c in kept if c[1] == b] for b in beams}
        st.frees = [b for b in beams if not children[b]]
        new_beams, new_score = [], {}
        for b in beams:
            for i, c in enumerate(children[b]):
                if i == 0:
                    sid = b
                else:
                    sid = next_id
                    next_id += 1
                    st.forks.append((b, sid))
                new_beams.append(sid)
                new_score[sid] = c[0]
        st.appends = list(new_beams)
        out.append(st)
        beams, score = new_beams, new_score
    out.append(TreeStep(frees=list(beams)))
    return TreeTrace("beam_search", prompt_len, root, out)


@dataclass
class Request:
    req_id: int
    arrival: int          # step at which the request becomes visible to the scheduler
    prompt_len: int
    output_len: int       # decode tokens it produces before finishing


def request_stream(rng: np.random.Generator, num_requests: int, arrivals_per_step: float,
                   prompt_range: tuple, output_mean: float, output_max: int) -> list:
    """Poisson arrivals (mean arrivals_per_step per step), prompt lengths uniform on
    prompt_range (inclusive), output lengths geometric with the given mean, clipped to
    [1, output_max]."""
    reqs, step = [], 0
    while len(reqs) < num_requests:
        for _ in range(int(rng.poisson(arrivals_per_step))):
            if len(reqs) == num_requests:
                break
            p = int(rng.integers(prompt_range[0], prompt_range[1] + 1))
            o = int(min(output_max, max(1, rng.geometric(1.0 / output_mean))))
            reqs.append(Request(len(reqs), step, p, o))
        step += 1
    return reqs
