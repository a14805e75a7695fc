"""Cost model of a draft-and-verify round with the full KV staged through device slots.

The pith.science record of arXiv 2605.17613 shows the speedup over full-KV inference
as a function of the KV-cache budget and of the ratio of HBM to interconnect bandwidth
(Figure 13) and the acceptance length as a function of the draft length (Figure 9);
the summary page ("What the paper found") says why: drafting on the compressed cache
is bound by HBM, the full KV's swap-in by the link, and the round overlaps the two.
This module models one round of this library's loop (round.VeriCacheLoop) from
measured component times, so that round time and accepted tokens per second can be
predicted for other horizons, link rates, slot counts and acceptance rates, and the
speedup surface drawn.

The round, as the loop runs it (one compute stream, one copy stream):
  * the copy stream stages layer l's full KV (rows [0, n)) into slot l mod R: layers
    0 .. R-1 at once, layer l >= R once the verify pass has released layer l - R;
  * the compute stream drafts k steps over the compressed cache, then runs the k-row
    verify pass layer by layer, layer l once its rows have landed;
  * then the greedy tokens, acceptance, and the cache update, and the host's sync.
The model is that schedule with constant durations: t_step per draft step, t_layer
per verified layer (for k rows), t_stage per staged layer (its bytes over the link
rate) and t_tail for what follows the last layer.  Pure arithmetic on measured
numbers: it runs on the host, never on the hot path.
"""
from dataclasses import dataclass, replace
from typing import Sequence


@dataclass(frozen=True)
class RoundCosts:
    layers: int          # decoder layers (each staged and verified once per round)
    slots: int           # device layer slots of the staged full KV
    t_step: float        # seconds per draft step (compressed-cache forward + argmax)
    t_layer: float       # seconds per layer of the k-row verify pass, full KV resident
    t_stage: float       # seconds to stage one layer's full KV over the link
    t_tail: float        # seconds after the last verified layer (tokens, accept, update, sync)

    def with_link(self, layer_bytes: float, bytes_per_s: float) -> "RoundCosts":
        """The same round over a link of another rate."""
        return replace(self, t_stage=layer_bytes / bytes_per_s)


def round_time(k: int, c: RoundCosts) -> float:
    """Seconds of one round with horizon k (c.t_layer measured at this k)."""
    R = max(1, min(c.slots, c.layers))
    draft_end = k * c.t_step
    copy_free = 0.0
    verify_end = []
    for l in range(c.layers):
        start = copy_free if l < R else max(copy_free, verify_end[l - R])
        staged = start + c.t_stage
        copy_free = staged
        ready = draft_end if l == 0 else verify_end[l - 1]
        verify_end.append(max(ready, staged) + c.t_layer)
    return verify_end[-1] + c.t_tail


def expected_commits(accept_p: float, k: int) -> float:
    """E[min(a + 1, k)] tokens committed per sequence and round when each draft is
    accepted with probability accept_p given the previous ones were (a geometric run,
    as in speculative decoding): sum_{i<k} accept_p^i."""
    if accept_p >= 1.0:
        return float(k)
    return (1.0 - accept_p ** k) / (1.0 - accept_p)


def accept_p_from_commits(commits: float, k: int) -> float:
    """The acceptance probability whose expected commits per round at horizon k equal
    `commits` (bisection; commits in [1, k])."""
    lo, hi = 0.0, 1.0
    commits = min(max(commits, 1.0), float(k))
    for _ in range(100):
        mid = 0.5 * (lo + hi)
        if expected_commits(mid, k) < commits:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def tokens_per_s(batch: int, k: int, accept_p: float, c: RoundCosts) -> float:
    """Accepted tokens per second of `batch` sequences at horizon k."""
    return batch * expected_commits(accept_p, k) / round_time(k, c)


def staged_greedy_tokens_per_s(batch: int, c: RoundCosts, t_token: float) -> float:
    """Greedy decoding that stages the whole full KV every token (the baseline the
    method is measured against when the full KV lives off the GPU): one token per
    sequence per pass of L staged layers, a 1-row forward of t_token overlapped with
    the staging the same way."""
    one = replace(c, t_step=0.0, t_layer=t_token / c.layers, t_tail=0.0)
    return batch / round_time(1, one)


def best_horizon(batch: int, horizons: Sequence[int], accept_p: float, costs_at) -> int:
    """The horizon with the most accepted tokens per second; costs_at(k) gives the
    RoundCosts of horizon k (t_layer depends on k)."""
    return max(horizons, key=lambda k: tokens_per_s(batch, k, accept_p, costs_at(k)))


def speedup_surface(batch: int, k: int, costs: RoundCosts, layer_bytes: float, t_token: float,
                    accepted_lens: Sequence[float], link_rates: Sequence[float], draft_step_scale=(1.0,)):
    """Speedup of draft-and-verify over greedy with the full KV staged every token, on a
    grid of mean accepted drafts per round, link rates (bytes/s) and draft-step cost
    factors (a smaller KV budget makes each draft step cheaper: scale t_step).  Rows
    of (accepted, link rate, step scale, speedup)."""
    out = []
    for s in draft_step_scale:
        for rate in link_rates:
            c = replace(costs.with_link(layer_bytes, rate), t_step=costs.t_step * s)
            base = staged_greedy_tokens_per_s(batch, c, t_token)
            for a in accepted_lens:
                p = accept_p_from_commits(min(a + 1.0, float(k)), k)
                out.append((a, rate, s, tokens_per_s(batch, k, p, c) / base))
    return out
