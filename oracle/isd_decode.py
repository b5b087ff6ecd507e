"""Plain CPU oracle for the multi-step ISD decoding loop around the step.

TEST INFRASTRUCTURE ONLY, like ``isd_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may use it,
and it imports nothing from the product path.

Sources (cited by page title and section):

* "Introspective Diffusion Language Models | Summary", section 3.2
  "Introspective Strided Decoding (ISD)": the loop around the step.  A step
  whose L proposals all pass (accept_len == L) also yields a bonus token from
  its anchor row L; a step with a rejection leaves the sequence in a state
  whose next step verifies nothing and only makes proposals.
* same page, section 3.2 (tokens per forward) and appendix B "TPF and Compute
  Overhead Analysis": with cumulative acceptance probabilities P_k the tokens
  per forward of stride N are (2 + P_1 + ... + P_{N-2}) / (2 - P_{N-1}); under
  uniform acceptance a, P_k = a^k.  The appendix derives it from a renewal
  cycle: one proposal-only step, then verify-and-propose steps until a
  rejection.

Reading of the pages: stride N means L = N - 1 proposals per step.
A sequence is in one of two states.  In the *recovery* state its step draws
one token from its anchor row (the last clean position) and proposes L
tokens; it then verifies.  In the *verify* state its step checks its L
pending proposals with the ISD rule: a rejection at j < L emits j accepted
tokens plus the correction (j + 1 tokens) and moves it to recovery; accepting
all L emits them plus a bonus token drawn from the (L+1)-th anchor row
(L + 1 tokens) and keeps it in the verify state with the new proposals.
"""

from __future__ import annotations

import numpy as np

from . import isd_oracle as O

RECOVER = 0
VERIFY = 1


def ledger_step(state: np.ndarray, accept_len: np.ndarray, L: int):
    """One step of the loop's bookkeeping.

    state: [C] RECOVER or VERIFY before the step; accept_len: [C] first
    rejected position j of verifying sequences (ignored for recovering ones).
    Returns (emitted [C], next_state [C], bonus_mask [C], anchor_mask [C]):
    the tokens the step emits, the state after it, and which sequences draw a
    bonus token (all L accepted) or an anchor token (recovery step).
    """
    state = np.asarray(state)
    j = np.asarray(accept_len)
    verifying = state == VERIFY
    all_acc = verifying & (j == L)
    emitted = np.where(verifying, np.where(all_acc, L + 1, j + 1), 1)
    next_state = np.where(verifying & ~all_acc, RECOVER, VERIFY)
    return emitted.astype(np.int64), next_state.astype(np.int32), all_acc, ~verifying


def decode_step(state, p, q, x, ua, ur, qn, up, ub, uz, temperature=1.0):
    """One batched step of the loop (sample mode), on decoded float64 logits.

    p: [C, L+1, V] anchor rows (rows 0..L-1 score the pending proposals of a
    verifying sequence; row L is its bonus anchor; row 0 is the anchor of a
    recovering sequence).  q, qn: [C, L, V]; x: [C, L] pending proposals;
    ua, ur, up: [C, L]; ub, uz: [C] uniforms of the bonus and anchor draws.
    Returns a dict with the step's verify outputs (only meaningful for
    verifying sequences), the bonus / anchor tokens (-1 where not drawn), the
    next proposals, the emitted counts and the next state.
    """
    C, L1, V = p.shape
    L = L1 - 1
    v = O.verify_sample(p[:, :L], q, x, ua, ur, temperature)
    bonus, _, bonus_margin, _ = O.propose_sample(p[:, L:L + 1], ub[:, None], temperature)
    anchor, _, anchor_margin, _ = O.propose_sample(p[:, 0:1], uz[:, None], temperature)
    nxt, _, next_margin, _ = O.propose_sample(qn, up, temperature)
    emitted, next_state, bmask, amask = ledger_step(state, v["accept_len"], L)
    verifying = np.asarray(state) == VERIFY
    return dict(
        accept_len=np.where(verifying, v["accept_len"], -1),
        out_tokens=np.where(verifying[:, None], v["out_tokens"], -1),
        flagged=verifying & v["flagged"],
        resid_flagged=verifying & v["resid_flagged"],
        bonus=np.where(bmask, bonus[:, 0], -1),
        bonus_flagged=bmask & (bonus_margin[:, 0] < O.TIE_WINDOW),
        anchor=np.where(amask, anchor[:, 0], -1),
        anchor_flagged=amask & (anchor_margin[:, 0] < O.TIE_WINDOW),
        next_tokens=nxt,
        next_flagged=next_margin < O.TIE_WINDOW,
        emitted=emitted,
        next_state=next_state,
    )


def tpf_closed_form(a: float, N: int) -> float:
    """Tokens per forward of stride N under uniform acceptance a (the
    appendix's renewal result, written as printed)."""
    if N < 2:
        raise ValueError("stride N must be >= 2")
    num = 2.0 + sum(a ** k for k in range(1, N - 1))
    return num / (2.0 - a ** (N - 1))


def tpf_stationary(a: float, N: int) -> float:
    """The same quantity from the two-state chain of this module's reading:
    the long-run tokens per forward, i.e. the stationary mean reward."""
    L = N - 1
    all_acc = a ** L
    # verify state: reject at j < L with probability a^j (1 - a), else all accepted
    tok_verify = sum((j + 1) * a ** j * (1.0 - a) for j in range(L)) + (L + 1) * all_acc
    # transitions: recovery -> verify always; verify -> recovery with 1 - a^L
    pi_recover = (1.0 - all_acc) / (2.0 - all_acc)
    pi_verify = 1.0 / (2.0 - all_acc)
    return pi_recover * 1.0 + pi_verify * tok_verify
