"""Plain CPU oracle for the Introspective Strided Decoding (ISD) verify-and-propose step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(``libisd`` and its Python binding) never imports, links or calls it, and this
module imports nothing from the product path: the two share no code.

Everything here is float64 numpy evaluated on exactly decoded inputs, written
as the plain definitions, with no blocking, fusion or reordering.

Sources (cited by page title and section):

* "Introspective Diffusion Language Models | Summary" (greeksharifa.github.io),
  section 2 "Background and Motivation": the introspective acceptance rate
  alpha is the mean over the L proposed positions of min(1, p_k(x_k)/q_k(x_k)),
  where q_k is the distribution that generated x_k and p_k is the causal anchor
  that scores it once the tokens are revealed.
* same page, section 3.2 "Introspective Strided Decoding (ISD)": each proposal
  is kept with probability min(1, p_k(x_k)/q_k(x_k)); at the first rejection a
  replacement is drawn from the normalised residual max(0, p_k - q_k) and every
  later proposal is dropped; the mask positions of the same forward pass give
  the proposals of the next step.
* same page, section 3.3 "I-DLM Serving Stack": the serving stack proposes by
  argmax and verifies strictly, so the acceptance test must use the law of the
  proposal mechanism that was actually used (greedy mode below).

Readings where the pages leave a step open (each one is listed in the design doc):

* draws: one uniform per decision, passed in as an input (``ua`` for the
  accept test, ``ur`` for the residual draw, ``up`` for each proposal draw);
  a proposal is accepted iff ``ua < r`` (strict), so r = 1 always accepts;
* the residual and proposal draws are inverse-CDF draws over ascending vocab
  index: the token is the smallest i with cum_i > u * Z (cumulative of the
  weights, Z their total), clamped to the last positive weight when rounding
  pushes the target past the end;
* the residual uses ``ur[c, j]`` at the first rejected position j;
* alpha is averaged over all L positions, not only up to the first rejection;
* if the proposal probability q_k(x_k) is 0 the ratio is 1 when p_k(x_k) > 0
  and 0 otherwise; if the residual mass Z is 0 the draw falls back to p_k and
  the sequence is flagged;
* no bonus token: a step that accepts all L proposals emits exactly L tokens;
* greedy mode: argmax of the raw anchor logits with ties to the lowest index,
  a proposal is accepted iff it equals that argmax, the correction is the
  anchor argmax at the first mismatch, alpha is the match fraction, and the
  next proposals are the argmax of the mask-position logits.

Near-tie flags: a decision whose margin (|u - r| for the accept test, distance
of u to the two cumulative boundaries of the chosen token for a draw) is below
``TIE_WINDOW`` is reported so that a comparison can leave it out.
"""

from __future__ import annotations

import numpy as np

TIE_WINDOW = 1e-6
# Gumbel-max draws are flagged when the best two perturbed log-weights are this close.
GUMBEL_WINDOW = 1e-4


# ---------------------------------------------------------------------------
# Input decoding
# ---------------------------------------------------------------------------

def decode_logits(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of a logits buffer.

    ``dtype`` is ``"bf16"`` (raw holds the uint16 bit patterns) or ``"f32"``.
    A bf16 value is the upper half of the float32 with the same bits.
    """
    if dtype == "bf16":
        bits = np.asarray(raw, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Distributions
# ---------------------------------------------------------------------------

def softmax(logits: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """softmax(logits / T) along the last axis, in float64.

    -inf logits get probability 0.  NaN or +inf logits, or a row that is all
    -inf, have no defined distribution and raise ``ValueError``.
    """
    a = np.asarray(logits, dtype=np.float64) / float(temperature)
    if np.isnan(a).any() or np.isposinf(a).any():
        raise ValueError("logits contain NaN or +inf")
    m = a.max(axis=-1, keepdims=True)
    if np.isneginf(m).any():
        raise ValueError("a logits row is entirely -inf")
    e = np.exp(a - m)
    return e / e.sum(axis=-1, keepdims=True)


def cdf_interval(weights: np.ndarray, index: int):
    """The interval [cum_{i-1} / Z, cum_i / Z] of token i in the inverse-CDF
    draw over ``weights`` [V] (cum the running sum in ascending index, Z the
    total, cum_{-1} = 0): the uniforms u for which the draw picks i are those
    with cum_{i-1} <= u Z < cum_i."""
    w = np.asarray(weights, dtype=np.float64)
    cum = np.cumsum(w)
    total = cum[-1]
    lo = cum[index - 1] if index > 0 else 0.0
    return lo / total, cum[index] / total


def inverse_cdf(weights: np.ndarray, u: np.ndarray):
    """Inverse-CDF draw over ascending index, batched over leading axes.

    Returns ``(index, margin, total)``: ``index`` is the smallest i with
    cum_i > u * Z where cum is the running sum of ``weights`` and Z its total;
    when no such i exists (rounding), the last index with positive weight.
    ``margin`` is min(|cum_{i-1}/Z - u|, |cum_i/Z - u|) with cum_{-1} = 0.
    Rows whose total is 0 get index -1 and margin 0.
    """
    w = np.asarray(weights, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    cum = np.cumsum(w, axis=-1)
    total = cum[..., -1]
    target = u * total
    idx = np.sum(cum <= target[..., None], axis=-1)
    V = w.shape[-1]
    positive = w > 0
    last_pos = V - 1 - np.argmax(positive[..., ::-1], axis=-1)
    idx = np.where(idx >= V, last_pos, idx)
    safe_total = np.where(total > 0, total, 1.0)
    i_clip = np.clip(idx, 0, V - 1)
    cum_i = np.take_along_axis(cum, i_clip[..., None], axis=-1)[..., 0]
    prev = np.take_along_axis(cum, np.clip(i_clip - 1, 0, V - 1)[..., None], axis=-1)[..., 0]
    prev = np.where(i_clip == 0, 0.0, prev)
    margin = np.minimum(np.abs(prev / safe_total - u), np.abs(cum_i / safe_total - u))
    idx = np.where(total > 0, idx, -1)
    margin = np.where(total > 0, margin, 0.0)
    return idx.astype(np.int64), margin, total


# ---------------------------------------------------------------------------
# Truncated sampling laws (top-k, then top-p)
# ---------------------------------------------------------------------------
#
# The pages' quality runs sample at temperature 1 with top-k 50 and top-p 0.95
# ("Introspective Diffusion Language Models | Summary", section 4.1), and the
# verification must use the law of the proposal mechanism actually used
# (section 3.3): with truncation both P and Q are the truncated laws.
#
# Reading (listed in the design doc): entries are ranked by logit, larger first,
# ties to the lower vocabulary index; top-k keeps the first k of that ranking
# (exactly k, ties included in rank order); top-p then keeps an entry of the
# ranking iff the probability mass, within the top-k renormalised law, of the
# entries ranked before it is below p; the survivors are renormalised.  k = 0
# disables top-k and p >= 1 disables top-p.  The top-p cut is a floating-point
# decision: a row whose cumulative mass lies within TRUNC_WINDOW of p at some
# rank is flagged.

TRUNC_WINDOW = 1e-9


def truncated_probs(logits: np.ndarray, temperature: float = 1.0, top_k: int = 0,
                    top_p: float = 1.0):
    """The truncated law of each row, float64 [..., V], and the top-p margin
    [...] (smallest |mass before rank t - p| over the top-k ranks; inf when
    top-p is off)."""
    a = np.asarray(logits, dtype=np.float64) / float(temperature)
    if np.isnan(a).any() or np.isposinf(a).any():
        raise ValueError("logits contain NaN or +inf")
    if top_k < 0 or not top_p > 0:
        raise ValueError("top_k must be >= 0 and top_p > 0")
    V = a.shape[-1]
    rows = a.reshape(-1, V)
    out = np.zeros_like(rows)
    margin = np.full(rows.shape[0], np.inf)
    k = V if top_k == 0 else min(int(top_k), V)
    for n, z in enumerate(rows):
        # stable sort of the negated logits: larger first, ties to the lower index
        rank = np.argsort(-z, kind="stable")[:k]
        zk = z[rank]
        if np.isneginf(zk[0]):
            raise ValueError("a logits row is entirely -inf")
        w = np.exp(zk - zk[0])
        keep = np.ones(k, dtype=bool)
        if top_p < 1.0:
            pi = w / w.sum()
            before = np.concatenate([[0.0], np.cumsum(pi)[:-1]])
            keep = before < top_p
            margin[n] = np.abs(before - top_p).min()
        out[n, rank[keep]] = w[keep] / w[keep].sum()
    return out.reshape(a.shape), margin.reshape(a.shape[:-1])


def sampling_law(logits, temperature=1.0, top_k=0, top_p=1.0):
    """(law [..., V], top-p margin [...]): softmax(logits / T) when no
    truncation is asked for, else ``truncated_probs``."""
    if top_k == 0 and top_p >= 1.0:
        P = softmax(logits, temperature)
        return P, np.full(P.shape[:-1], np.inf)
    return truncated_probs(logits, temperature, top_k, top_p)


# ---------------------------------------------------------------------------
# Gumbel-max draws driven by a counter-based generator
# ---------------------------------------------------------------------------
#
# The correction of the pages' serving kernel is a Gumbel-max draw
# ("Introspective Diffusion Language Models | Summary", section 3.3): the
# token is argmax_i (ln w_i + G_i) with independent standard Gumbel noise G_i,
# which selects i with probability w_i / sum(w).  The noise of vocabulary
# entry i comes from Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
# random numbers: as easy as 1, 2, 3", SC 2011), written here from its
# published definition: ten rounds of two 32x32->64 multiplications by
# 0xD2511F53 and 0xCD9E8D57 with the key bumped by the Weyl constants
# 0x9E3779B9 and 0xBB67AE85 between rounds.
#
# Reading (listed in the design doc): for sequence c with first rejection j the key
# is (bits of the float32 u_resid[c, j], c) and entry i takes 32-bit word i % 4
# of the block with counter (i // 4, j, 0x15D, 0); U = (2 * (word >> 9) + 1) / 2^24
# (exact in float32, strictly inside (0, 1)) and G = -ln(-ln U).

_PHILOX_M = (0xD2511F53, 0xCD9E8D57)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)
_U32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter, key):
    """Philox4x32-10 blocks.  counter: four uint32 arrays (broadcast together),
    key: two uint32 arrays.  Returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(v, dtype=np.uint64) & _U32 for v in counter)
    k0, k1 = (np.asarray(v, dtype=np.uint64) & _U32 for v in key)
    for r in range(10):
        if r:
            k0 = (k0 + np.uint64(_PHILOX_W[0])) & _U32
            k1 = (k1 + np.uint64(_PHILOX_W[1])) & _U32
        p0 = np.uint64(_PHILOX_M[0]) * c0
        p1 = np.uint64(_PHILOX_M[1]) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _U32,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _U32)
    return tuple(v.astype(np.uint32) for v in (c0, c1, c2, c3))


def gumbel_noise(key0: int, key1: int, j: int, V: int) -> np.ndarray:
    """Standard Gumbel noise [V] (float64) of one correction draw."""
    i = np.arange(V, dtype=np.uint64)
    blocks = philox4x32_10((i >> np.uint64(2), np.full(V, j), np.full(V, 0x15D), np.zeros(V)),
                           (np.full(V, key0), np.full(V, key1)))
    words = np.stack(blocks, axis=-1)[np.arange(V), (i & np.uint64(3)).astype(np.int64)]
    u = (2.0 * (words >> np.uint32(9)).astype(np.float64) + 1.0) * 2.0 ** -24
    return -np.log(-np.log(u))


def gumbel_argmax(weights: np.ndarray, g: np.ndarray):
    """argmax over w > 0 of ln w + g (lowest index on ties), and the gap to the
    second best perturbed value (inf when only one weight is positive)."""
    w = np.asarray(weights, dtype=np.float64)
    with np.errstate(divide="ignore"):
        score = np.where(w > 0, np.log(w), -np.inf) + g
    best = int(np.argmax(score))
    rest = np.delete(score, best)
    gap = score[best] - rest.max() if rest.size and np.isfinite(rest.max()) else np.inf
    return best, gap


def accept_ratio(px: np.ndarray, qx: np.ndarray) -> np.ndarray:
    """min(1, px/qx), with the q(x) = 0 convention (1 if px > 0 else 0)."""
    px = np.asarray(px, dtype=np.float64)
    qx = np.asarray(qx, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.minimum(1.0, px / np.where(qx > 0, qx, 1.0))
    return np.where(qx > 0, r, np.where(px > 0, 1.0, 0.0))


# ---------------------------------------------------------------------------
# Sample mode
# ---------------------------------------------------------------------------

def residual_weights(P, Q):
    """Weights of the correction draw ("Introspective Diffusion Language
    Models | Summary", section 3.2): R = max(0, P - Q) over the last axis,
    unnormalised.  Returns (W, fallback): where the residual mass is 0 (P and
    Q equal) W is P instead and fallback is True."""
    P = np.asarray(P, dtype=np.float64)
    R = np.maximum(0.0, P - np.asarray(Q, dtype=np.float64))
    fallback = R.sum(axis=-1) == 0
    return np.where(fallback[..., None], P, R), fallback


def verify_sample(p, q, x, ua, ur, temperature=1.0, relax=0.0, q_onehot=False,
                  sampler="cdf", seq_ids=None, top_k=0, top_p=1.0):
    """ISD verification of proposals ``x`` against the anchor, batched.

    p, q: [B, L, V] logits (anchor rows, proposal rows that generated x);
    x: [B, L] int proposals; ua, ur: [B, L] uniforms in [0, 1).

    Variants ("Introspective Diffusion Language Models | Summary", section 3.3
    and the relaxed-acceptance ablation of section 4):
      relax = tau >= 0 accepts with min(1, (1 + tau) P(x)/Q(x)) (tau = 0 is
        the exact rule); the correction and alpha are unchanged;
      q_onehot: the proposals were argmax picks, so their law is one-hot at
        x (q is not read): the ratio is P(x) and the residual is P with x
        removed;
      sampler = "gumbel" draws the correction by Gumbel-max with the noise of
        ``gumbel_noise`` (seq_ids: the sequences' indices c in the batch, for
        the key; default 0..B-1) instead of by inverse CDF;
      top_k, top_p truncate both laws (``truncated_probs``): P and Q are the
        truncated anchor and proposal laws, and a sequence whose rows have a
        top-p margin under TRUNC_WINDOW is flagged.
    Returns a dict of per-sequence arrays:
      accept_len [B], out_tokens [B, L] (-1 padded), n_emitted [B],
      p_x, q_x, ratio [B, L], alpha [B], decision_margin [B] (smallest
      |ua - r| over k <= j), resid_margin [B] (inf when nothing was drawn),
      resid_fallback [B] (residual mass was 0), flagged [B] and
      resid_flagged [B].
    """
    p = np.asarray(p, dtype=np.float64)
    x = np.asarray(x, dtype=np.int64)
    ua = np.asarray(ua, dtype=np.float64)
    ur = np.asarray(ur, dtype=np.float64)
    B, L, V = p.shape
    if relax < 0:
        raise ValueError("relax must be >= 0")

    P, trunc_margin = sampling_law(p, temperature, top_k, top_p)
    trunc_margin = trunc_margin.min(axis=-1)
    if q_onehot:
        Q = np.zeros_like(P)
        np.put_along_axis(Q, x[..., None], 1.0, axis=-1)
    else:
        Q, mq = sampling_law(np.asarray(q, dtype=np.float64), temperature, top_k, top_p)
        trunc_margin = np.minimum(trunc_margin, mq.min(axis=-1))
    px = np.take_along_axis(P, x[..., None], axis=-1)[..., 0]
    qx = np.take_along_axis(Q, x[..., None], axis=-1)[..., 0]
    r = accept_ratio(px, qx)
    alpha = r.mean(axis=-1)
    r_acc = accept_ratio((1.0 + relax) * px, qx) if relax else r

    accepted = ua < r_acc
    rejected = ~accepted
    j = np.where(rejected.any(axis=-1), np.argmax(rejected, axis=-1), L)

    ks = np.arange(L)[None, :]
    considered = ks <= j[:, None]
    gap = np.where(considered, np.abs(ua - r_acc), np.inf)
    decision_margin = gap.min(axis=-1)

    out = np.where(ks < j[:, None], x, -1)
    n_emitted = j + (j < L)
    resid_margin = np.full(B, np.inf)
    resid_fallback = np.zeros(B, dtype=bool)

    rows = np.nonzero(j < L)[0]
    if rows.size:
        jj = j[rows]
        W, fallback = residual_weights(P[rows, jj], Q[rows, jj])
        resid_fallback[rows] = fallback
        if sampler == "gumbel":
            ids = np.arange(B) if seq_ids is None else np.asarray(seq_ids)
            bits = np.asarray(ur, dtype=np.float32).view(np.uint32)
            tok = np.empty(rows.size, dtype=np.int64)
            margin = np.empty(rows.size)
            for n, (b, jb) in enumerate(zip(rows, jj)):
                g = gumbel_noise(int(bits[b, jb]), int(ids[b]), int(jb), V)
                tok[n], gap = gumbel_argmax(W[n], g)
                # a gap under GUMBEL_WINDOW counts as a near tie
                margin[n] = TIE_WINDOW * gap / GUMBEL_WINDOW
        elif sampler == "cdf":
            tok, margin, _ = inverse_cdf(W, ur[rows, jj])
        else:
            raise ValueError(f"unknown sampler {sampler!r}")
        out[rows, jj] = tok
        resid_margin[rows] = np.where(fallback, 0.0, margin)

    flagged = (decision_margin < TIE_WINDOW) | (trunc_margin < TRUNC_WINDOW)
    resid_flagged = (resid_margin < TIE_WINDOW) | resid_fallback
    return dict(accept_len=j, out_tokens=out, n_emitted=n_emitted, p_x=px, q_x=qx,
                ratio=r, alpha=alpha, decision_margin=decision_margin,
                resid_margin=resid_margin, resid_fallback=resid_fallback,
                flagged=flagged, resid_flagged=resid_flagged)


def propose_sample(qn, up, temperature=1.0, top_k=0, top_p=1.0):
    """Draw the next proposals from the mask-position logits, batched.

    qn: [..., V] logits; up: [...] uniforms.  Returns ``(tokens, prob,
    margin, flagged)`` where prob is the sampling law (softmax(qn/T), or its
    top-k / top-p truncation) at the drawn token.
    """
    Qn, trunc_margin = sampling_law(qn, temperature, top_k, top_p)
    tok, margin, _ = inverse_cdf(Qn, up)
    prob = np.take_along_axis(Qn, tok[..., None], axis=-1)[..., 0]
    return tok, prob, margin, (margin < TIE_WINDOW) | (trunc_margin < TRUNC_WINDOW)


def alpha_sample(p, q, x, temperature=1.0):
    """Introspective acceptance rate per sequence, [B, L, V] -> [B]."""
    P = softmax(p, temperature)
    Q = softmax(q, temperature)
    x = np.asarray(x, dtype=np.int64)
    px = np.take_along_axis(P, x[..., None], axis=-1)[..., 0]
    qx = np.take_along_axis(Q, x[..., None], axis=-1)[..., 0]
    return accept_ratio(px, qx).mean(axis=-1)


# ---------------------------------------------------------------------------
# Greedy (strict, argmax-proposal) mode
# ---------------------------------------------------------------------------

def argmax_first(logits):
    """Index of the largest logit along the last axis, lowest index on ties."""
    return np.argmax(np.asarray(logits, dtype=np.float64), axis=-1).astype(np.int64)


def verify_greedy(p, x):
    """Strict verification: accept x_k iff it equals argmax p_k.

    p: [B, L, V] logits; x: [B, L].  The correction at the first mismatch is
    the anchor argmax there.  Returns the same keys as ``verify_sample`` for
    tokens and counts, with ``alpha`` the match fraction.
    """
    x = np.asarray(x, dtype=np.int64)
    B, L, _ = np.shape(p)
    g = argmax_first(p)
    match = x == g
    mismatch = ~match
    j = np.where(mismatch.any(axis=-1), np.argmax(mismatch, axis=-1), L)
    ks = np.arange(L)[None, :]
    out = np.where(ks < j[:, None], x, -1)
    rows = np.nonzero(j < L)[0]
    out[rows, j[rows]] = g[rows, j[rows]]
    return dict(accept_len=j, out_tokens=out, n_emitted=j + (j < L),
                argmax=g, alpha=match.mean(axis=-1))


def propose_greedy(qn):
    """Next proposals by argmax of the mask-position logits."""
    return argmax_first(qn)


# ---------------------------------------------------------------------------
# LM head (logits GEMM feeding the step)
# ---------------------------------------------------------------------------

def lm_head(h, w):
    """logits = h @ w in float64 on exactly decoded inputs."""
    return np.asarray(h, dtype=np.float64) @ np.asarray(w, dtype=np.float64)


# ---------------------------------------------------------------------------
# Segment-gated LoRA projection
# ---------------------------------------------------------------------------

def lora_gemm(x, w, a, b, mask):
    """h_j = W x_j + [j is a mask position] * B A x_j ("Introspective Diffusion
    Language Models | Summary", appendix G; section 3.2: the adapter acts only
    at mask positions, clean and introspection positions keep the base
    weights), in float64 on exactly decoded inputs.

    x [M, K]; w [N, K]; a [r, K]; b [N, r] (output features first); mask [M]
    (nonzero = mask position).  Returns h [M, N].
    """
    x = np.asarray(x, dtype=np.float64)
    base = x @ np.asarray(w, dtype=np.float64).T
    t = x @ np.asarray(a, dtype=np.float64).T
    gate = (np.asarray(mask) != 0).astype(np.float64)[:, None]
    return base + gate * (t @ np.asarray(b, dtype=np.float64).T)
