"""The pages' streaming algorithms, float64 reference models.  TEST INFRASTRUCTURE.

These are not used to check the GPU; they check the pages' own claims
(exactness, associativity, the invariants) against the direct definitions
in ``attention`` and ``softmax``.  They model the recurrences the pages
derive, in the pages' notation: ``single_query_blockwise`` the single-query
recurrence of page "Derive online softmax, prove it is exact", section "A
strong answer" (written here as a fold of per-block (m, l, a) states under
the merge rule), and ``blockwise_attention`` the query-tile recurrence of
page "Online softmax for a whole query tile, matrix form", section "A
strong answer", whose update equations (running maximum, guarded
reference, rescale factor, P, l, A) are that page's and so appear here as
the same few lines.

``blockwise_attention`` accepts a ``mutation`` name that plants one of the
mistakes the pages list, so that the tests can show their pins catch it.
"""
from __future__ import annotations

import math

import numpy as np

NEG_INF = -np.inf

# ---------------------------------------------------------------------------
# Online normalizer (m, d) -- article "Online softmax", Steps 2-4
# ---------------------------------------------------------------------------


def online_normalizer_step(m: float, d: float, x: float) -> tuple[float, float]:
    """One element of article "Online softmax", Step 2.

    The new maximum is max(m, x); the old sum is scaled by exp(m - m_new)
    (referencing it to the new maximum) and exp(x - m_new) is added.  The
    start state is (-inf, 0); exp(-inf - m_new) is 0 for the first element.
    """
    m_new = max(m, x)
    return m_new, d * math.exp(m - m_new) + math.exp(x - m_new)


def online_normalizer(x) -> tuple[float, float, list[tuple[float, float]]]:
    """Run Step 2 over the vector; return (m, d, trace of (m, d) after each element)."""
    m, d = NEG_INF, 0.0
    trace = []
    for xi in np.asarray(x, dtype=np.float64).ravel():
        m, d = online_normalizer_step(m, d, float(xi))
        trace.append((m, d))
    return m, d, trace


def merge_md(a: tuple[float, float], b: tuple[float, float]) -> tuple[float, float]:
    """Article "Online softmax", Step 4: merge two (m, d) pairs.

    Take the larger maximum and rescale each block's sum to it before adding.
    An empty block (-inf, 0) contributes nothing.
    """
    (m1, d1), (m2, d2) = a, b
    M = max(m1, m2)
    if M == NEG_INF:
        return NEG_INF, 0.0
    w1 = 0.0 if m1 == NEG_INF else math.exp(m1 - M)
    w2 = 0.0 if m2 == NEG_INF else math.exp(m2 - M)
    return M, d1 * w1 + d2 * w2


def online_softmax(x) -> np.ndarray:
    """Article "Online softmax", Step 3: pass 1 gives (m, d); pass 2 writes exp(x - m) / d."""
    x = np.asarray(x, dtype=np.float64).ravel()
    m, d, _ = online_normalizer(x)
    return np.array([math.exp(float(xi) - m) / d for xi in x])


def two_pass_unshifted_softmax(x) -> np.ndarray:
    """Article "Online softmax", Step 1, naive form: no maximum subtracted.

    Kept only to show the failure the maximum prevents (overflow to inf and
    then NaN at large scores).
    """
    x = np.asarray(x, dtype=np.float64).ravel()
    with np.errstate(over="ignore", invalid="ignore"):
        e = np.exp(x)
        return e / e.sum()


# ---------------------------------------------------------------------------
# Single-query blockwise recurrence -- page "Derive online softmax, prove it
# is exact", section "A strong answer"
# ---------------------------------------------------------------------------


def merge_state(x, y):
    """Merge two single-query states (m, l, a) by the rescale rule (article "Online softmax", Step 4).

    Both are referenced to the larger maximum; an empty state (-inf, 0, 0)
    contributes nothing.
    """
    (m1, l1, a1), (m2, l2, a2) = x, y
    M = max(m1, m2)
    if M == NEG_INF:
        return NEG_INF, 0.0, a1 + a2
    w1 = 0.0 if m1 == NEG_INF else math.exp(m1 - M)
    w2 = 0.0 if m2 == NEG_INF else math.exp(m2 - M)
    return M, w1 * l1 + w2 * l2, w1 * a1 + w2 * a2


def single_query_blockwise(q, K, V, block: int = 128, scale: float | None = None) -> np.ndarray:
    """The single-query recurrence over key blocks; returns a / l.

    The running state (m, l, a) starts empty; each block contributes its own
    state (its maximum, the sum of exp(s - max) and the matching weighted
    sum of V rows), merged into the running one.  Merging is exactly the
    update of the page: m' = max(m, block max), l and a rescaled by
    exp(m - m'), the block's terms exp(s_i - m') added.
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    sigma = 1.0 / math.sqrt(q.shape[0]) if scale is None else float(scale)
    state = (NEG_INF, 0.0, np.zeros(V.shape[1]))
    for j0 in range(0, K.shape[0], block):
        s = sigma * (K[j0:j0 + block] @ q)
        mb = float(s.max())
        w = np.exp(s - mb)
        state = merge_state(state, (mb, float(w.sum()), w @ V[j0:j0 + block]))
    _, l, a = state
    return a / l


# ---------------------------------------------------------------------------
# Query-tile matrix form -- page "Online softmax for a whole query tile,
# matrix form", section "A strong answer" (with the guard and FA2's deferred
# division)
# ---------------------------------------------------------------------------

MUTATIONS = (
    None,
    "m_init_zero",          # page 1, "Common mistakes": m starts at 0, not -inf
    "no_acc_rescale",       # page 1, "Common mistakes": l rescaled, A not
    "fa1_wrong_ratio",      # page 2, "Common mistakes": normalized O, wrong rescale ratio
    "tile_scalar_max",      # page 2, "Common mistakes": one max for the whole tile
    "no_guard",             # page 2, the guard on m_ref left out
    "drop_partial_block",   # page 2, "Common mistakes": only whole blocks handled
)


def blockwise_attention(Q, K, V, scale: float, *, q0: int = 0, N: int | None = None,
                        Bc: int = 64, causal: bool = False, window: int = 0,
                        kv_len: int | None = None, mutation: str | None = None):
    """One query tile Q [Br, d] (rows q0 .. q0+Br-1) against K, V [N, d].

    State per row: m (running max), l (running normalizer), A (unnormalized
    accumulator).  For each key block K_j, V_j:
        S_j = sigma Q K_j^T (masked entries -inf)
        m'  = max(m, rowmax S_j)
        m_ref = 0 where m' = -inf, else m'       (guard: rows with nothing yet)
        alpha = exp(m - m_ref);  P_j = exp(S_j - m_ref)
        l' = alpha * l + rowsum P_j;  A' = diag(alpha) A + P_j V_j
    After the last block O = diag(l)^-1 A (divided once); rows with l = 0
    give O = 0 and LSE = -inf.  LSE = m + log l.  Returns (O, LSE).
    """
    if mutation not in MUTATIONS:
        raise ValueError(mutation)
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Br, d = Q.shape
    N = K.shape[0] if N is None else N
    klen = N if kv_len is None else kv_len
    sigma = float(scale)
    rows = q0 + np.arange(Br)
    m = np.full(Br, 0.0 if mutation == "m_init_zero" else NEG_INF)
    l = np.zeros(Br)
    A = np.zeros((Br, V.shape[1]))
    stop = N - (N % Bc) if mutation == "drop_partial_block" else N
    for j0 in range(0, stop, Bc):
        cols = np.arange(j0, min(j0 + Bc, N))
        S = sigma * (Q @ K[cols].T)
        vis = (cols[None, :] < klen) & np.ones((Br, 1), bool)
        if causal:
            vis &= cols[None, :] <= rows[:, None]
        if window > 0:
            vis &= np.abs(rows[:, None] - cols[None, :]) < window
        S = np.where(vis, S, NEG_INF)
        if mutation == "tile_scalar_max":
            m_new = np.full(Br, max(float(m.max()), float(S.max())))
        else:
            m_new = np.maximum(m, S.max(axis=1))
        if mutation == "no_guard":
            m_ref = m_new
        else:
            m_ref = np.where(np.isneginf(m_new), 0.0, m_new)
        with np.errstate(invalid="ignore", over="ignore"):
            alpha = np.exp(m - m_ref)
            P = np.exp(S - m_ref[:, None])
            l_new = alpha * l + P.sum(axis=1)
            if mutation == "fa1_wrong_ratio":
                # Keeps A normalized but rescales it by alpha alone, not by alpha * l / l'.
                A = (alpha[:, None] * A + P @ V[cols]) / l_new[:, None]
            elif mutation == "no_acc_rescale":
                A = A + P @ V[cols]
            else:
                A = alpha[:, None] * A + P @ V[cols]
        l = l_new
        m = m_new
    with np.errstate(invalid="ignore", divide="ignore"):
        if mutation == "fa1_wrong_ratio":
            O = A
        elif mutation == "no_guard":
            O = A / l[:, None]
        else:
            O = np.where(l[:, None] > 0, A / np.where(l > 0, l, 1.0)[:, None], 0.0)
        if mutation == "no_guard":
            lse = m + np.log(l)
        else:
            lse = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), NEG_INF)
    return O, lse


def blockwise_attention_full(Q, K, V, scale: float, *, Br: int = 128, Bc: int = 64,
                             causal: bool = False, window: int = 0, kv_len: int | None = None,
                             mutation: str | None = None):
    """Tile the queries of one (b, h) slice into blocks of Br and run each tile."""
    Q = np.asarray(Q, np.float64)
    N = Q.shape[0]
    O = np.zeros((N, np.asarray(V).shape[1]))
    L = np.zeros(N)
    for q0 in range(0, N, Br):
        o, lse = blockwise_attention(Q[q0:q0 + Br], K, V, scale, q0=q0, N=N, Bc=Bc, causal=causal,
                                     window=window, kv_len=kv_len, mutation=mutation)
        O[q0:q0 + Br] = o
        L[q0:q0 + Br] = lse
    return O, L


# ---------------------------------------------------------------------------
# Split-KV -- page "Derive online softmax, prove it is exact", section "What
# interviewers probe next" (batch-1 decoding); article "Online softmax",
# "Trade-offs and edge cases" (Flash-Decoding: per-chunk result plus a
# rescaling reduction)
# ---------------------------------------------------------------------------


def split_kv_partials(q, K, V, nsplit: int, scale: float | None = None):
    """Per chunk c = [c L, min((c+1) L, Nkv)), L = ceil(Nkv / nsplit): (m_c, l_c, a_c).

    An empty chunk has (-inf, 0, 0).
    """
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    Nkv, d = K.shape
    sigma = float(np.float32(1.0 / math.sqrt(d))) if scale is None else float(scale)
    L = -(-Nkv // nsplit)
    parts = []
    for c in range(nsplit):
        lo, hi = c * L, min((c + 1) * L, Nkv)
        if lo >= hi:
            parts.append((NEG_INF, 0.0, np.zeros(V.shape[1])))
            continue
        s = sigma * (K[lo:hi] @ q)
        m = float(s.max())
        e = np.exp(s - m)
        parts.append((m, float(e.sum()), e @ V[lo:hi]))
    return parts


def split_kv_merge(parts):
    """Merge (m_c, l_c, a_c): M = max m_c, w_c = exp(m_c - M) (0 for empty), o = sum w a / sum w l."""
    M = max(p[0] for p in parts)
    l = 0.0
    a = np.zeros_like(parts[0][2])
    for m_c, l_c, a_c in parts:
        w = 0.0 if m_c == NEG_INF else math.exp(m_c - M)
        l += w * l_c
        a = a + w * a_c
    return a / l, M + math.log(l)
