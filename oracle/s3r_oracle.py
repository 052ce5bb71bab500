"""Plain, slow, fp64 CPU oracle of the S3R hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by ``__graft_entry__.smoke()`` and
by the ``cpu_baseline`` leg of bench.py, never by the library or its binding.
It shares no code with the HIP path.

What is computed, and where it comes from
-----------------------------------------
"S3R: Fast and Faithful RL Rollouts via Self-Sparse Speculative Decoding",
Abstract: the policy drafts while attending to part of its KV cache, a dense
attention pass over the whole cached history checks the draft, and speculative
sampling keeps the output distributed as the dense policy's; drafter and
verifier are one model, so one KV cache serves both. The pages give no
equations, so every step below is the plain definition of the operation,
written out:

* page bounds / page select: the pages leave the sparse rule open; this library
  fixes a query-aware rule after the Quest title the page-3 reference list
  cites ("Quest: Query-Aware Sparsity ..."): per page elementwise key min/max,
  an upper bound on each query head's logit, top-k pages under a token budget.
* attention: softmax(scale * q K^T) V over a token set (textbook definition),
  paged as in the PagedAttention title of the same list.
* spec sample: the accept/residual rule of the two speculative-sampling titles
  the page-3 list cites ("Fast Inference from Transformers via Speculative
  Decoding"; "Accelerating Large Language Model Decoding with Speculative
  Sampling"): accept x with prob min(1, p(x)/q(x)), otherwise draw from
  norm(max(0, p - q)); a bonus draw from the last target row if all accept.
* RNG: Philox4x64-10 from Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:
  As Easy as 1, 2, 3" (SC'11), written from that definition.

Pins (tests/test_oracle_*.py): brute-force bounds and sort, torch SDPA on CPU,
a second streaming-softmax decode path, exact rational enumeration of the
sampler at vocab 8, chi-square Monte Carlo, q = p => full acceptance, the
accepted-length law prod(alpha_i), numpy.random.Philox known answers, and for
the acceptance rate its closed forms (q = p, disjoint supports, two tokens),
the total-variation identity and the enumerated accept probability.
Parity of the page-level figures (attention share, end-to-end speedup) is
unpinned: they need the model and workloads the pages measured.

Data layout (a format both sides must agree on):
  k_pool[N_phys][Hkv][P][D]   key of token t in page slot t % P
  v_pool[N_phys][Hkv][D][P]   value, transposed inside each page
  page_table[B][max_pages]    logical page -> physical page
  seq_lens[B]                 KV positions visible to the last query
  bounds[N_phys][Hkv][2][D]   [0] = elementwise min, [1] = elementwise max
Every physical page belongs to one sequence. Inputs are numpy arrays; bf16 data
is passed as its exact float64 upcast.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "PHILOX_M0", "PHILOX_M1", "PHILOX_W0", "PHILOX_W1",
    "philox4x64_10", "uniform",
    "key_row", "value_row", "n_pages",
    "page_bounds", "page_scores", "page_select", "round_forced_pages", "page_select_round",
    "kv_commit",
    "attend", "sparse_draft_attn", "dense_verify_attn", "decode_streaming",
    "softmax", "icdf", "spec_sample", "draw_draft_tokens", "draw_tokens", "acceptance_rate",
]

# ---------------------------------------------------------------------------
# Philox4x64-10 (Salmon et al., SC'11): 4x64-bit counter, 2x64-bit key, ten
# rounds of two 64x64->128 multiplies, key bumped by the two Weyl constants
# between rounds.
# ---------------------------------------------------------------------------
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15  # golden ratio
PHILOX_W1 = 0xBB67AE8584CAA73B  # sqrt(3) - 1
_MASK64 = (1 << 64) - 1


def philox4x64_10(counter, key):
    """Return the four 64-bit output words for one (counter, key) block."""
    x0, x1, x2, x3 = (int(c) & _MASK64 for c in counter)
    k0, k1 = (int(k) & _MASK64 for k in key)
    for _ in range(10):
        prod0 = PHILOX_M0 * x0
        prod1 = PHILOX_M1 * x2
        hi0, lo0 = prod0 >> 64, prod0 & _MASK64
        hi1, lo1 = prod1 >> 64, prod1 & _MASK64
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
        k0 = (k0 + PHILOX_W0) & _MASK64
        k1 = (k1 + PHILOX_W1) & _MASK64
    return x0, x1, x2, x3


def uniform(seed, offset, b, slot, stream):
    """U(b, slot, stream) in [0, 1): the top 53 bits of word 0, times 2^-53.

    key = (seed, 0), counter = (offset, b, slot, stream). Stream 0 holds the
    accept uniforms, stream 1 the residual/bonus draws, stream 2 the draft-token
    draws a drafter makes upstream of the sampler.
    """
    w0 = philox4x64_10((offset, b, slot, stream), (seed, 0))[0]
    return (w0 >> 11) * (2.0 ** -53)


# ---------------------------------------------------------------------------
# Paged KV access
# ---------------------------------------------------------------------------
def n_pages(seq_len, P):
    return -(-int(seq_len) // P)


def key_row(k_pool, page_table, b, h, t):
    P = k_pool.shape[2]
    return k_pool[page_table[b, t // P], h, t % P, :]


def value_row(v_pool, page_table, b, h, t):
    P = v_pool.shape[3]
    return v_pool[page_table[b, t // P], h, :, t % P]


# ---------------------------------------------------------------------------
# Page bounds and query-aware page selection
# ---------------------------------------------------------------------------
def page_bounds(k_pool, page_table, seq_lens, seqs=None):
    """bounds[phys][h][0|1][d] = min|max over the page's valid tokens of K[t][h][d].

    Valid tokens of logical page j of sequence b: j*P <= t < min((j+1)*P, seq_len).
    Physical pages not reached by any (b, j) are left as NaN; a negative table
    entry marks an unallocated page and is skipped.
    """
    n_phys, hkv, P, D = k_pool.shape
    out = np.full((n_phys, hkv, 2, D), np.nan)
    B = page_table.shape[0]
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        for j in range(n_pages(L, P)):
            phys = page_table[b, j]
            if phys < 0:
                continue
            for h in range(hkv):
                rows = np.stack([key_row(k_pool, page_table, b, h, t)
                                 for t in range(j * P, min((j + 1) * P, L))])
                out[phys, h, 0] = rows.min(axis=0)
                out[phys, h, 1] = rows.max(axis=0)
    return out


def kv_commit(k_pool, v_pool, page_table, k_new, v_new, first_pos, seq_lens, bounds):
    """Write new K/V rows into their pages, then bring the touched pages' bounds
    up to date for the committed lengths.

    The step either side of a round: the rows a forward pass produced are
    appended to the shared cache, and after the accept/reject decision the
    sequence's length is set back to what was committed. Row i of sequence b
    (k_new[b, i], v_new[b, i]: [Hkv][D]) goes to position first_pos[b] + i:
    logical page pos // P, slot pos % P, V transposed inside the page; rows
    past the page table, or in a page whose table entry is negative (not
    allocated), are dropped. seq_lens[b] is the committed length after
    the call; it may end inside the rows just written (a rollback: those rows
    stay in the pool but no longer count). Every logical page from
    min(first_pos[b], seq_lens[b] - 1) // P through the last page written or
    the tail page of seq_lens[b] gets its bounds recomputed over its tokens
    below seq_lens[b] (page_bounds' rule); a page left without valid tokens
    keeps its old bounds. Other pages are untouched.

    Returns new (k_pool, v_pool, bounds) arrays.
    """
    K, V, Bd = k_pool.copy(), v_pool.copy(), bounds.copy()
    n_phys, hkv, P, D = K.shape
    B, max_pages = page_table.shape
    count = k_new.shape[1]
    for b in range(B):
        f = int(first_pos[b])
        for i in range(count):
            pos = f + i
            if pos // P >= max_pages or page_table[b, pos // P] < 0:
                continue
            phys = page_table[b, pos // P]
            K[phys, :, pos % P, :] = k_new[b, i]
            V[phys, :, :, pos % P] = v_new[b, i]
    fresh = page_bounds(K, page_table, seq_lens)
    for b in range(B):
        f, L = int(first_pos[b]), int(seq_lens[b])
        lo = min(f, max(L - 1, 0)) // P
        hi = max((f + count - 1) // P if count > 0 else -1, n_pages(L, P) - 1)
        for j in range(lo, min(hi, max_pages - 1) + 1):
            if j < n_pages(L, P) and page_table[b, j] >= 0:
                Bd[page_table[b, j]] = fresh[page_table[b, j]]
    return K, V, Bd


def page_scores(bounds, q, page_table, seq_lens, scale, b, h, P=16):
    """Scores of every logical page of (sequence b, kv head h).

    score_j = max over the q heads g of the group of
              scale * sum_d max(q[g,d] * kmin[j,d], q[g,d] * kmax[j,d]),
    an upper bound on scale * q_g . k_t for every token t of page j. One
    selection per kv head lets the whole query group share the pages it reads.
    q: [B][Hq][D].
    """
    hkv = bounds.shape[1]
    G = q.shape[1] // hkv
    n = n_pages(int(seq_lens[b]), P)
    scores = np.empty(n)
    for j in range(n):
        kmin = bounds[page_table[b, j], h, 0]
        kmax = bounds[page_table[b, j], h, 1]
        best = -math.inf
        for g in range(h * G, (h + 1) * G):
            s = scale * float(np.sum(np.maximum(q[b, g] * kmin, q[b, g] * kmax)))
            best = max(best, s)
        scores[j] = best
    return scores


def page_select(bounds, q, page_table, seq_lens, budget_tokens, scale, P=16, seqs=None):
    """Top-k pages per (sequence, kv head) under a token budget.

    k = budget_tokens // P (a partial tail page costs a full page). With n pages
    in the sequence: if k >= n every page is taken; otherwise pages are ranked by
    (score descending, logical index ascending) and the first k kept. The kept
    indices are emitted in ascending order and padded with -1 to length k.

    Returns (selected[B][Hkv][k] int32, num_selected[B] int32, scores) where
    scores[(b, h)] holds every page score (None when k >= n).
    """
    B = page_table.shape[0]
    hkv = bounds.shape[1]
    k = budget_tokens // P
    selected = np.full((B, hkv, k), -1, dtype=np.int32)
    num_selected = np.zeros(B, dtype=np.int32)
    scores = {}
    for b in (range(B) if seqs is None else seqs):
        n = n_pages(int(seq_lens[b]), P)
        num_selected[b] = min(k, n)
        for h in range(hkv):
            if k >= n:
                selected[b, h, :n] = np.arange(n)
                scores[(b, h)] = None
                continue
            sc = page_scores(bounds, q, page_table, seq_lens, scale, b, h, P)
            order = sorted(range(n), key=lambda j: (-sc[j], j))
            selected[b, h, :] = sorted(order[:k])
            scores[(b, h)] = sc
    return selected, num_selected, scores


def round_forced_pages(seq_len, gamma, P, max_pages):
    """Logical pages holding the positions of one round's gamma draft queries.

    Draft step j of a round queries position seq_len - 1 + j (seq_len is the
    length at step 0), so the round's queries sit at positions
    max(seq_len - 1, 0) .. seq_len + gamma - 2; their pages, below max_pages,
    ascending. With gamma <= P that is one or two pages.
    """
    lo, hi = max(seq_len - 1, 0), seq_len + gamma - 2
    return sorted({p // P for p in range(lo, hi + 1) if p // P < max_pages})


def page_select_round(bounds, q, page_table, seq_lens, budget_tokens, gamma, scale, P=16,
                      seqs=None):
    """Once-per-round selection: the round's forced tail pages plus the best rest.

    Selection-frequency variant of page_select (a reading of the pages: they do
    not say how often drafting re-selects). Made once at draft step 0 and
    reused by the round's later steps, it must keep the pages the later queries
    sit in, which may not exist yet at step 0: every page of
    round_forced_pages(seq_len, gamma, ...) is kept, and the remaining
    k - |forced| slots go to the other existing pages ranked as in page_select
    (score descending, index ascending), or to all of them if they fit. Output
    ascending, -1 padded; num_selected[b] counts the kept pages. Requires
    k >= |forced|.

    Returns (selected[B][Hkv][k], num_selected[B], scores) with scores[(b, h)]
    the candidate pages' scores (None when every candidate is kept).
    """
    B, max_pages = page_table.shape
    hkv = bounds.shape[1]
    k = budget_tokens // P
    selected = np.full((B, hkv, k), -1, dtype=np.int32)
    num_selected = np.zeros(B, dtype=np.int32)
    scores = {}
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        n = n_pages(L, P)
        forced = round_forced_pages(L, gamma, P, max_pages)
        if k < len(forced):
            raise ValueError("budget smaller than the round's forced pages")
        candidates = [j for j in range(n) if j not in forced]
        rest = k - len(forced)
        for h in range(hkv):
            if rest >= len(candidates):
                chosen = candidates
                scores[(b, h)] = None
            else:
                sc = page_scores(bounds, q, page_table, seq_lens, scale, b, h, P)
                chosen = sorted(candidates, key=lambda j: (-sc[j], j))[:rest]
                scores[(b, h)] = {j: sc[j] for j in candidates}
            kept = sorted(set(forced) | set(chosen))
            selected[b, h, :len(kept)] = kept
            num_selected[b] = len(kept)
    return selected, num_selected, scores


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------
def attend(qv, Kt, Vt, scale):
    """softmax(scale * Kt @ qv) @ Vt, the textbook definition, in fp64.

    An empty token set (a sequence or causal row that sees no position) has no
    softmax; the library defines its output as zeros, and so does the oracle.
    """
    if len(Kt) == 0:
        return np.zeros(Vt.shape[1] if np.ndim(Vt) == 2 else 0)
    logits = scale * (Kt @ qv)
    m = logits.max()
    w = np.exp(logits - m)
    return (w / w.sum()) @ Vt


def _gather(k_pool, v_pool, page_table, b, h, positions):
    positions = list(positions)
    D = k_pool.shape[3]
    if not positions:
        return np.zeros((0, D)), np.zeros((0, D))
    Kt = np.stack([key_row(k_pool, page_table, b, h, t) for t in positions])
    Vt = np.stack([value_row(v_pool, page_table, b, h, t) for t in positions])
    return Kt, Vt


def sparse_draft_attn(q, k_pool, v_pool, page_table, seq_lens, selected, scale,
                      seqs=None, heads=None):
    """Single-query GQA decode over the selected pages only.

    q: [B][Hq][D]; selected: [B][Hkv][k] logical page ids (-1 = unused). Query
    head g reads kv head g // G over T = {t < seq_len : t // P in sel(b, h)}.
    Returns out[B][Hq][D] (NaN where not computed).
    """
    B, Hq, D = q.shape
    hkv = k_pool.shape[1]
    P = k_pool.shape[2]
    G = Hq // hkv
    out = np.full((B, Hq, D), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        for g in (range(Hq) if heads is None else heads):
            h = g // G
            pages = sorted({int(j) for j in selected[b, h] if j >= 0})
            positions = [t for j in pages for t in range(j * P, min((j + 1) * P, L))]
            Kt, Vt = _gather(k_pool, v_pool, page_table, b, h, positions)
            out[b, g] = attend(q[b, g], Kt, Vt, scale)
    return out


def dense_verify_attn(q, k_pool, v_pool, page_table, seq_lens, scale,
                      seqs=None, heads=None):
    """Causal attention of nq query positions over the complete paged KV.

    q: [B][nq][Hq][D]. Query i sits at position seq_len - nq + i and sees every
    position <= its own. Returns out[B][nq][Hq][D] (NaN where not computed).
    """
    B, nq, Hq, D = q.shape
    hkv = k_pool.shape[1]
    G = Hq // hkv
    out = np.full((B, nq, Hq, D), np.nan)
    for b in (range(B) if seqs is None else seqs):
        L = int(seq_lens[b])
        for g in (range(Hq) if heads is None else heads):
            h = g // G
            Kt, Vt = _gather(k_pool, v_pool, page_table, b, h, range(max(L, 0)))
            for i in range(nq):
                visible = max(0, L - nq + i + 1)
                out[b, i, g] = attend(q[b, i, g], Kt[:visible], Vt[:visible], scale)
    return out


def decode_streaming(qv, k_pool, v_pool, page_table, b, h, n_visible, scale):
    """A second, independent decode path: one token at a time, running max/sum.

    o_n = (sum_{t<n} e^{s_t - m_n} v_t) / (sum_{t<n} e^{s_t - m_n}), updated per
    token; used to pin the batched verify against sequential single decodes.
    """
    m = -math.inf
    den = 0.0
    num = np.zeros(k_pool.shape[3])
    for t in range(n_visible):
        s = scale * float(np.dot(key_row(k_pool, page_table, b, h, t), qv))
        m_new = max(m, s)
        c = math.exp(m - m_new) if m != -math.inf else 0.0
        e = math.exp(s - m_new)
        num = num * c + e * value_row(v_pool, page_table, b, h, t)
        den = den * c + e
        m = m_new
    return num / den if n_visible > 0 else num


# ---------------------------------------------------------------------------
# Exact speculative sampling
# ---------------------------------------------------------------------------
def softmax(logits, temperature):
    z = np.asarray(logits, dtype=np.float64) / temperature
    e = np.exp(z - z.max())
    return e / e.sum()


def icdf(w, u):
    """Smallest t with sum_{s<=t} w_s > u * sum(w), ascending token order.

    Returns (t, margin): margin is the distance of u*sum(w) from the nearer
    boundary of the chosen bin, over sum(w). If rounding leaves no such t the
    last t with w_t > 0 is returned with margin 0.
    """
    w = np.asarray(w, dtype=np.float64)
    total = float(w.sum())
    target = u * total
    c = np.cumsum(w)
    hits = np.nonzero(c > target)[0]
    if hits.size == 0:
        return int(np.nonzero(w > 0)[0][-1]), 0.0
    t = int(hits[0])
    lo = float(c[t - 1]) if t > 0 else 0.0
    return t, min(target - lo, float(c[t]) - target) / total


def spec_sample(draft_logits, target_logits, draft_tokens, temperature, seed, offset,
                uniform_fn=None):
    """One round of exact speculative sampling per sequence.

    draft_logits [B][gamma][V], target_logits [B][gamma+1][V], draft_tokens
    [B][gamma]. p_i = softmax(target_i / T), q_i = softmax(draft_i / T).
    For i = 0..gamma-1 with x = draft_tokens[b][i], u = U(b, i, 0):
      accept iff (q_i(x) > 0 and u < p_i(x) / q_i(x)) or (q_i(x) = 0 and p_i(x) > 0);
      on reject draw out[i] = ICDF(max(0, p_i - q_i), U(b, i, 1)) (p_i if that
      residual has no mass) and stop.
    If all gamma accept, out[gamma] = ICDF(p_gamma, U(b, gamma, 1)).

    Returns (out_tokens[B][gamma+1] int32 with -1 after the last emitted token,
    num_accepted[B] int32, decisions) where decisions[b] lists
    (slot, kind, margin) in order: kind "accept" (margin |u - p/q|, inf when
    q(x) = 0) or "draw" (margin from icdf()).

    uniform_fn(b, slot, stream), when given, replaces the Philox uniforms (used
    to enumerate the sampler's outcomes exactly in tests).
    """
    if uniform_fn is None:
        def uniform_fn(b, slot, stream):
            return uniform(seed, offset, b, slot, stream)
    B, gamma, V = draft_logits.shape
    out = np.full((B, gamma + 1), -1, dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    decisions = []
    for b in range(B):
        dec = []
        n = 0
        rejected = False
        for i in range(gamma):
            p = softmax(target_logits[b, i], temperature)
            q = softmax(draft_logits[b, i], temperature)
            x = int(draft_tokens[b, i])
            u = uniform_fn(b, i, 0)
            if q[x] > 0:
                ratio = p[x] / q[x]
                accept = u < ratio
                dec.append((i, "accept", abs(u - ratio)))
            else:
                accept = p[x] > 0
                dec.append((i, "accept", math.inf))
            if accept:
                out[b, i] = x
                n += 1
                continue
            w = np.maximum(0.0, p - q)
            if w.sum() == 0.0:
                w = p
            t, margin = icdf(w, uniform_fn(b, i, 1))
            out[b, i] = t
            dec.append((i, "draw", margin))
            rejected = True
            break
        if not rejected:
            p = softmax(target_logits[b, gamma], temperature)
            t, margin = icdf(p, uniform_fn(b, gamma, 1))
            out[b, gamma] = t
            dec.append((gamma, "draw", margin))
        n_acc[b] = n
        decisions.append(dec)
    return out, n_acc, decisions


def draw_tokens(logits, temperature, seed, offset, first_slot=0):
    """Direct sampling from a row's own softmax: the drafter's draws.

    S3R Abstract: the sparse-attention policy proposes tokens; sampling from it
    directly, with no dense check, is the comparator the abstract calls
    unstable. Row r of sequence b (logits[b][r], one draft position) draws
      x[b][r] = ICDF(softmax(logits[b][r] / T), U(b, first_slot + r, 2)),
    stream 2 being the drafter's own uniforms; first_slot lets a drafter that
    samples one position at a time use the slot of that position.

    Returns (x[B][R] int32, margin[B][R]) with margin as in icdf().
    """
    B, R, _ = logits.shape
    x = np.empty((B, R), dtype=np.int32)
    margin = np.empty((B, R))
    for b in range(B):
        for r in range(R):
            x[b, r], margin[b, r] = icdf(softmax(logits[b, r], temperature),
                                         uniform(seed, offset, b, first_slot + r, 2))
    return x, margin


def draw_draft_tokens(draft_logits, temperature, seed, offset):
    """x[b][i] = ICDF(q_i, U(b, i, 2)): the drafter's own draws from q_i."""
    return draw_tokens(draft_logits, temperature, seed, offset)[0]


def acceptance_rate(draft_logits, target_logits, temperature):
    """alpha[b][i] = sum_x min(p_i(x), q_i(x)) for the gamma draft positions.

    p_i = softmax(target_logits[b][i] / T), q_i = softmax(draft_logits[b][i] / T).
    Under the speculative-sampling rule (the titles the S3R reference list
    cites) a draft x ~ q_i is accepted with probability min(1, p_i(x)/q_i(x)),
    so the chance of accepting position i is sum_x q_i(x) min(1, p_i/q_i) =
    alpha_i; and 1 - alpha_i is the total-variation distance TV(p_i, q_i), how
    far one token sampled directly from the sparse policy is from the dense
    policy's law (the direct-sparse-sampling comparator of the S3R Abstract).
    target_logits may hold gamma + 1 rows; the bonus row has no draft partner
    and is not used. Returns alpha[B][gamma] float64.
    """
    B, gamma, _ = draft_logits.shape
    alpha = np.empty((B, gamma))
    for b in range(B):
        for i in range(gamma):
            p = softmax(target_logits[b, i], temperature)
            q = softmax(draft_logits[b, i], temperature)
            alpha[b, i] = float(np.minimum(p, q).sum())
    return alpha
