"""Plain fp64 CPU oracle for the FlashAttention-style attention forward pass.

TEST INFRASTRUCTURE ONLY.  This module exists to check the HIP path.  Only the
test suite, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` may import it; nothing on the product path calls it, and it shares
no code, tables or helpers with the HIP library.

Sources, cited by page title and section:

* [cuTile]  "Tuning Flash Attention for peak performance in NVIDIA CUDA Tile"
            (NVIDIA technical blog post on cuTile, Japanese-titled mirror).
* [Journey] "How I Beat PyTorch's Flash Attention: A CUDA Optimization Journey".
* [Tiled]   "TiledAttention: a CUDA Tile SDPA Kernel for PyTorch" (abstract and
            Figure 1).

What is computed (every input is converted exactly to float64 first):

    kvh    = hq // (Hq // Hkv)                                  [cuTile] "Grouped-query attention"
    V(i)   = { j < Skv : not causal  or  j <= input_pos + i }   [cuTile] "Causal attention",
                                                                 Part 1 "Applying the causal mask"
             minus { j < input_pos + i - W + 1 } for a sliding window of W >= 1 keys
             (causal only; [Journey] "Future work" names sliding-window attention)
    s_j    = scale * <q[b,hq,i,:], k[b,kvh,j,:]>     for j in V(i)
    O      = sum_j exp(s_j - m) v[b,kvh,j,:] / sum_j exp(s_j - m),  m = max_j s_j
    LSE    = m + ln(sum_j exp(s_j - m))

The attention formula itself was lost when the [cuTile] page was extracted
("What is attention?"); the textbook reading softmax(scale * Q K^T + M) V is
the one its kernel code (Part 1, "Online softmax update" and "Final
normalization and store") implements, with the default scale 1/sqrt(D) from
its host code ("Launching the kernel: Host-side code").  The log-sum-exp output
is on no page; it is read as the natural-log log-sum-exp of the scaled, masked
scores of each row.  The sliding window is only named on the pages; it is read as
the common causal form in which query i sees the W most recent keys up to its own
position.  A row whose V(i) is empty (possible only with a window, when
input_pos + i - W + 1 >= Skv) is read as O = 0 and LSE = -inf, the values of an
empty sum.

Several forms are provided, written independently of one another:

* ``attention_naive``          pure-Python loops over the definition (tiny shapes);
* ``attention_blocked``        the definition with NumPy matmuls, row block by row
                               block (the oracle used for parity and the CPU baseline);
* ``attention_online_tiled``   online softmax over key blocks: a running (max, sum,
                               output) state per query block, folded one key block
                               at a time, with fully masked blocks skipped and the
                               mask consulted only on partly visible blocks.
* ``attention_key_range`` and ``merge_partials``: the definition over one key
                               range, and the online-softmax fold of several ranges
                               into one result (split-KV).
* ``fp8_e4m3_decode`` and ``attention_fp8_blocked``: fp8 E4M3 codes decoded
                               from the format's definition, and the definition over
                               dequantised fp8 queries and keys (and values).
* ``attention_backward_blocked``: the gradients dQ, dK, dV from the softmax
                               derivative (the backward pass); ``attention_backward_sampled``
                               evaluates them at sampled rows of full-size problems.

Parity status: every function here is pinned by the CPU test suite against
brute force, an independent library routine (PyTorch's CPU float64
scaled_dot_product_attention), closed forms and invariants.  Nothing is
"parity unpinned".
"""

from __future__ import annotations

import math

import numpy as np

LN2 = math.log(2.0)
LOG2E = 1.0 / LN2


# ----------------------------------------------------------------------------
# Shape checks shared by the NumPy forms (argument checking only, no arithmetic)
# ----------------------------------------------------------------------------

def _shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if k.shape != v.shape or Bk != B or Dk != D:
        raise ValueError(f"shape mismatch q{q.shape} k{k.shape} v{v.shape}")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if Skv < 1:
        raise ValueError("Skv must be >= 1")
    return B, Hq, Hkv, Sq, Skv, D


# ----------------------------------------------------------------------------
# Form (i): pure-Python loops over the definition
# ----------------------------------------------------------------------------

def attention_naive(q, k, v, scale, causal=False, input_pos=0, window=0):
    """Brute-force definition with pure-Python loops; float64; tiny shapes only.

    Follows [cuTile] "What is attention?" (textbook softmax(scale Q K^T + M) V),
    "Causal attention" (key j visible to query i iff j is not later than the
    query's position input_pos + i, Part 1 "Initializing accumulators") and
    "Grouped-query attention" (query heads in contiguous groups of Hq/Hkv share
    one K/V head).  window > 0 (causal only) also hides
    keys before input_pos + i - window + 1; a row left with no key gets O = 0,
    LSE = -inf.

    Returns (O [B,Hq,Sq,D], LSE [B,Hq,Sq]) as float64 arrays.
    """
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    ql, kl, vl = np.asarray(q, np.float64).tolist(), np.asarray(k, np.float64).tolist(), \
        np.asarray(v, np.float64).tolist()
    O = np.zeros((B, Hq, Sq, D))
    L = np.zeros((B, Hq, Sq))
    for b in range(B):
        for hq in range(Hq):
            g = hq // group
            for i in range(Sq):
                first, last = 0, Skv - 1
                if causal:
                    last = min(last, input_pos + i)
                    if window > 0:
                        first = max(0, input_pos + i - window + 1)
                if first > last:
                    L[b, hq, i] = -math.inf
                    continue
                qi = ql[b][hq][i]
                s = []
                for j in range(first, last + 1):
                    kj = kl[b][g][j]
                    acc = 0.0
                    for d in range(D):
                        acc += qi[d] * kj[d]
                    s.append(scale * acc)
                m = max(s)
                e = [math.exp(x - m) for x in s]
                den = sum(e)
                for d in range(D):
                    num = 0.0
                    for n, j in enumerate(range(first, last + 1)):
                        num += e[n] * vl[b][g][j][d]
                    O[b, hq, i, d] = num / den
                L[b, hq, i] = m + math.log(den)
    return O, L


def attention_probs_naive(q, k, scale, causal=False, input_pos=0):
    """The attention-weight matrix P = softmax(scale Q K^T + M), pure Python, float64.

    [cuTile] "What is attention?" and "Causal attention": masked entries are
    exactly zero.  Returns P [B, Hq, Sq, Skv].
    """
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    ql, kl = np.asarray(q, np.float64).tolist(), np.asarray(k, np.float64).tolist()
    P = np.zeros((B, Hq, Sq, Skv))
    for b in range(B):
        for hq in range(Hq):
            g = hq // group
            for i in range(Sq):
                last = Skv - 1 if not causal else min(Skv - 1, input_pos + i)
                s = [scale * sum(ql[b][hq][i][d] * kl[b][g][j][d] for d in range(D))
                     for j in range(last + 1)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                den = sum(e)
                for j in range(last + 1):
                    P[b, hq, i, j] = e[j] / den
    return P


# ----------------------------------------------------------------------------
# Form (ii): the definition, NumPy matmuls, one block of query rows at a time
# ----------------------------------------------------------------------------

def kv_head_of(hq, Hq, Hkv):
    """Index of the K/V head that query head ``hq`` reads.

    [cuTile] "Grouped-query attention" and Part 1 "Block ID mapping":
    kv_head = head // query_group_size with query_group_size = Hq // Hkv, so
    query heads 0..G-1 share K/V head 0, G..2G-1 share head 1, and so on.
    """
    return hq // (Hq // Hkv)


def key_visibility(rows, Skv, causal, input_pos, window=0):
    """Boolean [len(rows), Skv]: may query row i attend to key j?

    [cuTile] "Causal attention" and Part 1 "Applying the causal mask": with
    causal masking key j is visible iff j <= input_pos + i (the query position
    carries input_pos, Part 1 "Initializing accumulators"); without it every
    key 0..Skv-1 is visible and input_pos plays no part.  A sliding window of
    W = window > 0 keys (causal only) also requires j >= input_pos + i - W + 1.
    """
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.arange(Skv, dtype=np.int64)
    if not causal:
        return np.ones((rows.size, Skv), dtype=bool)
    pos = rows[:, None] + input_pos
    vis = cols[None, :] <= pos
    if window > 0:
        vis &= cols[None, :] >= pos - window + 1
    return vis


def scaled_scores(q_rows, k_head, scale):
    """scale * Q K^T for a block of query rows against one K head (float64).

    [cuTile] "What is attention?"; the scale multiplies the raw dot products
    (Part 1 "Online softmax update", default 1/sqrt(D) from the host code).
    """
    return scale * (q_rows @ k_head.T)


def masked_softmax_stats(s, visible):
    """Row maximum m, un-normalised weights e = exp(s - m) and row sum l.

    Masked entries contribute nothing ([cuTile] "Causal attention": adding -inf
    makes them zero after the softmax).  This is the numerically safe softmax
    of "Understanding online softmax", computed over the whole row at once.
    """
    s = np.where(visible, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return m, e, l


def normalise(e, l, v_head):
    """O = (e V) / l: [cuTile] Part 1 "Final normalization and store"."""
    return (e @ v_head) / l


def log_sum_exp(m, l):
    """Natural-log log-sum-exp of the scaled, masked scores: m + ln(l)."""
    return m[:, 0] + np.log(l[:, 0])


def attention_blocked(q, k, v, scale, causal=False, input_pos=0, rows_per_block=512, window=0):
    """The definition in float64 with NumPy matmuls, ``rows_per_block`` query rows at a time.

    Row blocking only bounds memory: every row is computed from its full set of
    visible scores in one pass, exactly as defined (module docstring); rows
    with no visible key (sliding window only) get O = 0 and LSE = -inf.  A block
    reads only the keys from the first to the last one that some row of the
    block can see: the keys outside that span are masked for every row of the
    block, so they would add exp(-inf) = 0 to every sum.
    Returns (O [B,Hq,Sq,D], LSE [B,Hq,Sq]) as float64 arrays.
    """
    B, Hq, Hkv, Sq, Skv, D = _shapes(q, k, v)
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and > 0")
    _check_window(causal, window)
    O = np.zeros((B, Hq, Sq, D))
    L = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for hq in range(Hq):
            g = kv_head_of(hq, Hq, Hkv)
            kh = np.asarray(k[b, g], np.float64)
            vh = np.asarray(v[b, g], np.float64)
            for i0 in range(0, Sq, rows_per_block):
                i1 = min(Sq, i0 + rows_per_block)
                vis = key_visibility(np.arange(i0, i1), Skv, causal, input_pos, window)
                rows = i0 + np.nonzero(vis.any(axis=1))[0]
                if rows.size == 0:
                    continue
                j0, j1 = visible_key_span(vis[rows - i0])
                s = scaled_scores(np.asarray(q[b, hq, rows], np.float64), kh[j0:j1], scale)
                m, e, l = masked_softmax_stats(s, vis[rows - i0, j0:j1])
                O[b, hq, rows] = normalise(e, l, vh[j0:j1])
                L[b, hq, rows] = log_sum_exp(m, l)
    return O, L


def _check_window(causal, window):
    if window < 0:
        raise ValueError("window must be >= 0 (0 = no window)")
    if window > 0 and not causal:
        raise ValueError("a sliding window needs causal masking")


def attention_rows(q, k, v, scale, causal, input_pos, samples, window=0):
    """The blocked definition evaluated only at sampled rows.

    ``samples`` is an iterable of (b, hq, i).  Used to check full-size runs
    whose complete oracle would take too long.  Returns (O [n,D], LSE [n]).
    """
    B, Hq, Hkv, Sq, Skv, D = _shapes(q, k, v)
    _check_window(causal, window)
    samples = list(samples)
    O = np.zeros((len(samples), D))
    L = np.full(len(samples), -np.inf)
    for n, (b, hq, i) in enumerate(samples):
        g = kv_head_of(hq, Hq, Hkv)
        vis = key_visibility([i], Skv, causal, input_pos, window)
        if not vis.any():
            continue
        last = int(np.nonzero(vis[0])[0].max()) + 1  # only rows up to the last visible key are read
        kh = np.asarray(k[b, g, :last], np.float64)
        vh = np.asarray(v[b, g, :last], np.float64)
        s = scaled_scores(np.asarray(q[b, hq, i:i + 1], np.float64), kh, scale)
        m, e, l = masked_softmax_stats(s, vis[:, :last])
        O[n] = normalise(e, l, vh)[0]
        L[n] = log_sum_exp(m, l)[0]
    return O, L


# ----------------------------------------------------------------------------
# Form (iii): online softmax, one key block at a time
# ----------------------------------------------------------------------------

def _cdiv(a, b):
    return -(-a // b)


def visible_key_span(vis):
    """(first, last + 1) of the keys that at least one row of a visibility block sees.

    Keys outside this span are masked for every row of the block.  Requires a
    block in which some row sees some key.
    """
    seen = np.nonzero(vis.any(axis=0))[0]
    return int(seen[0]), int(seen[-1]) + 1


def tile_plan(q_tile, tile_m, tile_n, Skv, causal, input_pos):
    """Key blocks a query block must visit, and how many leading blocks need no mask.

    Derived from the visibility rule (``key_visibility``) for the rows
    q_tile*tile_m .. (q_tile+1)*tile_m - 1 (padded rows included, as a kernel
    computes them):
      * the latest key any of those rows sees is min(input_pos + last row,
        Skv - 1) under causal masking, else Skv - 1, so the blocks up to the one
        holding it are visited and the rest are skipped ([cuTile] Part 1, main
        loop over K/V tiles; "Causal attention": fully masked tiles are never
        loaded);
      * every row sees the keys 0 .. min(input_pos + first row, Skv - 1) under
        causal masking (all Skv keys otherwise); the whole key blocks inside
        that common prefix need no mask ([cuTile] Part 2 "K-loop split").
    Returns (n_visited, n_unmasked); n_unmasked <= n_visited.
    """
    first_row = q_tile * tile_m
    last_row = first_row + tile_m - 1
    last_key = min(input_pos + last_row, Skv - 1) if causal else Skv - 1
    common_keys = min(input_pos + first_row, Skv - 1) + 1 if causal else Skv
    n_visited = last_key // tile_n + 1
    return n_visited, min(common_keys // tile_n, n_visited)


def classify_tiles(Sq, Skv, tile_m, tile_n, causal, input_pos=0):
    """Count (unmasked, masked, skipped) K/V tiles over all query tiles.

    [cuTile] Part 2 "K-loop split": tiles inside every row's visible prefix run
    without mask code, the other visited tiles build the mask, and the rest
    are skipped.  Without causal masking and with Skv a whole number of tiles,
    no tile needs a mask.
    """
    n_q = _cdiv(Sq, tile_m)
    n_k = _cdiv(Skv, tile_n)
    unmasked = masked = 0
    for t in range(n_q):
        visited, free = tile_plan(t, tile_m, tile_n, Skv, causal, input_pos)
        unmasked += free
        masked += visited - free
    return unmasked, masked, n_q * n_k - unmasked - masked


def _block_state(s, vis, v_blk):
    """Partial softmax state of one key block: its row maximum, its row sum of
    exp(s - max) and its un-normalised output, over the visible entries only.
    A row with no visible entry in the block gets (-inf, 0, 0)."""
    s = np.where(vis, s, -np.inf)
    blk_max = s.max(axis=1)
    ref = np.where(np.isfinite(blk_max), blk_max, 0.0)
    w = np.exp(s - ref[:, None])
    return blk_max, w.sum(axis=1), w @ v_blk


def _fold(state, part):
    """Combine two partial softmax states over disjoint key sets ("Understanding
    online softmax": when the running maximum grows, what was summed so far is
    scaled by exp(old max - new max)).  -inf maxima carry zero weight."""
    run_max, run_sum, run_out = state
    blk_max, blk_sum, blk_out = part
    new_max = np.maximum(run_max, blk_max)
    ref = np.where(np.isfinite(new_max), new_max, 0.0)
    a = np.where(np.isfinite(run_max), np.exp(run_max - ref), 0.0)
    c = np.where(np.isfinite(blk_max), np.exp(blk_max - ref), 0.0)
    return new_max, a * run_sum + c * blk_sum, a[:, None] * run_out + c[:, None] * blk_out


def attention_online_tiled(q, k, v, scale, causal=False, input_pos=0, tile_m=64, tile_n=64,
                           split_loop=True):
    """Online softmax over key blocks, in float64, one (batch, head, query block) at a time.

    The algorithm of [cuTile] "How Flash Attention solves the memory bandwidth
    problem" and "Understanding online softmax": a query block keeps a running
    (maximum, sum, un-normalised output) and folds in one key block after
    another; only at the end is the output divided by the sum and the
    log-sum-exp formed (Part 1, final normalisation).  The key blocks visited
    and the ones that need no mask come from ``tile_plan``: blocks past the
    last visible key are never touched, and with ``split_loop`` the blocks
    every row sees in full are folded without consulting the mask (Part 2
    "K-loop split"); with ``split_loop`` False every block is masked.  Rows past
    Sq are not formed; keys past Skv do not exist.  The log-sum-exp (on no page)
    is max + ln(sum).  The GQA head map is ``kv_head_of``.
    Returns (O [B,Hq,Sq,D], LSE [B,Hq,Sq]).
    """
    B, Hq, Hkv, Sq, Skv, D = _shapes(q, k, v)
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and > 0")
    O = np.empty((B, Hq, Sq, D))
    L = np.empty((B, Hq, Sq))
    for b in range(B):
        for hq in range(Hq):
            g = kv_head_of(hq, Hq, Hkv)
            kh = np.asarray(k[b, g], np.float64)
            vh = np.asarray(v[b, g], np.float64)
            for qt in range(_cdiv(Sq, tile_m)):
                r0, r1 = qt * tile_m, min(Sq, (qt + 1) * tile_m)
                q_blk = np.asarray(q[b, hq, r0:r1], np.float64)
                n = r1 - r0
                state = (np.full(n, -np.inf), np.zeros(n), np.zeros((n, D)))
                n_visited, n_free = tile_plan(qt, tile_m, tile_n, Skv, causal, input_pos)
                for kt in range(n_visited):
                    c0, c1 = kt * tile_n, min(Skv, (kt + 1) * tile_n)
                    s = scaled_scores(q_blk, kh[c0:c1], scale)
                    if split_loop and kt < n_free:
                        vis = np.ones(s.shape, dtype=bool)
                    else:
                        vis = key_visibility(np.arange(r0, r1), Skv, causal, input_pos)[:, c0:c1]
                    state = _fold(state, _block_state(s, vis, vh[c0:c1]))
                run_max, run_sum, run_out = state
                O[b, hq, r0:r1] = run_out / run_sum[:, None]
                L[b, hq, r0:r1] = run_max + np.log(run_sum)
    return O, L


# ----------------------------------------------------------------------------
# Form (iv): attention over a key range, and the merge of ranges (split-KV)
# ----------------------------------------------------------------------------

def attention_key_range(q, k, v, scale, causal, input_pos, key_lo, key_hi, window=0):
    """The definition with each row's visible keys cut to key_lo <= j < key_hi.

    The pages split the work over query tiles only; splitting the key loop is
    the answer here to launches with too few query tiles to fill the GPU
    ([cuTile] Part 2 "Autotuning", [Journey] "Phase 5: Adaptive Tile
    Dispatch").  Each range is the module-docstring definition over V(i)
    intersected with [key_lo, key_hi).  Returns (O_s [B,Hq,Sq,D], LSE_s
    [B,Hq,Sq]) as float64; a row with no visible key in the range gets
    O_s = 0 and LSE_s = -inf (the log of an empty sum).
    """
    B, Hq, Hkv, Sq, Skv, D = _shapes(q, k, v)
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and > 0")
    O = np.zeros((B, Hq, Sq, D))
    L = np.full((B, Hq, Sq), -np.inf)
    _check_window(causal, window)
    in_range = (np.arange(Skv) >= key_lo) & (np.arange(Skv) < key_hi)
    vis = key_visibility(np.arange(Sq), Skv, causal, input_pos, window) & in_range[None, :]
    rows = np.nonzero(vis.any(axis=1))[0]
    if rows.size == 0:
        return O, L
    for b in range(B):
        for hq in range(Hq):
            g = kv_head_of(hq, Hq, Hkv)
            kh = np.asarray(k[b, g], np.float64)
            vh = np.asarray(v[b, g], np.float64)
            s = scaled_scores(np.asarray(q[b, hq, rows], np.float64), kh, scale)
            m, e, l = masked_softmax_stats(s, vis[rows])
            O[b, hq, rows] = normalise(e, l, vh)
            L[b, hq, rows] = log_sum_exp(m, l)
    return O, L


def merge_partials(o_parts, lse_parts):
    """Fold per-range results (O_s, LSE_s) into the attention over all the ranges.

    This is the [cuTile] online-softmax update (Part 1 "Online softmax update",
    "Accumulating the output", "Final normalization and store") with whole key
    ranges in place of K/V tiles, in natural-log units.  A range enters as the
    state (m, l, acc) = (LSE_s, 1, O_s): after a range the kernel holds m and l
    with m + ln l = LSE_s and acc / l = O_s, and scaling l and acc by one
    common factor changes neither O nor LSE.  For each range in turn:

        m_new = max(m, LSE_s);  alpha = exp(m - m_new);  beta = exp(LSE_s - m_new)
        l = alpha * l + beta;   acc = alpha * acc + beta * O_s;   m = m_new

    and at the end O = acc / l, LSE = m + ln l.  A range with LSE_s = -inf (no
    visible key) has weight 0; when every range is empty, O = 0, LSE = -inf.

    o_parts: [S, ..., D]; lse_parts: [S, ...].  Returns (O [..., D], LSE [...]).
    """
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    m = np.full(lse_parts.shape[1:], -np.inf)
    l = np.zeros(lse_parts.shape[1:])
    acc = np.zeros(o_parts.shape[1:])
    for o_s, lse_s in zip(o_parts, lse_parts):
        m_new = np.maximum(m, lse_s)
        live = m_new > -np.inf               # some range so far has a visible key
        safe = np.where(live, m_new, 0.0)
        alpha = np.where(live, np.exp(m - safe), 1.0)
        beta = np.where(live, np.exp(lse_s - safe), 0.0)
        l = alpha * l + beta
        acc = alpha[..., None] * acc + beta[..., None] * o_s
        m = m_new
    nonempty = l > 0
    O = np.where(nonempty[..., None], acc / np.where(nonempty, l, 1.0)[..., None], 0.0)
    LSE = np.where(nonempty, m + np.log(np.where(nonempty, l, 1.0)), -np.inf)
    return O, LSE


# ----------------------------------------------------------------------------
# fp8 inputs: decoding E4M3 codes, and attention over dequantised q and k
# ----------------------------------------------------------------------------

def fp8_e4m3_decode(codes):
    """Values of fp8 E4M3 codes (the OCP "E4M3FN" variant): float64 array.

    Bit layout, sign-exponent-mantissa = 1-4-3, exponent bias 7.  Exponent field 0
    encodes subnormals m * 2^-9 (and zero); exponent 1..15 encodes (1 + m/8) *
    2^(e-7), except that exponent 15 with mantissa 7 is NaN -- the format has no
    infinities, so its largest finite value is 1.75 * 2^8 = 448.  The pages give
    no low-precision format; this is the one gfx950's fp8 matrix instructions read.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def attention_fp8_blocked(q_codes, k_codes, v, scale, q_descale, k_descale, causal=False,
                          input_pos=0, window=0, v_descale=None):
    """Attention of fp8-coded queries and keys: the module-docstring definition applied
    to q = q_descale * decode(q_codes), k = k_descale * decode(k_codes) and v, in
    float64 (``attention_blocked``).  With ``v_descale`` given, v holds fp8 codes as well
    and the values are v_descale * decode(v).  Returns (O, LSE)."""
    factors = [q_descale, k_descale] + ([] if v_descale is None else [v_descale])
    if not all(math.isfinite(f) and f > 0 for f in factors):
        raise ValueError("descale factors must be finite and > 0")
    q = q_descale * fp8_e4m3_decode(q_codes)
    k = k_descale * fp8_e4m3_decode(k_codes)
    vv = np.asarray(v, np.float64) if v_descale is None else v_descale * fp8_e4m3_decode(v)
    return attention_blocked(q, k, vv, scale, causal, input_pos, window=window)


# ----------------------------------------------------------------------------
# Form (v): the backward pass (gradients of O with respect to q, k, v)
# ----------------------------------------------------------------------------

def attention_backward_blocked(q, k, v, do, scale, causal=False, input_pos=0, window=0,
                               rows_per_block=512):
    """Gradients of the forward pass, written out from the softmax derivative, float64.

    With S = scale * Q K^T (masked), P = softmax(S) row-wise, O = P V and an upstream
    gradient dO ([Journey] "Future work" names the backward pass; the pages give no
    formulas for it, so these are the textbook derivatives):

        dV = P^T dO
        dP = dO V^T
        D_i = sum_j P_ij dP_ij  (= dO_i . O_i)
        dS = P * (dP - D)       (elementwise; zero where masked)
        dQ = scale * dS K,      dK = scale * dS^T Q

    Under grouped-query attention dK and dV of a K/V head sum the contributions of every
    query head in its group.  Rows with no visible key contribute nothing.  Returns
    (dQ, dK, dV) as float64 arrays of q's and k's shapes.
    """
    B, Hq, Hkv, Sq, Skv, D = _shapes(q, k, v)
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and > 0")
    _check_window(causal, window)
    do = np.asarray(do, np.float64)
    if do.shape != (B, Hq, Sq, D):
        raise ValueError("do must have q's shape")
    dQ = np.zeros((B, Hq, Sq, D))
    dK = np.zeros((B, Hkv, Skv, D))
    dV = np.zeros((B, Hkv, Skv, D))
    for b in range(B):
        for hq in range(Hq):
            g = kv_head_of(hq, Hq, Hkv)
            kh = np.asarray(k[b, g], np.float64)
            vh = np.asarray(v[b, g], np.float64)
            for i0 in range(0, Sq, rows_per_block):
                i1 = min(Sq, i0 + rows_per_block)
                vis = key_visibility(np.arange(i0, i1), Skv, causal, input_pos, window)
                rows = i0 + np.nonzero(vis.any(axis=1))[0]
                if rows.size == 0:
                    continue
                qr = np.asarray(q[b, hq, rows], np.float64)
                s = scaled_scores(qr, kh, scale)
                m, e, l = masked_softmax_stats(s, vis[rows - i0])
                P = e / l
                dOr = do[b, hq, rows]
                dV[b, g] += P.T @ dOr
                dP = dOr @ vh.T
                Dr = (P * dP).sum(axis=1, keepdims=True)
                dS = P * (dP - Dr)
                dQ[b, hq, rows] = scale * (dS @ kh)
                dK[b, g] += scale * (dS.T @ qr)
    return dQ, dK, dV


def attention_backward_sampled(q, k, v, do, scale, causal, input_pos, dq_samples, dkv_samples,
                               window=0):
    """The gradients of ``attention_backward_blocked`` evaluated at sampled rows only.

    ``dq_samples``: (b, hq, i) query rows whose dQ row is wanted; ``dkv_samples``: (b, g, j)
    key rows whose dK and dV rows are wanted.  A dQ row needs only its own softmax row.  A
    dK / dV row sums over every query row of every query head in its group that sees the
    key, and each term needs that query row's normaliser and D_i = sum_j P_ij dP_ij, so
    the (b, g) groups named in ``dkv_samples`` get their row statistics (log-sum-exp and
    D) for all query rows first, then the sampled keys' columns of P and dS.  The
    formulas are those of ``attention_backward_blocked``.  Returns (dQ [n, D], dK [m, D],
    dV [m, D]) as float64 arrays.
    """
    B, Hq, Hkv, Sq, Skv, D = _shapes(q, k, v)
    if not (math.isfinite(scale) and scale > 0):
        raise ValueError("scale must be finite and > 0")
    _check_window(causal, window)
    do = np.asarray(do)
    if do.shape != (B, Hq, Sq, D):
        raise ValueError("do must have q's shape")
    group = Hq // Hkv
    dq_samples, dkv_samples = list(dq_samples), list(dkv_samples)

    # dQ rows: the whole softmax row of each sampled query.
    dQ = np.zeros((len(dq_samples), D))
    for n, (b, hq, i) in enumerate(dq_samples):
        g = kv_head_of(hq, Hq, Hkv)
        vis = key_visibility([i], Skv, causal, input_pos, window)
        if not vis.any():
            continue
        kh = np.asarray(k[b, g], np.float64)
        vh = np.asarray(v[b, g], np.float64)
        s = scaled_scores(np.asarray(q[b, hq, i:i + 1], np.float64), kh, scale)
        m, e, l = masked_softmax_stats(s, vis)
        P = e / l
        dO_i = np.asarray(do[b, hq, i:i + 1], np.float64)
        dP = dO_i @ vh.T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dQ[n] = scale * (dS @ kh)[0]

    # dK / dV rows: row statistics of the whole group, then the sampled key columns.
    dK = np.zeros((len(dkv_samples), D))
    dV = np.zeros((len(dkv_samples), D))
    for (b, g) in sorted({(b, g) for b, g, _ in dkv_samples}):
        kh = np.asarray(k[b, g], np.float64)
        vh = np.asarray(v[b, g], np.float64)
        heads = range(g * group, (g + 1) * group)
        lse = np.full((group, Sq), -np.inf)
        dvec = np.zeros((group, Sq))
        for t, hq in enumerate(heads):
            for i0 in range(0, Sq, 512):
                i1 = min(Sq, i0 + 512)
                vis = key_visibility(np.arange(i0, i1), Skv, causal, input_pos, window)
                rows = i0 + np.nonzero(vis.any(axis=1))[0]
                if rows.size == 0:
                    continue
                s = scaled_scores(np.asarray(q[b, hq, rows], np.float64), kh, scale)
                m, e, l = masked_softmax_stats(s, vis[rows - i0])
                P = e / l
                dP = np.asarray(do[b, hq, rows], np.float64) @ vh.T
                lse[t, rows] = log_sum_exp(m, l)
                dvec[t, rows] = (P * dP).sum(axis=1)
        vis_all = key_visibility(np.arange(Sq), Skv, causal, input_pos, window)
        for n, (bb, gg, j) in enumerate(dkv_samples):
            if (bb, gg) != (b, g):
                continue
            rows = np.nonzero(vis_all[:, j])[0]
            for t, hq in enumerate(heads):
                if rows.size == 0:
                    continue
                qr = np.asarray(q[b, hq, rows], np.float64)
                dOr = np.asarray(do[b, hq, rows], np.float64)
                s = scale * (qr @ kh[j])
                P = np.exp(s - lse[t, rows])
                dP = dOr @ vh[j]
                dS = P * (dP - dvec[t, rows])
                dV[n] += P @ dOr
                dK[n] += scale * (dS @ qr)
    return dQ, dK, dV

