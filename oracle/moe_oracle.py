"""CPU oracle of the fused MoE forward pass (numpy, fp64).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import or call this module; the product path never does.
It shares no code with the HIP library: it is written from the pages below
and pinned by the `-m "not gpu"` tests (brute force, library routines,
closed forms and hand-derived vectors), not by the GPU path.

Pages:
  [SLOTS]  TensorRT-LLM PR #4495 "large-scale EP (part 3: refactor - FusedMoe
           for redundant expert)", Description (Expert versus Expert Slot).
  [A2A]    TensorRT-LLM PR #10985 "MoE all-to-all paradigm": walkthrough
           sequence diagram; review of torch_moe.py (_template_moe,
           is_gated_mlp / act_fn, output-side routing).
  [EPMASK] vLLM ep_fused_moe_patch.py: module docstring ("EP expert
           dispatch"), ep_mask_and_remap, ep_reduce_output, _ep_init, and the
           FusedMoE constructor arguments (top_k, renormalize=True).
  [AUTOTP] DeepSpeed PR #6964 "AutoTP for MoE models": the routed output is
           the weighted sum of the selected experts' outputs.

Readings where the pages are silent (the pages give neither formula):
  - router: softmax of the logits, top-K by logit (descending, expert id
    ascending on ties), weights = the selected probabilities, renormalised
    to sum 1 when renormalize is set, before any EP masking;
  - expert MLP: SwiGLU gated MLP without biases,
    y = Wd (silu(Wg x) * (Wu x)), silu(z) = z / (1 + exp(-z));
  - masked (non-local) pairs are excluded from the permutation and compute;
  - the order of pairs inside one slot is ascending pair index p = t*K + k;
  - the replica of a local expert is chosen by token index: t mod r.
Precision: every floating-point step runs in fp64 on inputs decoded exactly
(bf16 and f32 values are exact in fp64). Integer outputs are exact.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np


def _f64(a) -> np.ndarray:
    """Exact fp64 copy of a numpy array or a CPU torch tensor (f32 or bf16)."""
    if hasattr(a, "detach"):  # torch tensor: bf16 -> f32 -> f64 is exact
        import torch
        return a.detach().to(torch.float64).cpu().numpy()
    return np.asarray(a, dtype=np.float64)


def _take_rows(a, rows: np.ndarray):
    """a[rows] for a numpy array or a torch tensor (before any conversion)."""
    if hasattr(a, "detach"):
        import torch
        return a[torch.from_numpy(np.ascontiguousarray(rows, dtype=np.int64))]
    return np.asarray(a)[rows]


def _i64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        return a.detach().cpu().numpy().astype(np.int64)
    return np.asarray(a, dtype=np.int64)


# --------------------------------------------------------------------------
# Route. [EPMASK] docstring: top-k routing produces the same global expert
# ids on every rank; FusedMoE constructor: top_k and renormalize (default
# True). The softmax and the order of the K ids are readings (see header).
# --------------------------------------------------------------------------
def softmax(logits) -> np.ndarray:
    """p[t, e] = exp(l[t,e] - max_e l[t]) / sum_j exp(l[t,j] - max_e l[t]), fp64."""
    l = _f64(logits)
    m = l.max(axis=1, keepdims=True)
    z = np.exp(l - m)
    return z / z.sum(axis=1, keepdims=True)


def topk_ids(logits, K: int) -> np.ndarray:
    """ids[t, :K]: experts ordered by logit descending, expert id ascending on
    ties (a stable sort of the negated logits; -0.0 equals +0.0)."""
    l = _f64(logits)
    T, E = l.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    # lexsort: last key is primary. Primary: -logit ascending; secondary: id.
    ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((ids, -l), axis=-1)
    return order[:, :K].astype(np.int32)


def route(logits, K: int, renormalize: bool) -> Tuple[np.ndarray, np.ndarray]:
    """(ids [T,K] int32, w [T,K] fp64): w[t,k] = p[t, ids[t,k]], divided by
    sum_k w[t,k] when renormalize is set."""
    p = softmax(logits)
    ids = topk_ids(logits, K)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w


# --------------------------------------------------------------------------
# Slot map. [EPMASK] ep_mask_and_remap (local mask, weights multiplied by the
# mask, local ids = id - start, non-local ids spread by id mod E_local) and
# _ep_init (E_local = E / ep_size, start = ep_rank * E_local, divisibility
# asserted); [SLOTS] Description (expert id -> expert slot; the identity map
# when every expert has one slot). Replica choice t mod r is a reading.
# --------------------------------------------------------------------------
def route_grouped(logits, K: int, renormalize: bool, num_groups: int,
                  topk_groups: int) -> Tuple[np.ndarray, np.ndarray]:
    """Group-limited routing ([EPMASK] FusedMoE constructor: use_grouped_topk,
    num_expert_group, topk_group; the pages name the options only). Reading:
    the E experts form num_groups consecutive groups; a group's score is the
    largest softmax probability among its experts (equivalently its largest
    logit); the topk_groups best groups are kept (score descending, group
    index ascending on ties) and the top-K experts are chosen among their
    experts only, with the same key as route(); the weights are the full
    softmax probabilities, renormalised over the K when renormalize is set."""
    l = _f64(logits)
    T, E = l.shape
    Eg = E // num_groups
    p = softmax(l)
    gmax = l.reshape(T, num_groups, Eg).max(axis=2)
    ids = np.empty((T, K), dtype=np.int64)
    for t in range(T):
        order = np.lexsort((np.arange(num_groups), -gmax[t]))[:topk_groups]
        keep = np.zeros(E, dtype=bool)
        for g in order:
            keep[g * Eg:(g + 1) * Eg] = True
        masked = np.where(keep, l[t], -np.inf)
        ids[t] = topk_ids(masked[None, :], K)[0]
    w = np.take_along_axis(p, ids, axis=1)
    if renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w


def ep_partition(E_global: int, ep_size: int, ep_rank: int) -> Tuple[int, int]:
    if ep_size < 1 or E_global % ep_size != 0:
        raise ValueError("E_global must be divisible by ep_size")
    if not 0 <= ep_rank < ep_size:
        raise ValueError("ep_rank out of range")
    E_local = E_global // ep_size
    return E_local, ep_rank * E_local


def ep_mask_and_remap(ids, w, start: int, E_local: int):
    """(local_ids, w_masked, mask) for one rank's expert range [start, start+E_local).

    [EPMASK] ep_mask_and_remap, stated per pair (t, k) with expert e:
      - the pair is local when e lies in [start, start + E_local);
      - its weight is multiplied by 1 when local and by 0 otherwise;
      - a local pair's local id is e - start; a non-local pair still gets an
        id inside [0, E_local), the non-negative residue of e modulo E_local,
        so that non-local pairs spread over the local experts instead of all
        naming expert 0. (Later stages skip non-local pairs.)
    """
    ids = _i64(ids)
    wt = _f64(w)
    T, K = ids.shape
    local_ids = np.empty((T, K), dtype=np.int64)
    w_masked = np.empty((T, K), dtype=np.float64)
    mask = np.empty((T, K), dtype=bool)
    for t in range(T):
        for k in range(K):
            e = int(ids[t, k])
            local = start <= e < start + E_local
            mask[t, k] = local
            w_masked[t, k] = wt[t, k] * (1.0 if local else 0.0)
            local_ids[t, k] = e - start if local else e % E_local  # Python %: non-negative
    return local_ids, w_masked, mask


def slot_map(ids, w, E_global: int, ep_size: int = 1, ep_rank: int = 0,
             rep_off=None, rep_slots=None):
    """(slot [T,K] int32, w_masked [T,K] fp64, mask [T,K] uint8)."""
    E_local, start = ep_partition(E_global, ep_size, ep_rank)
    lid, w_masked, mask = ep_mask_and_remap(ids, w, start, E_local)
    if rep_off is None:
        slot = lid
    else:
        off = _i64(rep_off)
        slots = _i64(rep_slots)
        t = np.arange(lid.shape[0])[:, None]
        r = off[lid + 1] - off[lid]
        slot = slots[off[lid] + t % r]
    return slot.astype(np.int32), w_masked, mask.astype(np.uint8)


# --------------------------------------------------------------------------
# Permute. [EPMASK] docstring: per-expert compute that skips empty experts,
# and the ragged gather that drops non-local pairs before compute. Order of
# equal slots: ascending pair index (a reading). The sort is a library
# stable sort; the counts are a library bincount.
# --------------------------------------------------------------------------
def permute_indices(slot, mask, S: int):
    """(offsets [S+1], sorted_pairs [P_in], pair_row [P]) as int32."""
    slot = _i64(slot).ravel()
    inc = (np.asarray(mask).ravel() != 0) & (slot >= 0) & (slot < S)
    pairs = np.nonzero(inc)[0]
    order = np.argsort(slot[pairs], kind="stable")
    sorted_pairs = pairs[order]
    counts = np.bincount(slot[pairs], minlength=S)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    pair_row = np.full(slot.size, -1, dtype=np.int64)
    pair_row[sorted_pairs] = np.arange(sorted_pairs.size)
    return offsets.astype(np.int32), sorted_pairs.astype(np.int32), pair_row.astype(np.int32)


def permute_rows(x: np.ndarray, sorted_pairs, K: int) -> np.ndarray:
    """x_perm[row] = x[sorted_pairs[row] // K] (a copy, any dtype)."""
    return np.asarray(x)[_i64(sorted_pairs) // K]


# --------------------------------------------------------------------------
# All-to-all dispatch. [A2A] walkthrough sequence diagram: the fused op sends
# tokens to the ranks responsible for their experts, each rank computes the
# MoE on its local experts, and the results are gathered back; the mapping
# configuration's max-num-tokens field sizes the exchange workspace.
# Readings: a token goes once to every rank that owns at least one of its K
# experts (owner of e = e // E_local), carrying its full routing; rank r's
# block holds at most max-num-tokens rows and starts at row r * cap; inside
# a block tokens keep ascending index; the gathered result of a token is the
# sum of the ranks' partial outputs in ascending rank order.
# --------------------------------------------------------------------------
def a2a_dispatch_indices(ids, E_global: int, ep_size: int, cap: int):
    """(counts [ep], send_token [ep*cap] (-1 where unused), token_pos [T, ep]
    (row of token t in rank r's block, or -1))."""
    ids = _i64(ids)
    T = ids.shape[0]
    E_local, _ = ep_partition(E_global, ep_size, 0)
    valid = (ids >= 0) & (ids < E_global)
    owner = np.where(valid, ids // E_local, -1)
    counts = np.zeros(ep_size, dtype=np.int64)
    send_token = np.full(ep_size * cap, -1, dtype=np.int64)
    token_pos = np.full((T, ep_size), -1, dtype=np.int64)
    for r in range(ep_size):
        toks = np.nonzero((owner == r).any(axis=1))[0]
        assert toks.size <= cap, "rank block over capacity"
        counts[r] = toks.size
        rows = r * cap + np.arange(toks.size)
        send_token[rows] = toks
        token_pos[toks, r] = rows
    return counts.astype(np.int32), send_token.astype(np.int32), token_pos.astype(np.int32)


def a2a_forward(x, ids, w, w_gate_up, w_down, E_global: int, ep_size: int, cap: int):
    """Dispatch, per-rank expert compute on the received tokens (each rank
    masks to its own experts), and the gather-sum back to token order."""
    x64 = _f64(x)
    T, H = x64.shape
    K = np.asarray(ids).shape[1]
    counts, send_token, token_pos = a2a_dispatch_indices(ids, E_global, ep_size, cap)
    partial = np.zeros((ep_size * cap, H))
    for r in range(ep_size):
        rows = r * cap + np.arange(int(counts[r]))
        toks = _i64(send_token[rows])
        if toks.size == 0:
            continue
        partial[rows] = forward(x64[toks], None, w_gate_up, w_down, K, False, ep_size, r,
                                topk=(_i64(ids)[toks], _f64(w)[toks]))
    out = np.zeros((T, H))
    for r in range(ep_size):  # ascending rank
        has = token_pos[:, r] >= 0
        out[has] += partial[_i64(token_pos[has, r])]
    return out


# --------------------------------------------------------------------------
# Expert MLP. [A2A] review of torch_moe.py: gated MLP with an activation
# function; SwiGLU is the gate taken here: silu(z) = z / (1 + exp(-z)).
# --------------------------------------------------------------------------
def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu_mlp(xrows, w_gate, w_up, w_down) -> np.ndarray:
    """y = (silu(x Wg^T) * (x Wu^T)) Wd^T for rows x [n, H]; Wg, Wu [I, H],
    Wd [H, I]. Library matmuls in fp64."""
    x = _f64(xrows)
    g = x @ _f64(w_gate).T
    u = x @ _f64(w_up).T
    return (silu(g) * u) @ _f64(w_down).T


def grouped_gate_up(a, offsets, w_gate_up, I: int) -> np.ndarray:
    """Stage form of grouped GEMM 1: rows [offsets[s], offsets[s+1]) of a use
    slot s's weights w_gate_up[s] ([2I, H], gate rows then up rows)."""
    a = _f64(a)
    off = _i64(offsets)
    out = np.zeros((a.shape[0], I))
    for s in range(off.size - 1):
        lo, hi = off[s], off[s + 1]
        if hi > lo:
            w = _f64(w_gate_up[s])
            out[lo:hi] = silu(a[lo:hi] @ w[:I].T) * (a[lo:hi] @ w[I:].T)
    return out


def grouped_down(a, offsets, w_down) -> np.ndarray:
    """Stage form of grouped GEMM 2: rows of slot s times w_down[s]^T ([H, I])."""
    a = _f64(a)
    off = _i64(offsets)
    H = w_down.shape[1]
    out = np.zeros((a.shape[0], H))
    for s in range(off.size - 1):
        lo, hi = off[s], off[s + 1]
        if hi > lo:
            out[lo:hi] = a[lo:hi] @ _f64(w_down[s]).T
    return out


# --------------------------------------------------------------------------
# Combine. [AUTOTP]: the routed output is the weighted sum of the selected
# experts' outputs; [A2A] _template_moe: routing weights applied on the
# output side. Sum over k ascending, included pairs only.
# --------------------------------------------------------------------------
def combine_rows(y, pair_row, w_masked, K: int) -> np.ndarray:
    """Stage form: out[t] = sum_k w_masked[t,k] * y[pair_row[t,k]] over pairs
    with pair_row >= 0."""
    y = _f64(y)
    pr = _i64(pair_row).reshape(-1, K)
    wm = _f64(w_masked).reshape(-1, K)
    T = pr.shape[0]
    out = np.zeros((T, y.shape[1]))
    for k in range(K):
        sel = pr[:, k] >= 0
        out[sel] += wm[sel, k, None] * y[pr[sel, k]]
    return out


# --------------------------------------------------------------------------
# Whole forward pass with expert-indexed weights.
# --------------------------------------------------------------------------
def forward(x, logits, w_gate_up, w_down, K: int, renormalize: bool,
            ep_size: int = 1, ep_rank: int = 0,
            tokens: Optional[Sequence[int]] = None,
            topk: Optional[Tuple[np.ndarray, np.ndarray]] = None,
            routing_on_input: bool = False, shared=None) -> np.ndarray:
    """Output rows for `tokens` (default: all), fp64 [n, H].

    x [T, H]; logits [T, E_global]; w_gate_up [E_global, 2I, H] and
    w_down [E_global, H, I] indexed by global expert id (slots are not used:
    replicas hold copies of the same expert). topk=(ids, w) replaces routing
    (the fused op given precomputed experts and weights, [A2A]).
    Each included pair (t, k) with expert e contributes
    w_masked[t,k] * MLP_e(x[t]); the MLP of expert e is evaluated for all of
    its pairs at once with library matmuls (each row independent).
    routing_on_input ([A2A] review: _template_moe's apply_routing_on_input):
    the pair contributes MLP_e(w_masked[t,k] * x[t]) instead.
    shared [T, H] ([EPMASK] ep_reduce_output: out = routed_out + shared_out):
    added to the routed sum of each returned token.
    """
    T = (logits.shape[0] if topk is None else np.asarray(topk[0]).shape[0])
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    if topk is None:
        ids, w = route(_f64(logits)[tok], K, renormalize)
    else:
        ids, w = np.asarray(topk[0])[tok], _f64(topk[1])[tok]
    E_global = w_gate_up.shape[0]
    E_local, start = ep_partition(E_global, ep_size, ep_rank)
    _, w_masked, mask = ep_mask_and_remap(ids, w, start, E_local)
    I = w_down.shape[2]
    xt = _f64(_take_rows(x, tok))
    n = tok.size
    y = np.zeros((n, K, xt.shape[1]))
    for e in range(start, start + E_local):
        sel = np.nonzero((ids == e) & mask)
        if sel[0].size == 0:
            continue
        wgu = _f64(w_gate_up[e])
        xin = xt[sel[0]]
        if routing_on_input:
            xin = w_masked[sel][:, None] * xin
        y[sel] = swiglu_mlp(xin, wgu[:I], wgu[I:], w_down[e])
    out = np.zeros((n, xt.shape[1]))
    for k in range(K):
        m = mask[:, k]
        out[m] += (1.0 if routing_on_input else w_masked[m, k, None]) * y[m, k]
    if shared is not None:
        out += _f64(_take_rows(shared, tok))
    return out


# --------------------------------------------------------------------------
# The same forward pass written literally, one pair at a time: [AUTOTP]
# Description (each token's routed output is the weighted sum of its selected
# experts' outputs) with the expert MLP of [A2A] evaluated as three
# matrix-vector products per pair. It cross-checks forward(), which evaluates
# each expert's rows together. Pairs are visited expert by expert only so
# that each expert's weights are decoded to fp64 once; the arithmetic of a
# pair does not depend on the other pairs.
# --------------------------------------------------------------------------
def forward_per_pair(x, logits, w_gate_up, w_down, K: int, renormalize: bool,
                     ep_size: int = 1, ep_rank: int = 0,
                     tokens: Optional[Sequence[int]] = None,
                     topk: Optional[Tuple[np.ndarray, np.ndarray]] = None) -> np.ndarray:
    """Output rows for `tokens` (default: all), fp64 [n, H]: for each token,
    the sum over k = 0..K-1 ascending of w_masked[t,k] * MLP_e(x[t]) over its
    local pairs, MLP_e(v) = Wd[e] (silu(Wg[e] v) * (Wu[e] v))."""
    T = (logits.shape[0] if topk is None else np.asarray(topk[0]).shape[0])
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    E_global = w_gate_up.shape[0]
    E_local, start = ep_partition(E_global, ep_size, ep_rank)
    I = w_down.shape[2]
    n = tok.size
    ids = np.empty((n, K), dtype=np.int64)
    wts = np.empty((n, K))
    for i, t in enumerate(tok):  # routing of one token at a time
        if topk is None:
            ri, rw = route(_f64(logits)[t:t + 1], K, renormalize)
        else:
            ri, rw = np.asarray(topk[0])[t:t + 1], _f64(topk[1])[t:t + 1]
        ids[i], wts[i] = ri[0], rw[0]
    _, w_masked, mask = ep_mask_and_remap(ids, wts, start, E_local)
    pairs = {}  # (i, k) -> expert output row
    for e in sorted({int(ids[i, k]) for i in range(n) for k in range(K) if mask[i, k]}):
        wgu = _f64(w_gate_up[e])
        wg, wu, wd = wgu[:I], wgu[I:], _f64(w_down[e])
        for i in range(n):
            for k in range(K):
                if mask[i, k] and ids[i, k] == e:
                    v = _f64(_take_rows(x, tok[i:i + 1]))[0]
                    a = silu(wg @ v) * (wu @ v)
                    pairs[(i, k)] = wd @ a
    out = np.zeros((n, w_down.shape[1]))
    for i in range(n):
        for k in range(K):
            if mask[i, k]:
                out[i] += w_masked[i, k] * pairs[(i, k)]
    return out
