"""Plain fp64 CPU oracle of the SparsePR per-call sparse attention operator.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
this module: only the tests, the smoke check and the bench's CPU-baseline leg
use it. It shares no code with the HIP path; the two meet only through the
seeded input generators, which hold none of the method's arithmetic.

Every step is written from the method's description on the pages, in their
order, with library primitives (matmul, sort, eigh, solve) as steps and no
blocking or fusion beyond that. Sources, cited by page and section:

* [AD]  arxivdaily 2608.18484, "English abstract" section: keys are grouped
        by how they respond to sampled queries (paired K/V groups); queries
        are grouped by their responses to the key-group centroids for shared
        routing; attention runs only between selected groups; a few query
        rows get exact attention; a weighted ridge regression fits an affine
        correction from sparse output to the dense-minus-sparse difference;
        the fitted map's predicted residual is added to each unprobed row;
        error is the per-query relative L2 against that query's dense output,
        averaged over unprobed queries; density counts the exact probes.
* [SK]  skillfed.io article "Partition the Support, Reconstruct the
        Residual: Training-Free Sparse Attention for Video Generation and World
        Models", paragraph introducing the two components: keys clustered by
        response profiles under a query sample; centroids define query
        coordinates; one asymmetric pass without alternating refinement;
        exact rows per head; a call-specific affine map applied within the
        output subspace seen in the probe residuals. Results paragraph:
        probe rows are counted in the executed-pair density.
* [PC]  peercurrent summary, abstract: centroids induce query-response
        coordinates; the correction is restricted to the probe residuals'
        output subspace.
* [CPU3D] cpu3d.com "SparsePR accelerates video generators with training-free
        sparse attention", summary: key responses to sampled queries form
        paired K/V groups.

Where the pages leave a step open the plainest reading is taken; each such
reading is named in the function that makes it (``Reading:``). The notation
follows the pages' prose: N tokens, d head dim, tau softmax scale, S sampled
queries, G key groups, T Lloyd iterations, B_q query block, rho density
including probes, m probes, k subspace rank, lambda ridge.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms, brute force, library reductions or invariants.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# Response-coupled partitioning, key side  ([AD], [SK] two components, [CPU3D])
# ---------------------------------------------------------------------------

def key_responses(Q, K, scale, sample_idx):
    """Response profile of every key: r_j = tau * Q[sample_idx] k_j, shape [N, S].

    Reading: a key's "response" to a sampled query is the scaled attention
    logit tau * q_s . k_j (the quantity the softmax consumes).
    """
    Qs = np.asarray(Q, F64)[np.asarray(sample_idx)]
    return F64(scale) * (np.asarray(K, F64) @ Qs.T)


def squared_distances(X, C):
    """D[j, g] = ||x_j - c_g||^2, expanded as ||x||^2 - 2 x.c + ||c||^2."""
    X = np.asarray(X, F64)
    C = np.asarray(C, F64)
    return (X * X).sum(1)[:, None] - 2.0 * (X @ C.T) + (C * C).sum(1)[None, :]


def argmin_lowest(D):
    """Row-wise argmin; on exact ties the lowest column wins."""
    return np.argmin(np.asarray(D), axis=1).astype(np.int64)


def group_means(X, labels, n_groups, previous=None):
    """Mean of the rows of X in each group. A group with no member keeps
    ``previous[g]`` (zeros when no previous centroids are given)."""
    X = np.asarray(X, F64)
    labels = np.asarray(labels)
    out = np.zeros((n_groups, X.shape[1]), F64) if previous is None else np.array(previous, F64)
    sizes = np.bincount(labels, minlength=n_groups)
    order = np.argsort(labels, kind="stable")
    starts = np.concatenate([[0], np.cumsum(sizes)[:-1]])
    nz = np.nonzero(sizes)[0]
    if nz.size:
        sums = np.add.reduceat(X[order], starts[nz], axis=0)
        out[nz] = sums / sizes[nz, None]
    return out, sizes


@dataclass
class KMeansResult:
    labels: np.ndarray           # [N] final labels (those of the T-th assignment)
    centroids: np.ndarray        # [G, S] response-space centroids after the T-th update
    scores: List[np.ndarray] = field(default_factory=list)   # per iteration D [N, G]
    labels_per_iter: List[np.ndarray] = field(default_factory=list)
    objective: List[float] = field(default_factory=list)      # sum_j D[j, a_j] per iteration


def kmeans(X, init_idx, iters, keep_scores=False):
    """Lloyd k-means of the rows of X (squared Euclidean).

    Reading: the pages name no clustering algorithm; this is plain Lloyd
    iteration with T fixed steps, initial centroids = the rows at
    ``init_idx`` (so labels are ordered by init order), lowest-index
    tie-break, and an empty group keeping its previous centroid.
    """
    X = np.asarray(X, F64)
    C = X[np.asarray(init_idx)].copy()
    res = KMeansResult(labels=np.zeros(X.shape[0], np.int64), centroids=C)
    G = C.shape[0]
    for _ in range(iters):
        D = squared_distances(X, C)
        lab = argmin_lowest(D)
        res.objective.append(float(D[np.arange(X.shape[0]), lab].sum()))
        if keep_scores:
            res.scores.append(D)
        res.labels_per_iter.append(lab)
        C, _ = group_means(X, lab, G, previous=C)
        res.labels = lab
    res.centroids = C
    return res


def group_members(labels, n_groups):
    """Group-contiguous key order: keys sorted by (label, token index).

    Returns ``key_perm`` [N] (position -> key token), ``group_off`` [G+1]
    and ``sizes`` [G]. Group g's keys are key_perm[group_off[g]:group_off[g+1]].
    """
    labels = np.asarray(labels)
    key_perm = np.argsort(labels, kind="stable").astype(np.int64)
    sizes = np.bincount(labels, minlength=n_groups).astype(np.int64)
    group_off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return key_perm, group_off, sizes


def random_block_labels(rand_key_perm, n_groups):
    """Random-block ablation (no response-coupled partitioning, [SK] ablation
    paragraph): the seeded permutation is cut into G near-equal runs,
    run g = positions floor(gN/G) .. floor((g+1)N/G)-1."""
    perm = np.asarray(rand_key_perm)
    n = perm.size
    lab = np.empty(n, np.int64)
    for g in range(n_groups):
        lo, hi = (g * n) // n_groups, ((g + 1) * n) // n_groups
        lab[perm[lo:hi]] = g
    return lab


def semantic_order(X, init_idx, iters, n_groups):
    """Semantic block-sparse comparator ([AD]: the error reduction is measured
    against semantic block-sparse attention without residual correction).

    Reading: the pages name the comparator but do not define it. Its
    partition here is the same Lloyd k-means as ``kmeans`` (T steps, initial
    centroids = the rows at ``init_idx``, lowest-index ties, empty groups
    keep their centroid) on the raw feature rows X instead of on response
    profiles, and the rows are ordered by (cluster, token). Applied to K it
    gives the key groups; applied to Q, the query order.
    Returns (labels, order).
    """
    km = kmeans(X, init_idx, iters)
    order, _, _ = group_members(km.labels, n_groups)
    return km.labels, order


# ---------------------------------------------------------------------------
# Query coordinates, grouping and shared routing  ([AD], [PC], [SK])
# ---------------------------------------------------------------------------

def key_centroids(K, labels, n_groups):
    """Key-space centroid of each group (zero rows for empty groups) and sizes."""
    return group_means(K, labels, n_groups)


def query_coordinates(Q, kbar, scale):
    """C[q, g] = tau * q . kbar_g: a query's response to each key-group centroid.

    Reading: the centroid that induces the coordinates is the key-space mean
    of the group; by linearity tau * Q_s kbar_g is also the response-space
    centroid, so this is the same object the key clustering used.
    """
    return F64(scale) * (np.asarray(Q, F64) @ np.asarray(kbar, F64).T)


def dominant_groups(C, sizes):
    """Per query: g1 = argmax over non-empty groups of C (lowest g on ties),
    v = C[q, g1]."""
    C = np.asarray(C)
    masked = np.where(np.asarray(sizes)[None, :] > 0, C, -np.inf)
    g1 = np.argmax(masked, axis=1).astype(np.int64)
    v = C[np.arange(C.shape[0]), g1]
    return g1, v


def query_order(g1, v):
    """Query order pi_Q: sort by (g1 ascending, v descending, token ascending).

    Reading: queries are grouped by their dominant key group, strongest
    response first inside a group, and the order is cut into blocks of B_q.
    """
    n = len(g1)
    return np.lexsort((np.arange(n), -np.asarray(v, F64), np.asarray(g1))).astype(np.int64)


def query_blocks(query_perm, q_block):
    """Blocks of the query order: block b = pi_Q[b*B_q : min((b+1)*B_q, N)]."""
    n = len(query_perm)
    return [np.asarray(query_perm[s:min(s + q_block, n)]) for s in range(0, n, q_block)]


def block_scores(C, blocks):
    """sigma[b, g] = mean over the block's queries of C[q, g]."""
    C = np.asarray(C, F64)
    return np.stack([C[b].mean(axis=0) for b in blocks])


def key_budget(n_tokens, density, n_probes):
    """Per-row key budget kappa = floor(rho * N - m).

    Reading: density counts probes ([SK] results paragraph, [AD]); every probe
    row costs N pairs, so the sparse pass gets rho*N - m keys per row.
    """
    return int(math.floor(density * n_tokens - n_probes))


def select_groups(sigma_b, sizes, kappa):
    """Groups routed to one query block, ascending.

    Non-empty groups are ranked by (sigma descending, g ascending) and the
    longest ranked prefix whose total size stays within kappa is taken; if
    even the first group exceeds kappa, that group alone is taken.
    """
    sizes = np.asarray(sizes)
    cand = np.nonzero(sizes > 0)[0]
    sb = np.asarray(sigma_b, F64)[cand]
    ranked = cand[np.lexsort((cand, -sb))]
    total = np.cumsum(sizes[ranked])
    count = max(1, int(np.count_nonzero(total <= kappa)))
    return np.sort(ranked[:count]).astype(np.int64)


def route(sigma, sizes, kappa):
    """CSR block map: block_ptr [nb+1], block_groups [nnz]."""
    sel = [select_groups(s, sizes, kappa) for s in sigma]
    ptr = np.concatenate([[0], np.cumsum([len(s) for s in sel])]).astype(np.int64)
    grp = np.concatenate(sel).astype(np.int64) if sel else np.zeros(0, np.int64)
    return ptr, grp


def block_key_sets(block_ptr, block_groups, key_perm, group_off):
    """K(b): key tokens of every selected group of block b (group order)."""
    out = []
    for b in range(len(block_ptr) - 1):
        gs = block_groups[block_ptr[b]:block_ptr[b + 1]]
        out.append(np.concatenate([key_perm[group_off[g]:group_off[g + 1]] for g in gs]))
    return out


# ---------------------------------------------------------------------------
# Attention: sparse over routed groups, exact on probe rows  ([AD], [SK])
# ---------------------------------------------------------------------------

def softmax_attention(q_rows, K_set, V_set, scale):
    """Softmax attention of query rows over a key set; returns (out, lse) with
    lse = log sum_j exp(tau q.k_j)."""
    q = np.asarray(q_rows, F64)
    logits = F64(scale) * (q @ np.asarray(K_set, F64).T)
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    s = e.sum(axis=1, keepdims=True)
    out = (e @ np.asarray(V_set, F64)) / s
    return out, (mx + np.log(s))[:, 0]


def sparse_attention(Q, K, V, scale, blocks, key_sets):
    """Block-sparse attention: each query of block b attends, with the softmax
    renormalised over K(b) only, to the keys of its block's selected groups.
    Returns (S, lse) in token order."""
    n, d = np.shape(Q)
    S = np.zeros((n, d), F64)
    lse = np.zeros(n, F64)
    for qb, kb in zip(blocks, key_sets):
        S[qb], lse[qb] = softmax_attention(np.asarray(Q)[qb], np.asarray(K)[kb],
                                           np.asarray(V)[kb], scale)
    return S, lse


def dense_attention(Q, K, V, scale, rows=None):
    """Exact softmax attention over all keys for the given query rows."""
    Q = np.asarray(Q)
    q = Q if rows is None else Q[np.asarray(rows)]
    return softmax_attention(q, K, V, scale)


def probe_positions(n_tokens, n_probes):
    """Probe positions in query order: floor((i + 1/2) * N / m), i < m.

    Reading: the pages say only "a small set of exact query rows per head";
    they are spread evenly over the query order so every routing region is
    sampled.
    """
    i = np.arange(n_probes, dtype=np.int64)
    return ((2 * i + 1) * n_tokens) // (2 * n_probes) if n_probes > 0 else np.zeros(0, np.int64)


def executed_pairs(blocks, key_sets, n_probes, n_tokens):
    """E = sum_b n_b |K(b)| + m N: every probe row is charged a full row."""
    return int(sum(len(b) * len(k) for b, k in zip(blocks, key_sets)) + n_probes * n_tokens)


# ---------------------------------------------------------------------------
# Probe-fitted residual reconstruction  ([AD], [SK] two components, [PC])
# ---------------------------------------------------------------------------

def probe_weights(O_probe):
    """w_p proportional to 1/||o_p||^2, normalised to sum 1 (0 where o_p = 0).

    Reading: the ridge regression is "weighted" and the reported metric is the
    relative error per query, so each probe is weighted by its inverse squared
    dense norm; the fit then minimises the mean squared relative error.
    """
    n2 = (np.asarray(O_probe, F64) ** 2).sum(axis=1)
    w = np.zeros_like(n2)
    nz = n2 > 0
    w[nz] = 1.0 / n2[nz]
    tot = w.sum()
    return w / tot if tot > 0 else w


def residual_subspace(R_probe, w, rank):
    """Top eigenvectors of the weighted uncentred residual scatter
    Sigma = sum_p w_p r_p r_p^T. Returns (U [d, k_eff], eigenvalues
    descending [d]). k_eff = min(k, m, d), or 0 when trace(Sigma) = 0.

    Reading: "the output subspace observed in the probe residuals" is the
    span of the leading principal directions of the residuals, weighted as the
    ridge fit is.
    """
    R_probe = np.asarray(R_probe, F64)
    m, d = R_probe.shape
    Sig = (R_probe * np.asarray(w, F64)[:, None]).T @ R_probe
    evals, evecs = np.linalg.eigh(Sig)
    evals, evecs = evals[::-1], evecs[:, ::-1]
    k_eff = min(rank, m, d) if np.trace(Sig) > 0 else 0
    return evecs[:, :k_eff].copy(), evals


def map_inputs(S_rows, U):
    """Inputs of the fitted map: each sparse output's coordinates in the
    residual subspace, z = U^T s.

    Reading: the pages describe the correction as a small linear map from the
    sparse output that reaches the residual subspace ([SK], paragraph on
    partition geometry) and as an affine correction from the sparse output
    within the output subspace seen in the probe residuals ([PC]). The map
    therefore reads s through the same k_eff directions it writes: it has
    k_eff + 1 inputs (with the bias), not d + 1.
    """
    return np.asarray(S_rows, F64) @ np.asarray(U, F64)


def ridge_penalty(Z, w, lam):
    """Penalty on the slopes: lam times the mean, over the k input
    coordinates, of their weighted variance about their weighted mean.

    Reading: the pages say only "weighted ridge regression" ([AD]). The
    penalty is taken relative to the spread of the map's inputs, so that
    scaling V (hence s, o and r) by c scales the correction by c and the same
    lam means the same amount of shrinkage on every head.
    """
    Z = np.asarray(Z, F64)
    w = np.asarray(w, F64)
    k = Z.shape[1]
    tw = w.sum()
    if k == 0 or tw <= 0:
        return 0.0
    zbar = (w[:, None] * Z).sum(axis=0) / tw
    var = (w[:, None] * (Z - zbar) ** 2).sum(axis=0) / tw
    var[np.all(Z == Z[:1], axis=0)] = 0.0     # a constant input has no spread
    return float(lam * var.mean())


def ridge_fit(Z, Y, w, lam):
    """Weighted ridge regression of Y on [z, 1] with an unpenalised bias.

    Solves (X^T W X + lam_eff I~) Theta = X^T W Y with X = [Z, 1],
    W = diag(w), I~ = diag(1, ..., 1, 0) and lam_eff = ridge_penalty(Z, w,
    lam). Returns Theta [k+1, q]: rows 0..k-1 are the slopes, row k the bias.
    When lam > 0 but the inputs do not vary, the slopes are 0 (any positive
    penalty forces them there) and the bias is the weighted mean of Y.
    """
    Z = np.asarray(Z, F64)
    Y = np.asarray(Y, F64)
    w = np.asarray(w, F64)
    m, k = Z.shape
    X = np.hstack([Z, np.ones((m, 1))])
    A = X.T @ (w[:, None] * X)
    B = X.T @ (w[:, None] * Y)
    lam_eff = ridge_penalty(Z, w, lam)
    if lam > 0 and lam_eff == 0.0:
        Th = np.zeros((k + 1, Y.shape[1]))
        Th[k] = B[k] / A[k, k]
        return Th
    A[np.arange(k), np.arange(k)] += lam_eff
    return np.linalg.solve(A, B)


def normal_equation_residual(Z, Y, w, lam, Theta):
    """||(X^T W X + lam_eff I~) Theta - X^T W Y|| / ||X^T W Y||, X = [Z, 1]."""
    Z = np.asarray(Z, F64)
    m, k = Z.shape
    X = np.hstack([Z, np.ones((m, 1))])
    W = np.asarray(w, F64)[:, None]
    A = X.T @ (W * X)
    A[np.arange(k), np.arange(k)] += ridge_penalty(Z, w, lam)
    B = X.T @ (W * np.asarray(Y, F64))
    nb = np.linalg.norm(B)
    return float(np.linalg.norm(A @ Theta - B) / nb) if nb > 0 else float(np.linalg.norm(A @ Theta))


def lift_map(U, Theta_z):
    """The fitted map written on [s; 1]: Theta = [U Theta_z[:k]; Theta_z[k]]
    ([d+1, k]), so that Theta^T [s; 1] = Theta_z^T [U^T s; 1]."""
    U = np.asarray(U, F64)
    Theta_z = np.asarray(Theta_z, F64)
    k = U.shape[1]
    return np.vstack([U @ Theta_z[:k], Theta_z[k:k + 1]])


def fit_probe_map(S_probe, O_probe, rank, lam):
    """The reconstruction fit from the probe rows' sparse and exact outputs:
    weights, residual subspace, then the ridge map on the subspace
    coordinates. Returns (w, U [d, k_eff], eigenvalues, Theta [d+1, k_eff])."""
    S_probe = np.asarray(S_probe, F64)
    O_probe = np.asarray(O_probe, F64)
    m, d = S_probe.shape
    w = probe_weights(O_probe)
    if m == 0:
        return w, np.zeros((d, 0)), np.zeros(d), np.zeros((d + 1, 0))
    Rp = O_probe - S_probe
    U, evals = residual_subspace(Rp, w, rank)
    if U.shape[1] == 0:
        return w, U, evals, np.zeros((d + 1, 0))
    Theta_z = ridge_fit(map_inputs(S_probe, U), Rp @ U, w, lam)
    return w, U, evals, lift_map(U, Theta_z)


def predicted_residual(S_rows, U, Theta):
    """U Theta^T [s; 1] for each row s (Theta on [s; 1], [d+1, k])."""
    S_rows = np.asarray(S_rows, F64)
    if U.shape[1] == 0:
        return np.zeros_like(S_rows)
    Xa = np.hstack([S_rows, np.ones((S_rows.shape[0], 1))])
    return (Xa @ Theta) @ U.T


# ---------------------------------------------------------------------------
# One call, one head
# ---------------------------------------------------------------------------

@dataclass
class HeadResult:
    labels: np.ndarray
    key_perm: np.ndarray
    group_off: np.ndarray
    sizes: np.ndarray
    kbar: np.ndarray
    C: np.ndarray
    g1: np.ndarray
    v: np.ndarray
    query_perm: np.ndarray
    blocks: list
    sigma: np.ndarray
    block_ptr: np.ndarray
    block_groups: np.ndarray
    key_sets: list
    S: np.ndarray            # sparse output, token order
    lse: np.ndarray
    probe_tokens: np.ndarray
    O_probe: np.ndarray
    w: np.ndarray
    U: np.ndarray
    evals: np.ndarray
    Theta: np.ndarray        # fitted map on [s; 1], [d+1, k_eff]
    O: np.ndarray            # final output, token order
    executed_pairs: int
    density: float
    kmeans: Optional[KMeansResult] = None


def sparsepr_head(Q, K, V, scale, *, q_block, n_groups, kmeans_iters, density, n_probes,
                  rank, ridge_lambda, sample_idx=None, init_idx=None, partition_mode=0,
                  rand_key_perm=None, rand_query_perm=None, keep_scores=False, probe_pos=None):
    """The whole operator for one head, in the pages' order ([AD]).

    1. keys: response profiles under the sampled queries, k-means, paired K/V
       groups (random-block variant: a seeded permutation cut into G runs;
       semantic comparator, partition_mode 2: k-means on the raw key rows);
    2. queries: coordinates against the key-group centroids, grouped into
       blocks of B_q (random-block variant: a seeded permutation; semantic
       comparator: k-means on the raw query rows, ordered by cluster);
    3. route each block to its best groups within the key budget;
    4. block-sparse attention; exact attention on the probe rows;
    5. weighted ridge fit of the probe residuals' subspace coordinates on the
       sparse outputs' subspace coordinates (and a bias);
    6. add the predicted residual to unprobed rows; probes keep their exact
       output.

    probe_pos: the probe positions in the query order (strictly increasing,
    in [0, N)); None takes floor((i + 1/2) N / m).
    """
    Q = np.asarray(Q, F64)
    K = np.asarray(K, F64)
    V = np.asarray(V, F64)
    n, d = Q.shape
    km = None
    if partition_mode == 0:
        R = key_responses(Q, K, scale, sample_idx)
        km = kmeans(R, init_idx, kmeans_iters, keep_scores=keep_scores)
        labels = km.labels
    elif partition_mode == 2:
        km = kmeans(K, init_idx, kmeans_iters, keep_scores=keep_scores)
        labels = km.labels
    else:
        labels = random_block_labels(rand_key_perm, n_groups)
    key_perm, group_off, sizes = group_members(labels, n_groups)
    kbar, _ = key_centroids(K, labels, n_groups)
    C = query_coordinates(Q, kbar, scale)
    g1, v = dominant_groups(C, sizes)
    if partition_mode == 0:
        qperm = query_order(g1, v)
    elif partition_mode == 2:
        _, qperm = semantic_order(Q, init_idx, kmeans_iters, n_groups)
    else:
        qperm = np.asarray(rand_query_perm, np.int64)
    blocks = query_blocks(qperm, q_block)
    sigma = block_scores(C, blocks)
    kappa = key_budget(n, density, n_probes)
    if kappa < 1:
        raise ValueError("key budget floor(rho*N - m) must be at least 1")
    bptr, bgrp = route(sigma, sizes, kappa)
    ksets = block_key_sets(bptr, bgrp, key_perm, group_off)
    S, lse = sparse_attention(Q, K, V, scale, blocks, ksets)
    if probe_pos is None:
        ppos = probe_positions(n, n_probes)
    else:
        ppos = np.asarray(probe_pos, np.int64).ravel()
        if ppos.size != n_probes or (ppos.size and (ppos[0] < 0 or ppos[-1] >= n
                                                    or np.any(np.diff(ppos) <= 0))):
            raise ValueError("probe_pos must hold m strictly increasing positions in [0, N)")
    ptok = qperm[ppos]
    if n_probes > 0:
        O_p, _ = dense_attention(Q, K, V, scale, rows=ptok)
    else:
        O_p = np.zeros((0, d), F64)
    w, U, evals, Theta = fit_probe_map(S[ptok], O_p, rank, ridge_lambda)
    O = S + predicted_residual(S, U, Theta)
    O[ptok] = O_p
    E = executed_pairs(blocks, ksets, n_probes, n)
    return HeadResult(labels=labels, key_perm=key_perm, group_off=group_off, sizes=sizes,
                      kbar=kbar, C=C, g1=g1, v=v, query_perm=qperm, blocks=blocks, sigma=sigma,
                      block_ptr=bptr, block_groups=bgrp, key_sets=ksets, S=S, lse=lse,
                      probe_tokens=ptok, O_probe=O_p, w=w, U=U, evals=evals, Theta=Theta, O=O,
                      executed_pairs=E, density=E / float(n) ** 2, kmeans=km)


# ---------------------------------------------------------------------------
# Support and mass diagnostics  ([SK] the two problem paragraphs; [AD] the
# partition decides how far grouped queries' preferred supports overlap)
# ---------------------------------------------------------------------------

def support_threshold(x, mass):
    """For one query's logits x over all keys: the largest logit t whose
    upper set {j : x_j >= t} holds at least `mass` of the softmax, and that
    set. Reading: "the keys a query prefers" is the smallest upper set of its
    logits that holds the target mass; keys tied at the threshold all count.
    Returns (t, boolean mask of the set)."""
    x = np.asarray(x, F64)
    xs = np.sort(x)[::-1]                           # logits, descending
    cum = np.cumsum(np.exp(xs - xs[0]))
    # an upper set {x >= t} ends where a run of equal logits ends
    ends = np.nonzero(np.append(xs[1:] != xs[:-1], True))[0]
    reach = cum[ends] >= mass * cum[-1]
    t = xs[ends[int(np.argmax(reach))]]
    return t, x >= t


def support_stats(Q, K, scale, labels, query_perm, block_ptr, block_groups, q_block, blocks,
                  mass):
    """Per sampled block b and row q (all N keys): full-row lse, the softmax
    mass on the block's routed keys, the size of q's preferred support at the
    target mass and its part on routed keys; per block the pooled support
    (union over the block's rows) and its routed part. Rows past N are
    skipped (NaN / 0)."""
    Q = np.asarray(Q, F64)
    K = np.asarray(K, F64)
    n = Q.shape[0]
    labels = np.asarray(labels)
    nbk = len(blocks)
    out = {"lse": np.full((nbk, q_block), -np.inf), "routed_mass": np.zeros((nbk, q_block)),
           "support": np.zeros((nbk, q_block), np.int64),
           "support_routed": np.zeros((nbk, q_block), np.int64),
           "pooled": np.zeros(nbk, np.int64), "pooled_routed": np.zeros(nbk, np.int64)}
    for i, b in enumerate(blocks):
        groups = np.asarray(block_groups[block_ptr[b]:block_ptr[b + 1]], np.int64)
        sel = np.isin(labels, groups)                # key j routed to block b
        union = np.zeros(n, bool)
        for r in range(q_block):
            p = b * q_block + r
            if p >= n:
                break
            x = scale * (K @ Q[query_perm[p]])
            mx = x.max()
            z = np.exp(x - mx).sum()
            out["lse"][i, r] = mx + np.log(z)
            out["routed_mass"][i, r] = np.exp(x[sel] - mx).sum() / z
            _, S = support_threshold(x, mass)
            out["support"][i, r] = int(S.sum())
            out["support_routed"][i, r] = int((S & sel).sum())
            union |= S
        out["pooled"][i] = int(union.sum())
        out["pooled_routed"][i] = int((union & sel).sum())
    return out


# ---------------------------------------------------------------------------
# Evaluation  ([AD] error definition; [SK] ablation paragraph for p99)
# ---------------------------------------------------------------------------

def relative_l2_rows(O_rows, O_ref_rows):
    """Per-row relative L2 error ||o - o_ref|| / ||o_ref||."""
    diff = np.linalg.norm(np.asarray(O_rows, F64) - np.asarray(O_ref_rows, F64), axis=1)
    ref = np.linalg.norm(np.asarray(O_ref_rows, F64), axis=1)
    return diff / ref


def error_summary(errors):
    e = np.asarray(errors, F64)
    return {"mean": float(e.mean()), "p99": float(np.percentile(e, 99))}


# ---------------------------------------------------------------------------
# Cross-check forms (exact identities; not used by sparsepr_head)
# ---------------------------------------------------------------------------

def sampled_metric(Q, scale, sample_idx):
    """M = tau^2 Q_s^T Q_s, so that ||r_i - r_j||^2 = (k_i - k_j)^T M (k_i - k_j)."""
    Qs = np.asarray(Q, F64)[np.asarray(sample_idx)]
    return F64(scale) ** 2 * (Qs.T @ Qs)


def kmeans_metric_form(K, M, init_idx, iters):
    """k-means of keys under the metric M, with key-space centroids. Gives the
    same labels as response-space k-means because responses are linear in k."""
    K = np.asarray(K, F64)
    M = np.asarray(M, F64)
    Cb = K[np.asarray(init_idx)].copy()
    G = Cb.shape[0]
    lab = np.zeros(K.shape[0], np.int64)
    for _ in range(iters):
        diff = K[:, None, :] - Cb[None, :, :]
        D = np.einsum("ngi,ij,ngj->ng", diff, M, diff)
        lab = argmin_lowest(D)
        Cb, _ = group_means(K, lab, G, previous=Cb)
    return lab, Cb


def block_scores_mean_query(Q, blocks, kbar, scale):
    """sigma[b, g] = tau * qbar_b . kbar_g with qbar_b the block's mean query."""
    Q = np.asarray(Q, F64)
    qbar = np.stack([Q[b].mean(axis=0) for b in blocks])
    return F64(scale) * (qbar @ np.asarray(kbar, F64).T)
