"""Plain, slow fp64 CPU oracle of the SageSLA attention forward.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this module: only the
tests, the package smoke check and the benchmark's CPU-baseline leg use it. It shares no code, constant or
helper with the HIP library; both sides only consume the same seeded inputs.

What is computed, and where the pages say so
--------------------------------------------
Sources are the TurboDiffusion pages:
  [TD-news]  "Turbo Diffusion：秒级生成与高清保真的视频扩散技术突破" (lanhy.cn/news/1185.html)
             §三(一) SageAttention2++: item 1 outlier smoothing, item 2 independent quantization
             parameters per sub-block, item 3 low-bit attention matmuls;
             §三(二) SLA: item 1 keep the top-k (10%) most important regions, item 2 linear-complexity
             modelling of the rest plus a linear projection, item 3 SageSLA = select first, then INT8
             attention on the selected regions.
  [TD-guide] "TurboDiffusion技术指南：突破视频生成效率瓶颈的实践方案" (blog.gitcode.com), inference flags
             --attention_type sagesla and --sla_topk (fraction of blocks kept).
The pages describe the method only in prose. Every step they leave open is fixed here by the plainest
reading, stated at the function that applies it.

Optionally first, per token over all heads: Q, K <- RMSNorm with a per-channel weight (qk_rmsnorm; [TD-news]
§三(四) item 2, point 1).
Per (batch b, head h), with Q, K, V the [N, D] slices, bq/bk the query/key block sizes:
  1. mu     = fp32(sum_t K[t] / N)                       K-mean over all N tokens (smoothing)
  2. k'     = fp32(K - mu)                               smoothed keys; Q and V are not smoothed
  3. codes  = clamp(rne(fp32(x / s)), -127, 127), s = fp32(absmax_block / 127), per block of Q and of k'
  4. qbar_I = mean of raw Q over block I, kbar_J = mean of k' over block J
     score  = qbar_I . kbar_J / sqrt(D)
  5. crit(I) = the k blocks J with the largest score, ties to the lower J, stored ascending
  6. O_s    = softmax attention of block I's rows over the keys of crit(I), scores from the int codes:
              z = (codeQ . codeK) * s_q(I) * s_k(J) * sm_scale
  7. H_J    = phi(K_J)^T V_J, Z_J = sum phi(K_J) over the keys of block J, phi = elu + 1 on raw Q and K;
     H_m    = sum_J H_J - sum_{J in crit(I)} H_J (likewise Z_m)
     O_l    = phi(q) H_m / (phi(q) . Z_m)
  8. out    = O_s + O_l W_p
Arithmetic is fp64 except at the marked fp32(.) rounding points, which both sides share: each is a single
IEEE operation on fp32/bf16 operands, and computing it in fp64 then rounding to fp32 gives the correctly
rounded fp32 result (53 >= 2*24 + 2; Figueroa, "When is double rounding innocuous?", 1995).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_round", "qk_rmsnorm", "topk_count", "n_blocks", "block_rows", "exact_sum_ok", "k_mean", "smooth", "quantize",
    "pool", "block_scores", "select_topk", "sparse_attention", "phi", "linear_states", "linear_branch",
    "project", "forward_head", "forward",
]

QMAX = 127.0
NEAR_TIE = 1e-6  # a selection row whose k-th / (k+1)-th score gap is below this is a near-tie row


# --------------------------------------------------------------------------------------------------------
# blocks
# --------------------------------------------------------------------------------------------------------
def n_blocks(n: int, blk: int) -> int:
    return -(-n // blk)


def block_rows(n: int, blk: int, i: int) -> slice:
    """Rows of block i. The last block is ragged when blk does not divide n; it holds only valid tokens."""
    return slice(i * blk, min(n, (i + 1) * blk))


def topk_count(frac: float, n_kb: int) -> int:
    """--sla_topk is a fraction of key blocks ([TD-guide] flags; [TD-news] §三(二) item 1 uses 10%).
    Reading: k = round-half-up(frac * n_kb), at least 1; frac >= 1 keeps every block."""
    if frac >= 1.0:
        return n_kb
    return max(1, int(math.floor(frac * n_kb + 0.5)))


# --------------------------------------------------------------------------------------------------------
# 0. RMSNorm of Q and K before the path  ([TD-news] §三(四) item 2, point 1: LayerNorm and RMSNorm operators
#    rewritten for the GPU; §四 step 4: the sampler calls them)
# --------------------------------------------------------------------------------------------------------
def bf16_round(x):
    """Round values that are exact fp32 numbers (held in fp64) to bf16, round-to-nearest-even (finite inputs).

    bf16 keeps the top 16 bits of the fp32 pattern. Adding 0x7FFF plus the lowest kept bit to the pattern and
    clearing the low half rounds to nearest: a dropped half below 0x8000 never carries, one above always does,
    and an exact tie (0x8000) carries only when the kept part is odd, which makes it even."""
    u = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


NORM_AMBIGUOUS = 2.0 ** -48  # relative band around r's fp32 rounding points within which a token is flagged


def _sum_squares(sq):
    """Sum over axis 0 of non-negative fp64 values (exact squares), nearly exactly: a double-double accumulator
    (Knuth's error-free TwoSum, The Art of Computer Programming vol. 2, §4.2.2) whose error stays below
    n^2 2^-106 of the sum, then rounded once to fp64."""
    hi = np.zeros(sq.shape[1:])
    lo = np.zeros(sq.shape[1:])
    for v in sq:
        s = hi + v
        bb = s - hi
        lo += (hi - (s - bb)) + (v - bb)
        hi = s
    return hi + lo


def qk_rmsnorm(X, gamma, eps):
    """RMSNorm of every token over all H*D channels of its heads, with a per-channel weight.

    Reading: the pages name the RMSNorm/LayerNorm operators of the video DiTs they accelerate without their
    formula; those models normalize the projected queries and keys by RMSNorm over the model width (all heads
    of a token) with a learned weight, so: X [H, N, D] (one batch entry), gamma [H*D] (bf16 values), eps.
    Per token: S = the sum of x^2 over the H*D channels, rounded once to fp64 (squares of bf16 values are exact;
    the sum is taken nearly exactly), m = S / (H*D), r = fp32(1 / sqrt(m + eps)) (three fp64 operations, each
    correctly rounded, then fp32); the output is y = bf16(fp32(bf16(fp32(x * r)) * gamma)): the normalized value
    rounded to bf16 before the weight, as the models compute it.
    A token is flagged ambiguous when r's fp32 rounding changes within a relative 2^-48 of its fp64 value: any
    other faithful evaluation of S (within a few fp64 units) may then round r the other way. Returns
    (Y [H, N, D], r [N], ambiguous [N] bool)."""
    X = np.asarray(X, np.float64)
    H, N, D = X.shape
    sq = (X * X).transpose(0, 2, 1).reshape(H * D, N)  # squares of bf16 values: exact in fp64
    S = _sum_squares(sq)
    m = S / float(H * D)
    r64 = 1.0 / np.sqrt(m + float(np.float32(eps)))
    r = r64.astype(np.float32).astype(np.float64)
    amb = (r64 * (1 - NORM_AMBIGUOUS)).astype(np.float32) != (r64 * (1 + NORM_AMBIGUOUS)).astype(np.float32)
    g = np.asarray(gamma, np.float64).reshape(H, 1, D)
    n = bf16_round(X * r[None, :, None])  # the fp32 product rounds exactly like its fp64 value: 8 + 24 bits
    return bf16_round(n * g), r, amb


# --------------------------------------------------------------------------------------------------------
# 1-2. K-mean smoothing  ([TD-news] §三(一) item 1)
# --------------------------------------------------------------------------------------------------------
def exact_sum_ok(x: np.ndarray) -> bool:
    """True when every partial sum of each column of x (finite binary floats) is exact in fp64.

    Every value is an integer multiple of its granularity (the largest power of two dividing it), hence of the
    smallest granularity u in the column; every partial sum is then an integer multiple of u bounded by sum|x|,
    which fp64 holds exactly when sum|x| / u < 2**53."""
    x = np.asarray(x, dtype=np.float64)
    for c in range(x.shape[1]):
        col = x[:, c]
        nz = col[col != 0]
        if nz.size == 0:
            continue
        # granularity of each value: the largest power of two dividing it (x = m * 2^(e-53), m an integer)
        m, e = np.frexp(nz)
        mi = np.abs(m * 2.0 ** 53).astype(np.int64)
        low = (mi & -mi).astype(np.float64)
        u = float(np.min(np.ldexp(low, e - 53)))
        if float(np.sum(np.abs(nz))) / u >= 2.0 ** 53:
            return False
    return True


def k_mean(K: np.ndarray) -> np.ndarray:
    """mu[c] = fp32(S_c / N), S_c = sum over all N tokens of K[t, c].

    Reading of "outlier smoothing ... keeping the overall distribution": subtract from K its mean over all
    tokens of the head, per channel. Adding one vector to every key shifts every logit of a query row by
    the same amount, so the softmax is unchanged (checked by the tests). S_c is exact when exact_sum_ok(K);
    it is then rounded once by the fp64 division and once to fp32."""
    K = np.asarray(K, dtype=np.float64)
    S = K.sum(axis=0)
    return (S / float(K.shape[0])).astype(np.float32).astype(np.float64)


def smooth(K: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """k' = fp32(K - mu): one rounding of the difference to fp32."""
    return (np.asarray(K, np.float64) - np.asarray(mu, np.float64)[None, :]).astype(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------------------------
# 3. per-block INT8 quantization  ([TD-news] §三(一) item 2: independent parameters per sub-block)
# --------------------------------------------------------------------------------------------------------
def quantize(X: np.ndarray, blk: int):
    """Symmetric INT8 codes with one fp32 scale per block of blk rows × all D channels.

    s = fp32(absmax / 127); code = clamp(round-half-even(fp32(x / s)), -127, 127). A block whose absmax is 0
    gets s = 0 and all-zero codes. Returns (codes int8 [N, D], scales float64 holding fp32 values [n_blocks])."""
    X = np.asarray(X, dtype=np.float64)
    n = X.shape[0]
    nb = n_blocks(n, blk)
    codes = np.zeros(X.shape, dtype=np.int8)
    scales = np.zeros(nb, dtype=np.float64)
    for i in range(nb):
        rows = block_rows(n, blk, i)
        xb = X[rows]
        a = float(np.max(np.abs(xb)))
        if a == 0.0:
            continue
        s = float(np.float32(a / QMAX))
        q = (xb / s).astype(np.float32).astype(np.float64)  # the fp32 quotient
        codes[rows] = np.clip(np.rint(q), -QMAX, QMAX).astype(np.int8)  # np.rint rounds half to even
        scales[i] = s
    return codes, scales


# --------------------------------------------------------------------------------------------------------
# 4-5. block scores and top-k selection  ([TD-news] §三(二) item 1; [TD-guide] --sla_topk)
# --------------------------------------------------------------------------------------------------------
def pool(X: np.ndarray, blk: int) -> np.ndarray:
    """Mean of the valid rows of each block (fp64)."""
    X = np.asarray(X, dtype=np.float64)
    n = X.shape[0]
    return np.stack([X[block_rows(n, blk, i)].mean(axis=0) for i in range(n_blocks(n, blk))])


def block_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """score[I, J] = qbar_I . kbar_J / sqrt(D).

    Reading: the importance of key block J for query block I is the scaled dot product of the block-mean
    query and block-mean (smoothed) key. The pages' learned predictor needs trained weights; a softmax over
    J (or any temperature) would not change which blocks rank highest, so selection ranks these logits."""
    D = qbar.shape[1]
    return (np.asarray(qbar, np.float64) @ np.asarray(kbar, np.float64).T) / math.sqrt(D)


def select_topk(scores: np.ndarray, k: int):
    """crit(I) = the k key blocks with the largest score, exact ties to the lower block index, stored in
    ascending index order. Also returns gap[I] = score of the k-th kept block minus the best dropped one
    (inf when nothing is dropped or nothing kept); rows with gap < NEAR_TIE are near-tie rows."""
    n_qb, n_kb = scores.shape
    idx = np.zeros((n_qb, k), dtype=np.int32)
    gap = np.full(n_qb, np.inf)
    J = np.arange(n_kb)
    for I in range(n_qb):
        order = np.lexsort((J, -scores[I]))  # primary: descending score; secondary: ascending J
        idx[I] = np.sort(order[:k])
        if 0 < k < n_kb:
            gap[I] = scores[I, order[k - 1]] - scores[I, order[k]]
    return idx, gap


# --------------------------------------------------------------------------------------------------------
# 6. INT8 block-sparse attention over the selected blocks  ([TD-news] §三(一) item 3, §三(二) item 3)
# --------------------------------------------------------------------------------------------------------
def sparse_attention(q_codes, q_scales, k_codes, k_scales, V, idx, blk_q, blk_k, sm_scale, blocks=None,
                     q_group=None, k_group=None):
    """O_s[i] = sum_j softmax_j(z_ij) v_j over the keys j of the selected blocks of i's query block.

    z_ij = (codeQ_i . codeK_j) * s_q(i) * s_k(j) * sm_scale; the integer dot product is exact in fp64. s_q(i) is
    the scale of the q_group rows that hold row i (default q_group = blk_q: one scale per query block) and s_k(j)
    that of the k_group keys that hold key j (default blk_k). The finer "thread-level" variant ([TD-news]
    §三(一) item 2) uses groups of 32 tokens, so every 32×32 tile of scores has its own pair of scales.
    The softmax is normalised over the selected keys only. A query block with no selected block gets 0.
    blocks: optional list of query blocks to compute (the rows of the others are left 0)."""
    N, D = V.shape
    gq = blk_q if q_group is None else q_group
    gk = blk_k if k_group is None else k_group
    V = np.asarray(V, np.float64)
    out = np.zeros((N, D), dtype=np.float64)
    qc = q_codes.astype(np.float64)
    kc = k_codes.astype(np.float64)
    qs_row = np.repeat(np.asarray(q_scales, np.float64), gq)[:N]  # scale of each row
    ks_row = np.repeat(np.asarray(k_scales, np.float64), gk)[:N]  # scale of each key
    for I in (range(n_blocks(N, blk_q)) if blocks is None else blocks):
        rows = block_rows(N, blk_q, I)
        sel = list(idx[I])
        if not sel:
            continue
        key_rows = np.concatenate([np.arange(N)[block_rows(N, blk_k, J)] for J in sel])
        z = (qc[rows] @ kc[key_rows].T) * qs_row[rows][:, None] * ks_row[key_rows][None, :] * sm_scale
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        out[rows] = (p @ V[key_rows]) / p.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------------------------------------
# 7. linear branch over the remaining blocks  ([TD-news] §三(二) item 2)
# --------------------------------------------------------------------------------------------------------
def phi(x):
    """Feature map elu(x) + 1: x + 1 for x > 0, exp(x) otherwise (always positive)."""
    x = np.asarray(x, np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def linear_states(K, V, blk_k):
    """Per key block J: H_J = phi(K_J)^T V_J (D×D) and Z_J = sum of phi(K_J) rows (D), valid keys only.
    Reading: the linear branch sees the raw bf16 keys (not smoothed, not quantized)."""
    N, D = V.shape
    nkb = n_blocks(N, blk_k)
    PK = phi(K)
    V = np.asarray(V, np.float64)
    H = np.zeros((nkb, D, D))
    Z = np.zeros((nkb, D))
    for J in range(nkb):
        r = block_rows(N, blk_k, J)
        H[J] = PK[r].T @ V[r]
        Z[J] = PK[r].sum(axis=0)
    return H, Z


def linear_branch(Q, H, Z, idx, blk_q, blocks=None):
    """O_l[i] = phi(q_i) H_m / (phi(q_i) . Z_m) with H_m = sum_J H_J - sum_{J in crit(I)} H_J and Z_m alike.

    The total over all blocks is formed once; each query block subtracts its selected blocks' states. The
    subtraction is written as one product of the 0/1 selection matrix with the stacked states. A query block
    whose selection covers every key block has no remaining keys and gets O_l = 0.
    blocks: optional list of query blocks to compute (the rows of the others are left 0)."""
    N, D = Q.shape
    nkb = H.shape[0]
    todo = list(range(n_blocks(N, blk_q)) if blocks is None else blocks)
    PQ = phi(Q)
    Htot = H.sum(axis=0)
    Ztot = Z.sum(axis=0)
    M = np.zeros((len(todo), nkb))
    for r, I in enumerate(todo):
        M[r, idx[I]] = 1.0
    Hcrit = (M @ H.reshape(nkb, D * D)).reshape(len(todo), D, D)
    Zcrit = M @ Z
    out = np.zeros((N, D))
    for r, I in enumerate(todo):
        if len(set(int(j) for j in idx[I])) == nkb:
            continue
        rows = block_rows(N, blk_q, I)
        Hm = Htot - Hcrit[r]
        Zm = Ztot - Zcrit[r]
        out[rows] = (PQ[rows] @ Hm) / (PQ[rows] @ Zm)[:, None]
    return out


def project(O_l, W_p):
    """The linear branch's output projection: row vector times W_p[c, e]."""
    return np.asarray(O_l, np.float64) @ np.asarray(W_p, np.float64)


# --------------------------------------------------------------------------------------------------------
# 8. the whole forward
# --------------------------------------------------------------------------------------------------------
def forward_head(Q, K, V, W_p, blk_q, blk_k, topk, *, linear=True, smooth_k=True, quant=True,
                 sm_scale=None, mask=None, blocks=None, quant_group=None):
    """SageSLA forward for one (b, h) slice. Q, K, V: [N, D] arrays of exact bf16 values; W_p: [D, D].

    Switches for the tests: smooth_k=False skips K-mean smoothing, quant=False attends with the unquantized
    fp32 values, mask (int [n_qb, k] ascending) replaces the selection (used to compare with a GPU's own
    selection), blocks (list of query blocks) limits the attention outputs to those blocks, quant_group (rows
    per INT8 scale, for Q and K alike) replaces the default of one scale per block with finer groups (32 for the
    pages' thread-level granularity). Returns a dict with every intermediate and 'out' (fp64)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    N, D = Q.shape
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    r = {}
    if smooth_k:
        r["exact_sum_ok"] = exact_sum_ok(K)
        r["mu"] = k_mean(K)
    else:
        r["exact_sum_ok"] = True
        r["mu"] = np.zeros(D)
    kp = smooth(K, r["mu"])
    gq = blk_q if quant_group is None else quant_group
    gk = blk_k if quant_group is None else quant_group
    r["q_codes"], r["q_scales"] = quantize(Q, gq)
    r["k_codes"], r["k_scales"] = quantize(kp, gk)
    r["q_pool"] = pool(Q, blk_q)
    r["k_pool"] = pool(kp, blk_k)
    r["scores"] = block_scores(r["q_pool"], r["k_pool"])
    r["idx"], r["gap"] = select_topk(r["scores"], topk)
    idx = r["idx"] if mask is None else np.asarray(mask)
    if quant:
        r["o_s"] = sparse_attention(r["q_codes"], r["q_scales"], r["k_codes"], r["k_scales"], V, idx,
                                    blk_q, blk_k, sm_scale, blocks=blocks, q_group=gq, k_group=gk)
    else:
        ones_q = np.ones(n_blocks(N, blk_q))
        ones_k = np.ones(n_blocks(N, blk_k))
        # quantization off: the "codes" are the fp32 values themselves with unit scales
        r["o_s"] = _sparse_float(Q, kp, V, idx, blk_q, blk_k, sm_scale, ones_q, ones_k)
    if linear:
        H, Z = linear_states(K, V, blk_k)
        r["o_l"] = linear_branch(Q, H, Z, idx, blk_q, blocks=blocks)
        r["o_lin"] = project(r["o_l"], W_p)
    else:
        r["o_l"] = np.zeros((N, D))
        r["o_lin"] = np.zeros((N, D))
    r["out"] = r["o_s"] + r["o_lin"]
    return r


def _sparse_float(Q, Kp, V, idx, blk_q, blk_k, sm_scale, sq, sk):
    N, D = V.shape
    out = np.zeros((N, D))
    for I in range(n_blocks(N, blk_q)):
        rows = block_rows(N, blk_q, I)
        if len(idx[I]) == 0:
            continue
        key_rows = np.concatenate([np.arange(N)[block_rows(N, blk_k, J)] for J in idx[I]])
        z = (Q[rows] @ Kp[key_rows].T) * sm_scale
        z = z - z.max(axis=1, keepdims=True)
        p = np.exp(z)
        out[rows] = (p @ V[key_rows]) / p.sum(axis=1, keepdims=True)
    return out


def forward(q, k, v, w_p, blk_q, blk_k, topk, qk_norm=None, **kw):
    """Batched wrapper: q, k, v [B, H, N, D]; returns a list (over b, h) of forward_head results.

    qk_norm = (gamma_q [H*D], gamma_k [H*D], eps) first normalizes Q and K with qk_rmsnorm per batch entry; the
    whole path then sees the normalized values (each head's result also carries them as 'q_hat', 'k_hat')."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    B, H = q.shape[:2]
    out = []
    for b in range(B):
        qb, kb = q[b], k[b]
        if qk_norm is not None:
            gq, gk, eps = qk_norm
            qb = qk_rmsnorm(qb, gq, eps)[0]
            kb = qk_rmsnorm(kb, gk, eps)[0]
        row = []
        for h in range(H):
            r = forward_head(qb[h], kb[h], v[b, h], w_p, blk_q, blk_k, topk,
                             **{**kw, "mask": (kw.get("mask")[b][h] if kw.get("mask") is not None else None)})
            if qk_norm is not None:
                r["q_hat"], r["k_hat"] = qb[h], kb[h]
            row.append(r)
        out.append(row)
    return out
