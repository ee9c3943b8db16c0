"""Decode attention over a paged FP8 KV cache, written as its plain definition.

Test infrastructure only (see the package docstring).

Definition (page "fp8 paged attention for MoE serving", sections "Smallest
correct example" and "Expected result"): for sequence b with L = seq_lens[b]
valid tokens and query head h, reading KV head h // G (G = H_q / H_kv):

  J      = [max(0, L - W), L) if W > 0 else [0, L)      ("the last W keys")
  s_j    = sm_scale * sum_d q[h, d] * K[j, d]           (sm_scale replaces D**-0.5)
  m      = max(max_j s_j, sigma_h)                      (sigma_h = -inf: no sink)
  o[h]   = sum_j e^(s_j - m) V[j] / (sum_j e^(s_j - m) + e^(sigma_h - m))

where K, V are the exact dequantized values (code x scale) and sigma_h is the
per-head sink logit: one extra term in the denominator with no value.  An empty
J gives o = 0 (reading).  All arithmetic is float64; there is no online
softmax, no splitting and no blocking here.

Split partials (page section "Why it happens": the grid runs over (sequence,
KV head, split)): a split covering J_s gives o_s = sum e^(s_j - m_s) V_j / l_s
and lse_s = m_s + ln l_s, l_s = sum e^(s_j - m_s) (natural log; an empty split
has lse = -inf, o = 0).  The merge, which the pages do not print, is read as the
standard log-sum-exp combination, with the sink entering once:
  M = max(max_s lse_s, sigma);  w_s = e^(lse_s - M)
  o = sum_s w_s o_s / (sum_s w_s + e^(sigma - M))
"""
import math

import numpy as np

from . import fp8 as fp8mod
from . import pool as poolmod


def attended_positions(L: int, window: int) -> np.ndarray:
    """Logical positions the decode token attends: the last ``window`` keys
    (the current token included), or all L when window <= 0."""
    start = max(0, L - window) if window > 0 else 0
    return np.arange(start, L, dtype=np.int64)


def _softmax_out(s, v, sigma):
    """o = sum e^(s-m) v / (sum e^(s-m) + e^(sigma-m)) for scores s [G, n]."""
    G = s.shape[0]
    if s.shape[1] == 0:
        return np.zeros((G, v.shape[1]))
    m = np.maximum(s.max(axis=1), sigma)                        # [G]
    e = np.exp(s - m[:, None])
    z = e.sum(axis=1) + np.exp(sigma - m)
    return (e @ v) / z[:, None]


def fp8_query(q):
    """The query of the fp8 compute mode, as exact float64 values.

    The fp8 path of page "fp8 paged attention for MoE serving" (section "Two
    compute paths") adds one E4M3 rounding of q.  Reading: each (sequence,
    query head) row of q is quantized exactly like one KV block of the page's
    quantizer (section "Supported scope"): one fp32 scale s = fp32(amax / 448)
    (1 for an all-zero row) and codes e4m3(fp32(q / s)) with the correctly
    rounded fp32 quotient; the mode then attends with code x s.  The page does
    not say how q is scaled, and this is the rule it gives for every other
    E4M3 block.  The fp8-mode output is ``decode_ref(fp8_query(q), ...)``."""
    q = np.asarray(q, dtype=np.float64)
    out = np.empty_like(q)
    for idx in np.ndindex(q.shape[:-1]):
        codes, scale = fp8mod.quantize_fp32_block(q[idx])
        out[idx] = fp8mod.dequant(codes, scale)
    return out


def fp8_query_mx(q):
    """The query of the fp8 compute mode over pools with E8M0 (MXFP8) scales,
    as exact float64 values.

    The fp8 path of page "fp8 paged attention for MoE serving" (section "Two
    compute paths") adds one E4M3 rounding of q; with keys in the MXFP8 format
    of page "Attention MXFP8 TKG Kernel API Reference" (E4M3 codes, one E8M0
    scale per 32 elements), the reading taken is that q is rounded to the same
    format: each (sequence, query head) row is cut into 32-element groups along
    D and each group is quantized exactly like a 32-element KV group (the
    smallest power of two s with amax <= 448 s, codes e4m3(q / s)).  The
    fp8-mode output on such pools is ``decode_ref(fp8_query_mx(q), ...)``."""
    q = np.asarray(q, dtype=np.float64)
    codes, u = fp8mod.quantize_e8m0_g32(q)
    scale = np.repeat(fp8mod.E8M0_TABLE[u], 32, axis=-1)
    return fp8mod.dequant(codes, scale)


def decode_ref(q, k_pool, v_pool, kdesc, vdesc, block_table, seq_lens,
               window=0, sinks=None, sm_scale=None, heads=None, seqs=None):
    """float64 [B, H_q, D] attention output (rows not in ``seqs``/``heads`` are 0).

    q: [B, H_q, D] values (bf16-exact); pools: flat uint8; block_table [B, *]
    int; seq_lens [B]; window <= 0 means none; sinks [H_q] or None;
    sm_scale None means D**-0.5.  ``seqs`` and ``heads`` (KV heads) restrict the
    work to a sample."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = kdesc.num_kv_heads
    assert vdesc.num_kv_heads == Hkv and Hq % Hkv == 0
    G = Hq // Hkv
    scale = D ** -0.5 if sm_scale is None else float(sm_scale)
    out = np.zeros((B, Hq, D))
    for b in (range(B) if seqs is None else seqs):
        J = attended_positions(int(seq_lens[b]), int(window))
        for g in (range(Hkv) if heads is None else heads):
            K = poolmod.read_tokens(k_pool, kdesc, block_table[b], J, g)   # [n, D]
            V = poolmod.read_tokens(v_pool, vdesc, block_table[b], J, g)
            qg = q[b, g * G:(g + 1) * G]                                  # [G, D]
            s = scale * (qg @ K.T)                                        # [G, n]
            sig = np.full(G, -np.inf) if sinks is None else np.asarray(sinks, np.float64)[g * G:(g + 1) * G]
            out[b, g * G:(g + 1) * G] = _softmax_out(s, V, sig)
    return out


def partial_ref(q_rows, K, V, sm_scale):
    """Unnormalised-free partial of one split: (o_s [G, D], lse_s [G])."""
    s = sm_scale * (np.asarray(q_rows, np.float64) @ np.asarray(K, np.float64).T)
    G = s.shape[0]
    if s.shape[1] == 0:
        return np.zeros((G, V.shape[1])), np.full(G, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return (e @ V) / l[:, None], m + np.log(l)


def merge_ref(part_o, part_lse, sinks=None):
    """Log-sum-exp merge of split partials.

    part_o [B, H, S, D], part_lse [B, H, S] (natural log, -inf = empty split),
    sinks [H] or None.  Returns float64 [B, H, D]."""
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    B, H, S, D = part_o.shape
    sig = np.full(H, -np.inf) if sinks is None else np.asarray(sinks, np.float64)
    out = np.zeros((B, H, D))
    for b in range(B):
        for h in range(H):
            lse = part_lse[b, h]
            M = max(lse.max() if S else -math.inf, sig[h])
            if M == -math.inf:
                continue                      # nothing attended and no sink: o = 0
            w = np.exp(lse - M)
            den = w.sum() + math.exp(sig[h] - M)
            out[b, h] = (w[:, None] * np.where(w[:, None] > 0, part_o[b, h], 0.0)).sum(axis=0) / den
    return out


def dense_loops_ref(q, K, V, num_kv_heads, sm_scale, window=0, sinks=None):
    """Brute force with Python loops over contiguous per-sequence K/V.

    q [B][Hq][D]; K, V [B][L_b][Hkv][D] nested lists or arrays.  Tiny inputs only."""
    B = len(q)
    out = []
    for b in range(B):
        Hq = len(q[b]); D = len(q[b][0]); L = len(K[b])
        G = Hq // num_kv_heads
        rows = []
        for h in range(Hq):
            start = max(0, L - window) if window > 0 else 0
            scores = []
            for j in range(start, L):
                acc = 0.0
                for d in range(D):
                    acc += q[b][h][d] * K[b][j][h // G][d]
                scores.append(sm_scale * acc)
            sig = -math.inf if sinks is None else float(sinks[h])
            if not scores:
                rows.append([0.0] * D)
                continue
            m = max(max(scores), sig)
            ws = [math.exp(s - m) for s in scores]
            den = sum(ws) + math.exp(sig - m)
            o = []
            for d in range(D):
                num = 0.0
                for i, j in enumerate(range(start, L)):
                    num += ws[i] * V[b][j][h // G][d]
                o.append(num / den)
            rows.append(o)
        out.append(rows)
    return np.array(out, dtype=np.float64)
