"""Rounding bounds for the GPU paths whose arithmetic is coarser than the
forward tolerances allow: the FP8 prefill and the backward pass.

These are test models, not part of the oracle: the oracle computes the exact
values (the plain definitions, in fp64) and nothing else; each bound here
says how far a kernel with the stated arithmetic may lie from those exact
values, element by element.  Both are first-order error bounds (second-order
terms are below 2^-40 of the result and are covered by a factor 1.01), with
every floating-point sum charged one rounding per added term, whatever order
or blocking the hardware uses:

    gamma(n) = n v / (1 - n v),  v = 2^-24 (fp32 unit roundoff),
    u = 2^-8 (bf16 unit roundoff, nearest even).

Inputs are numpy fp64 arrays of the exact input values.
"""
import math

import numpy as np

U_BF16 = 2.0 ** -8
V_FP32 = 2.0 ** -24
E_EXP2 = 2.0 ** -22        # relative error allowed for the hardware exp2 (4 ulp)
LOG2E = 1.4426950408889634
SAFETY = 1.01


def gamma(n):
    """Relative error bound of an fp32 sum of n terms, any order."""
    n = np.asarray(n, dtype=np.float64)
    return n * V_FP32 / (1.0 - n * V_FP32)


# ---------------------------------------------------------------------------
# FP8 prefill: P rounded to e4m3 before P V
# ---------------------------------------------------------------------------
def fp8_output_bound(qs, b_idx, kvh_idx, i_idx, kv, vv, scale, lse, causal, q_offset=0,
                     chunk=256):
    """Per-element bound on |O_kernel - O_exact| for the FP8 prefill.

    Kernel arithmetic: scores from exact e4m3 products accumulated in fp32
    (d_h terms); weights p_j = 2^(c s_j - m) with m a running reference that
    never exceeds the row maximum and trails it by at most 8 (so
    1 <= max_j p_j <= 2^8); p_j rounded to e4m3 (nearest even; relative error
    <= 2^-4 where p_j >= 2^-6, absolute error <= 2^-10 below); P V
    accumulated in fp32 over the visible keys; the row sum from the unrounded
    p_j in fp32; O rounded to bf16 once.  With P_j the exact weights,
    n the visible key count and A_t = sum_j P_j |v_jt|:

      |dO_t| <= 2^-4 A_t + 2^-10 max_j P_j sum_j |v_jt|       (e4m3 weights)
              + 2 gamma(n) (A_t + |O_t|) + rho A_t            (fp32 sums, scores)
              + u |O_t|                                      (bf16 output)

    with rho = ln2 c gamma(d_h) max_j sum_t |q_t k_jt| the weights' relative
    error from the fp32 scores (c = scale log2 e).

    qs: [m, d] the requested query rows' values (decoded, times the descale);
    b_idx, kvh_idx, i_idx: their batch entry, key/value head and position;
    kv, vv: [B, n_kv, Lk, d] decoded keys and values times their descales;
    lse: exact LSE of the requested rows.  Returns [m, d].
    """
    m, d = qs.shape
    Lk = kv.shape[2]
    out = np.empty((m, d))
    c = scale * LOG2E
    b_idx, kvh_idx, i_idx = (np.asarray(x) for x in (b_idx, kvh_idx, i_idx))
    for b, kvh in {(int(x), int(y)) for x, y in zip(b_idx, kvh_idx)}:
        sel = np.nonzero((b_idx == b) & (kvh_idx == kvh))[0]
        absv = np.abs(vv[b, kvh])
        cum_absv = np.cumsum(absv, axis=0)
        for c0 in range(0, sel.size, chunk):
            idx = sel[c0:c0 + chunk]
            q_c = qs[idx]
            nvis = i_idx[idx] + q_offset + 1 if causal else np.full(idx.size, Lk)
            n_keys = int(nvis.max())
            kk = kv[b, kvh, :n_keys]
            s = scale * (kk @ q_c.T)                                # [n, m]
            mask = np.arange(n_keys)[:, None] < nvis[None, :]
            p = np.where(mask, np.exp(s - lse[idx][None, :]), 0.0)
            a_t = p.T @ absv[:n_keys]                               # [m, d]
            o_t = p.T @ vv[b, kvh, :n_keys]
            p_max = p.max(axis=0)
            plain = cum_absv[nvis - 1]                              # sum_j |v_jt|, visible j
            qk_abs = np.abs(kk) @ np.abs(q_c).T
            rho = math.log(2) * c * gamma(d) * np.max(np.where(mask, qk_abs, 0.0), axis=0)
            gn = gamma(nvis)[:, None]
            out[idx] = SAFETY * (2.0 ** -4 * a_t + 2.0 ** -10 * p_max[:, None] * plain
                                 + 2 * gn * (a_t + np.abs(o_t)) + rho[:, None] * a_t
                                 + U_BF16 * np.abs(o_t))
    return out


def fp8_rows_bound(q8, k8, v8, dq, dk, dv, scale, lse, rows, causal, q_offset, table):
    """fp8_output_bound for flat query rows of e4m3 inputs (codes + descales),
    decoding only the rows it needs of Q."""
    B, n_q, Lq, d = q8.shape
    n_kv = k8.shape[1]
    g = n_q // n_kv
    rows = np.asarray(rows, dtype=np.int64)
    b_idx, h_idx, i_idx = rows // (n_q * Lq), (rows // Lq) % n_q, rows % Lq
    qs = table[q8[b_idx, h_idx, i_idx]] * dq
    kv = table[k8] * dk
    vv = table[v8] * dv
    return fp8_output_bound(qs, b_idx, h_idx // g, i_idx, kv, vv, scale, lse, causal, q_offset)


# ---------------------------------------------------------------------------
# backward pass
# ---------------------------------------------------------------------------
def bwd_delta_bound(dov, ov):
    """|D_kernel - D_exact| for D_i = dO_i . O_i taken from O rounded to bf16
    and summed in fp32: (u + gamma(d)) sum_t |dO_it O_it|.  dov, ov: [n, d]."""
    d = dov.shape[-1]
    return SAFETY * (U_BF16 + gamma(d)) * np.sum(np.abs(dov * ov), axis=-1)


class BwdGroup:
    """One key/value group (batch b, kv head kvh) of a backward problem, with
    the exact row statistics of the query rows that the requested gradients
    depend on.

    Kernel arithmetic the bounds model: s = q.k from exact bf16 products
    accumulated in fp32 (d terms); P = 2^(c s - log2e LSE) with c = fp32(scale
    log2e) by one fused multiply-add and the hardware exp2, LSE given in fp32;
    dP = dO.v in fp32; D from the bf16-rounded output in fp32; dS = P (dP - D)
    in fp32; P and dS rounded to bf16 for the products; dQ = scale sum_j dS_ij
    k_j, dK = scale sum_i dS_ij q_i and dV = sum_i P_ij dO_i accumulated in
    fp32 over every term and rounded to bf16 once.  Per visible pair (i, j):

      rho_ij = ln2 |c| gamma(d) sum_t |q_it k_jt|
               + 4 v (|c s_ij| + log2e |LSE_i|) + v |x_ij| + E_EXP2
               (relative error of the fp32 P: scores, the constants, the
                fp32 LSE, the fused multiply-add and the exp2)
      E_ij   = (u + rho_ij + 2v) |dS_ij|
               + P_ij (gamma(d) sum_t |dO_it v_jt| + eD_i)
               (error of the bf16 dS; eD_i the delta bound above)
      |dQ_it err| <= |scale| (sum_j E_ij |k_jt| + gamma(n_i) sum_j (|dS_ij| + E_ij) |k_jt|)
                     + (u + v) |dQ_it|,        n_i = keys query i sees
      |dK_jt err| <= |scale| (sum_i E_ij |q_it| + gamma(m_j) sum_i (|dS_ij| + E_ij) |q_it|)
                     + (u + v) |dK_jt|,        m_j = g x queries that see key j
      |dV_jt err| <= sum_i (u + rho_ij) P_ij |dO_it|
                     + gamma(m_j) sum_i (1 + u + rho_ij) P_ij |dO_it| + u |dV_jt|

    qv, dov: [g, L, d] (the group's query heads); kv, vv: [L, d];
    lse, delta, ov: exact statistics and outputs of the group's query rows,
    [g, L] / [g, L, d], where rows the requested gradients do not depend on
    may hold anything finite (they are never read)."""

    def __init__(self, qv, kv, vv, dov, ov, lse, delta, scale, causal):
        self.q, self.k, self.v, self.do = qv, kv, vv, dov
        self.o, self.lse, self.delta = ov, lse, delta
        self.scale, self.causal = float(scale), bool(causal)
        self.g, self.L, self.d = qv.shape
        self.c = float(np.float32(scale * LOG2E))

    def _pair_terms(self, qs, dos, lse, delta, ob, kk, vv, mask):
        """Query rows (qs, dos, ob: [m, d]; lse, delta: [m]) against key rows
        (kk, vv: [n, d]) where mask [m, n] marks the visible pairs: P, dS, rho
        and E, each [m, n], zero at masked pairs."""
        d = self.d
        s = qs @ kk.T
        p = np.where(mask, np.exp(self.scale * s - lse[:, None]), 0.0)
        ds = p * ((dos @ vv.T) - delta[:, None])
        x = self.c * s - LOG2E * lse[:, None]
        rho = (math.log(2) * abs(self.c) * gamma(d) * (np.abs(qs) @ np.abs(kk).T)
               + 4 * V_FP32 * (np.abs(self.c * s) + LOG2E * np.abs(lse)[:, None])
               + V_FP32 * np.abs(x) + E_EXP2)
        rho = np.where(mask, rho, 0.0)
        e_d = bwd_delta_bound(dos, ob)
        e = ((U_BF16 + rho + 2 * V_FP32) * np.abs(ds)
             + p * (gamma(d) * (np.abs(dos) @ np.abs(vv).T) + e_d[:, None]))
        return p, ds, rho, e

    def dq_bound(self, heads, idx, dq_exact, chunk=64):
        """Bounds for dQ rows (heads[r], idx[r]); dq_exact: [m, d]."""
        heads = np.asarray(heads)
        idx = np.asarray(idx)
        out = np.empty((len(idx), self.d))
        for h in np.unique(heads):
            sel = np.nonzero(heads == h)[0]
            for c0 in range(0, sel.size, chunk):
                rr = sel[c0:c0 + chunk]
                ii = idx[rr]
                n = int(ii.max()) + 1 if self.causal else self.L
                keys = np.arange(n)
                mask = (keys[None, :] <= ii[:, None]) if self.causal else np.ones((rr.size, n), bool)
                p, ds, rho, e = self._pair_terms(self.q[h, ii], self.do[h, ii], self.lse[h, ii],
                                                 self.delta[h, ii], self.o[h, ii], self.k[:n],
                                                 self.v[:n], mask)
                absk = np.abs(self.k[:n])
                nvis = ii + 1 if self.causal else np.full(rr.size, self.L)
                acc = (e @ absk) + gamma(nvis)[:, None] * ((np.abs(ds) + e) @ absk)
                out[rr] = SAFETY * (abs(self.scale) * acc
                                    + (U_BF16 + V_FP32) * np.abs(dq_exact[rr]))
        return out

    def dkdv_bound(self, keys_req, dk_exact, dv_exact, chunk=4096):
        """Bounds for dK and dV rows keys_req; dk_exact, dv_exact: [m, d]."""
        keys_req = np.asarray(keys_req)
        m, d = len(keys_req), self.d
        acc_k = np.zeros((m, d))
        acc_kg = np.zeros((m, d))
        acc_v = np.zeros((m, d))
        acc_vg = np.zeros((m, d))
        kk, vv = self.k[keys_req], self.v[keys_req]
        i_start = int(keys_req.min()) if self.causal else 0
        for h in range(self.g):
            for c0 in range(i_start, self.L, chunk):
                ii = np.arange(c0, min(self.L, c0 + chunk))
                mask = (ii[:, None] >= keys_req[None, :]) if self.causal else np.ones((ii.size, m), bool)
                p, ds, rho, e = self._pair_terms(self.q[h, ii], self.do[h, ii], self.lse[h, ii],
                                                 self.delta[h, ii], self.o[h, ii], kk, vv, mask)
                aq = np.abs(self.q[h, ii])
                ado = np.abs(self.do[h, ii])
                acc_k += e.T @ aq
                acc_kg += (np.abs(ds) + e).T @ aq
                acc_v += ((U_BF16 + rho) * p).T @ ado
                acc_vg += ((1 + U_BF16 + rho) * p).T @ ado
        n_rows = self.g * (self.L - keys_req) if self.causal else np.full(m, self.g * self.L)
        gm = gamma(n_rows)[:, None]
        bk = SAFETY * (abs(self.scale) * (acc_k + gm * acc_kg)
                       + (U_BF16 + V_FP32) * np.abs(dk_exact))
        bv = SAFETY * (acc_v + gm * acc_vg + U_BF16 * np.abs(dv_exact))
        return bk, bv
