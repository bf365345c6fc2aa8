"""Error bounds for fa_bwd's gradients, derived from the points where its arithmetic rounds.

Test infrastructure: the GPU backward tests compare the kernels' gradients with the fp64
oracle's, and on inputs far from N(0,1) no single relative tolerance fits, because the
backward subtracts nearly equal numbers: dS = P * (dP - D) with D_i = dO_i . O_i, and for a
row whose softmax is close to one-hot, dP_ij and D_i agree to many digits.  What the kernels
round, and so what can move a gradient:

* the forward output O, stored in the input type u (unit roundoff 2^-11 for fp16, 2^-8 for
  bf16) after P was rounded for the P V product:
  |O_stored - O| <= u (|O| + P |V|)  (elementwise, to first order);
* D taken from that stored O:  |dD_i| <= sum_d |dO_id| |O_stored - O|_id;
* dS rounded to the input type before the dS K and dS^T Q products, and P before P^T dO:
  |d(dS_ij)| <= u |dS_ij| + eta + P_ij |dD_i|,  |d(P_ij)| <= u P_ij + eta,
  eta covering values that underflow: half fp16's smallest subnormal step, and for bf16,
  whose range is fp32's, fp32's smallest normal value (the kernels' fp32 arithmetic, the
  exp2 instruction and the MFMAs, may flush fp32 subnormals to zero);
* the gradients themselves rounded to the input type: u |g|.

Carried through the products, with absolute values (so no cancellation is assumed):

  |d dQ_i| <= scale sum_j |d(dS_ij)| |K_j|  + u |dQ_i|
  |d dK_j| <= scale sum_i |d(dS_ij)| |Q_i|  + u |dK_j|   (over the group's query heads)
  |d dV_j| <=       sum_i |d(P_ij)| |dO_i|  + u |dV_j|

``rounding_bound`` evaluates these from the oracle's fp64 P, dP and dS, times a safety
factor of 2 for the second-order and fp32-accumulation terms it leaves out.
``rounding_model`` is a CPU model of the same rounding steps, used to check that the bound
holds for them with room to spare and to give a measured (tighter) per-tensor bound.
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import attention as oa

UNIT_ROUNDOFF = {torch.float16: 2.0 ** -11, torch.bfloat16: 2.0 ** -8}
UNDERFLOW = {torch.float16: 2.0 ** -25, torch.bfloat16: 2.0 ** -126}


def rounding_bound(q, k, v, do, scale, causal, input_pos=0, window=0, safety=2.0):
    """Elementwise bounds (bq, bk, bv) on |g - g_exact| for fa_bwd's dQ, dK and dV, float64
    arrays of q's and k's shapes.  q, k, v, do: CPU tensors of the input type."""
    dtype = q.dtype
    u, eta = UNIT_ROUNDOFF[dtype], UNDERFLOW[dtype]
    q, k, v, do = (t.double().numpy() for t in (q, k, v, do))
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    bq, bk, bv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    gq, gk, gv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    vis = oa.key_visibility(np.arange(Sq), Skv, causal, input_pos, window)
    rows = np.nonzero(vis.any(axis=1))[0]
    for b in range(B):
        for hq in range(Hq):
            g = oa.kv_head_of(hq, Hq, Hkv)
            kh, vh = k[b, g], v[b, g]
            qr, dor = q[b, hq, rows], do[b, hq, rows]
            m, e, l = oa.masked_softmax_stats(oa.scaled_scores(qr, kh, scale), vis[rows])
            P = e / l
            O = P @ vh
            e_o = u * (np.abs(O) + P @ np.abs(vh)) + eta * np.abs(vh).sum(axis=0)
            dP = dor @ vh.T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            e_d = (np.abs(dor) * e_o).sum(axis=1, keepdims=True)
            e_ds = u * np.abs(dS) + eta + P * e_d
            bq[b, hq, rows] = scale * (e_ds @ np.abs(kh))
            gq[b, hq, rows] = scale * (dS @ kh)
            bk[b, g] += scale * (e_ds.T @ np.abs(qr))
            gk[b, g] += scale * (dS.T @ qr)
            bv[b, g] += (u * P + eta).T @ np.abs(dor)
            gv[b, g] += P.T @ dor
    return tuple(safety * (bb + u * np.abs(gg)) for bb, gg in ((bq, gq), (bk, gk), (bv, gv)))


def rounding_model(q, k, v, do, scale, causal, input_pos=0, window=0, mistake=None):
    """fa_bwd's rounding steps on the CPU: fp32 scores from the rounded inputs, P from an
    accurate LSE, the forward's O as fl(fl(P) V), D = rowsum(dO * O), dS = P (dP - D) in
    fp32, P and dS rounded to the input type before their products, fp32 sums, gradients
    rounded.  Returns (dq, dk, dv) in the input type.  ``mistake`` plants one error (for
    the tests that show the bound catches it): "no_d" (D dropped), "d_sign" (dP + D),
    "dk_no_scale" (dK without the softmax scale), "dq_keys_shifted" (dQ from the next key's
    row of K), "dv_from_ds" (dV from dS instead of P)."""
    dt = q.dtype
    qf, kf, vf, dof = (t.float() for t in (q, k, v, do))
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kf, vf = kf.repeat_interleave(G, 1), vf.repeat_interleave(G, 1)
    vis = torch.from_numpy(oa.key_visibility(np.arange(Sq), Skv, causal, input_pos, window))
    s = torch.matmul(qf, kf.transpose(-1, -2).contiguous()) * scale
    s = s.masked_fill(~vis, -float("inf"))
    lse = torch.logsumexp(s.double(), -1).float()
    p = torch.exp(s - lse[..., None]).nan_to_num(0.0)
    o = torch.matmul(p.to(dt).float(), vf).to(dt).float()
    d = (dof * o).sum(-1, keepdim=True)
    if mistake == "no_d":
        d = torch.zeros_like(d)
    dp = torch.matmul(dof, vf.transpose(-1, -2).contiguous())
    ds = p * (dp + d) if mistake == "d_sign" else p * (dp - d)
    pb, dsb = p.to(dt).float(), ds.to(dt).float()
    dv = torch.matmul((dsb if mistake == "dv_from_ds" else pb).transpose(-1, -2).contiguous(), dof)
    kq = torch.roll(kf, -1, dims=2) if mistake == "dq_keys_shifted" else kf
    dq = scale * torch.matmul(dsb, kq)
    dk = torch.matmul(dsb.transpose(-1, -2).contiguous(), qf)
    if mistake != "dk_no_scale":
        dk = scale * dk
    dk = dk.reshape(B, Hkv, G, Skv, D).sum(2)
    dv = dv.reshape(B, Hkv, G, Skv, D).sum(2)
    return dq.to(dt), dk.to(dt), dv.to(dt)


def check_within(got, ref, bounds, model=None, factor=3.0, floor=0.0):
    """Worst ratio |got - ref| / bound per gradient, and (when ``model`` is given) the
    per-tensor max error against ``factor`` x the model's max error + ``floor``.  Returns a
    list of (name, err_max, worst_ratio, measured_limit or None)."""
    out = []
    for i, (name, g, r, bd) in enumerate(zip(("dq", "dk", "dv"), got, ref, bounds)):
        err = np.abs(g.double().numpy() - r) if isinstance(g, torch.Tensor) else np.abs(g - r)
        ratio = float(np.max(err / bd)) if err.size else 0.0
        lim = None
        if model is not None:
            m_err = np.abs(model[i].double().numpy() - r)
            lim = factor * (float(m_err.max()) if m_err.size else 0.0) + floor
        out.append((name, float(err.max()) if err.size else 0.0, ratio, lim))
    return out
