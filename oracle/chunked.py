"""Float64 chunked (UT/WY) form of the gated delta rule, forward and backward.

TEST INFRASTRUCTURE ONLY.  An independent numpy rendering of the exact
chunk-wise re-association of the recurrence.  The tests compare it with the
token-by-token oracle (``gdr_oracle.c``): two different algorithms that must
agree to rounding, which pins both.  It also yields per-chunk intermediates
(A, W, U, chunk-boundary states) for stage-wise checks.

Per chunk of c rows with start state S (Dv x Dk), all float64:
  Gam_r = sum_{s<=r} lam_s (in-chunk cumsum), GamC = Gam of the last row,
  E_rs  = exp(Gam_r - Gam_s) for r >= s (a pairwise difference, always <= 1),
  M_rs  = sum_j kn_r kn_s E_rs   (r > s),   P_rs = scale sum_j qn_r kn_s E_rs (r >= s),
  A     = (I + StrictLower(diag(beta) M))^-1   -- the in-chunk UT/WY inverse,
  Kbar  = kn e^Gam,  Khat = kn e^(GamC - Gam),  Qbar = scale qn e^Gam,
  W = A diag(beta) Kbar,  U' = A diag(beta) V,  U = U' - W S^T,
  O = Qbar S^T + P U,  S_next = S Diag(e^GamC) + U^T Khat.
The backward runs the chunk recursion last to first:
  dU = P^T dO + Khat dS_next^T,  dS = dS_next Diag(e^GamC) + dO^T Qbar - dU^T W,
and the chunk-local gradients listed in :func:`_chunk_backward`.  The reverse
cumsum that maps dGam back to the per-token log decay is
:func:`reverse_cumsum_with_total`; the FlashKDA backward page works the same
suffix-sum example (§5.0 (e)).
"""

from __future__ import annotations

from typing import Dict

import numpy as np


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def reverse_cumsum_with_total(dgam: np.ndarray, dgam_total) -> np.ndarray:
    """Gradient of the in-chunk prefix sum: dlam_s = sum_{r >= s} dGam_r + dGamC.

    The prefix sum's adjoint is the suffix sum (FlashKDA backward page, §5.0);
    the chunk total Gam_C = sum_s lam_s adds its gradient to every row (§5.1).
    Works along axis 0.
    """
    suffix = np.flip(np.cumsum(np.flip(dgam, axis=0), axis=0), axis=0)
    return suffix + dgam_total


def _prep(inp, n, h):
    cu = np.asarray(inp["cu_seqlens"], dtype=np.int64)
    t0, t1 = int(cu[n]), int(cu[n + 1])
    H, K = int(inp["H"]), int(inp["K"])
    Hk = int(inp.get("Hk", H))   # grouped heads: value head h reads key head h // (H / Hk)

    def tok(name, heads=H, head=h):
        x = _f64(inp[name])
        return x.reshape((-1, heads) + x.shape[3:])[t0:t1, head]

    q, k = tok("q", Hk, h // (H // Hk)), tok("k", Hk, h // (H // Hk))
    v, dO, b, g = (tok(s) for s in ("v", "dO", "b", "g"))
    rq = 1.0 / np.sqrt((q * q).sum(-1) + 1e-6)
    rk = 1.0 / np.sqrt((k * k).sum(-1) + 1e-6)
    qn, kn = q * rq[:, None], k * rk[:, None]
    beta = _sigmoid(b)
    if int(inp["gate"]) == 0:
        lam = np.repeat(g[:, None], K, axis=1)
        x = None
        ea = None
    else:
        A_log, dtb = _f64(inp["A_log"]), _f64(inp["dt_bias"])
        ea = np.exp(A_log[h])
        x = g + dtb[h][None, :]
        if int(inp["gate"]) == 1:
            lam = -ea * _softplus(x)
        else:   # bounded sigmoid form (FlashKDA K1 page, section 5.2), natural log
            lam = float(inp["gate_scale"]) * _sigmoid(ea * x)
    return dict(t0=t0, t1=t1, q=q, k=k, v=v, dO=dO, qn=qn, kn=kn, rq=rq, rk=rk, beta=beta,
                lam=lam, x=x, ea=ea)


def _chunk_quantities(qn, kn, beta, lam, v, scale):
    c = qn.shape[0]
    gam = np.cumsum(lam, axis=0)
    gamC = gam[-1]
    diff = gam[:, None, :] - gam[None, :, :]            # [r, s, j]
    low = np.tril(np.ones((c, c), dtype=bool))          # r >= s
    E = np.where(low[:, :, None], np.exp(np.where(low[:, :, None], diff, 0.0)), 0.0)
    M = np.einsum("rj,sj,rsj->rs", kn, kn, E) * np.tril(np.ones((c, c)), -1)
    P = scale * np.einsum("rj,sj,rsj->rs", qn, kn, E)
    L = np.tril(beta[:, None] * M, -1)
    A = np.linalg.inv(np.eye(c) + L)
    Kbar = kn * np.exp(gam)
    Khat = kn * np.exp(gamC[None, :] - gam)
    Qbar = scale * qn * np.exp(gam)
    W = A @ (beta[:, None] * Kbar)
    Up = A @ (beta[:, None] * v)
    return dict(gam=gam, gamC=gamC, E=E, M=M, P=P, A=A, Kbar=Kbar, Khat=Khat, Qbar=Qbar, W=W, Up=Up)


def _chunk_backward(z, S, dS_next, U, dO, v, qn, kn, beta, scale):
    """Chunk-local gradients given the chunk's start state S and dS_next."""
    A, M, P, E, W = z["A"], z["M"], z["P"], z["E"], z["W"]
    Kbar, Khat, Qbar, gamC = z["Kbar"], z["Khat"], z["Qbar"], z["gamC"]
    c = qn.shape[0]
    dU = P.T @ dO + Khat @ dS_next.T
    dS = dS_next * np.exp(gamC)[None, :] + dO.T @ Qbar - dU.T @ W
    dP = np.tril(dO @ U.T)
    dQbar = dO @ S
    dKhat = U @ dS_next
    dY = A.T @ dU
    dv = beta[:, None] * dY
    X = v - Kbar @ S.T
    dbeta = (dY * X).sum(1)
    dL = -np.tril(dY @ U.T, -1)
    dbeta += (dL * M).sum(1)
    dM = beta[:, None] * dL
    dKbar = -(beta[:, None] * dY) @ S
    # pairwise terms through M and P, only bounded E entries are formed
    dkn = np.einsum("rs,sj,rsj->rj", dM, kn, E) + np.einsum("rs,rj,rsj->sj", dM, kn, E) \
        + scale * np.einsum("rs,rj,rsj->sj", dP, qn, E)
    dqn = scale * np.einsum("rs,sj,rsj->rj", dP, kn, E)
    T1 = np.einsum("rs,rj,sj,rsj->rsj", dM, kn, kn, E) + scale * np.einsum("rs,rj,sj,rsj->rsj", dP, qn, kn, E)
    dgam = T1.sum(1) - T1.sum(0)
    # terms through Kbar, Khat, Qbar
    dkn += dKbar * np.exp(z["gam"]) + dKhat * np.exp(gamC[None, :] - z["gam"])
    dqn += scale * dQbar * np.exp(z["gam"])
    dgam += dKbar * Kbar - dKhat * Khat + dQbar * Qbar
    dgamC = (dKhat * Khat).sum(0) + (dS_next * S).sum(0) * np.exp(gamC)
    del c
    return dict(dU=dU, dS=dS, dv=dv, dbeta=dbeta, dkn=dkn, dqn=dqn, dgam=dgam, dgamC=dgamC)


def run(inp: Dict, chunk: int = 64, dht="input") -> Dict[str, np.ndarray]:
    """Chunked forward + backward for every (sequence, head); float64 numpy."""
    B, T, H, K, V, N = (int(inp[s]) for s in ("B", "T", "H", "K", "V", "N"))
    gate, scale = int(inp["gate"]), float(inp["scale"])
    cu = np.asarray(inp["cu_seqlens"], dtype=np.int64)
    TT = B * T
    h0 = _f64(inp.get("h0"))
    dhtv = _f64(inp.get("dht") if isinstance(dht, str) else dht)
    gK = (K,) if gate >= 1 else ()
    Hk = int(inp.get("Hk", H))
    G = H // Hk
    o = np.zeros((TT, H, V)); dq = np.zeros((TT, Hk, K)); dk = np.zeros((TT, Hk, K))
    dv = np.zeros((TT, H, V)); dg = np.zeros((TT, H) + gK); db = np.zeros((TT, H))
    ht = np.zeros((N, H, V, K)); dh0 = np.zeros((N, H, V, K))
    dA = np.zeros(H); ddt = np.zeros((H, K))
    S_chunk, dS_chunk, A_chunk, U_all = [], [], [], np.zeros((TT, H, V))
    for h in range(H):
        S_h, dS_h, A_h = [], [], []
        for n in range(N):
            p = _prep(inp, n, h)
            t0, t1 = p["t0"], p["t1"]
            L = t1 - t0
            S = np.zeros((V, K)) if h0 is None else h0[n, h].copy()
            zs, Ss, Us, spans = [], [], [], []
            for cs in range(0, L, chunk):
                ce = min(L, cs + chunk)
                z = _chunk_quantities(p["qn"][cs:ce], p["kn"][cs:ce], p["beta"][cs:ce], p["lam"][cs:ce],
                                      p["v"][cs:ce], scale)
                U = z["Up"] - z["W"] @ S.T
                o[t0 + cs:t0 + ce, h] = z["Qbar"] @ S.T + z["P"] @ U
                U_all[t0 + cs:t0 + ce, h] = U
                zs.append(z); Ss.append(S); Us.append(U); spans.append((cs, ce))
                S = S * np.exp(z["gamC"])[None, :] + U.T @ z["Khat"]
            ht[n, h] = S
            dS = np.zeros((V, K)) if dhtv is None else dhtv[n, h].copy()
            dqn = np.zeros((L, K)); dkn = np.zeros((L, K)); dbeta = np.zeros(L); dlam = np.zeros((L, K))
            dSs = [None] * len(zs)
            for ci in range(len(zs) - 1, -1, -1):
                cs, ce = spans[ci]
                dSs[ci] = dS
                r = _chunk_backward(zs[ci], Ss[ci], dS, Us[ci], p["dO"][cs:ce], p["v"][cs:ce],
                                    p["qn"][cs:ce], p["kn"][cs:ce], p["beta"][cs:ce], scale)
                dS = r["dS"]
                dv[t0 + cs:t0 + ce, h] = r["dv"]
                dqn[cs:ce], dkn[cs:ce], dbeta[cs:ce] = r["dqn"], r["dkn"], r["dbeta"]
                dlam[cs:ce] = reverse_cumsum_with_total(r["dgam"], r["dgamC"][None, :])
            dh0[n, h] = dS
            qn, kn, rq, rk, beta = p["qn"], p["kn"], p["rq"], p["rk"], p["beta"]
            # grouped heads: a key head's gradient sums its value heads' contributions
            dq[t0:t1, h // G] += rq[:, None] * (dqn - qn * (qn * dqn).sum(1, keepdims=True))
            dk[t0:t1, h // G] += rk[:, None] * (dkn - kn * (kn * dkn).sum(1, keepdims=True))
            db[t0:t1, h] = dbeta * beta * (1 - beta)
            if gate == 0:
                dg[t0:t1, h] = dlam.sum(1)
            elif gate == 1:
                dgr = dlam * (-p["ea"] * _sigmoid(p["x"]))
                dg[t0:t1, h] = dgr
                ddt[h] += dgr.sum(0)
                dA[h] += (dlam * p["lam"]).sum()
            else:
                sz = _sigmoid(p["ea"] * p["x"])
                dz = dlam * float(inp["gate_scale"]) * sz * (1 - sz)
                dg[t0:t1, h] = dz * p["ea"]
                ddt[h] += (dz * p["ea"]).sum(0)
                dA[h] += (dz * p["ea"] * p["x"]).sum()
            S_h += Ss; dS_h += dSs; A_h += [z["A"] for z in zs]
        S_chunk.append(S_h); dS_chunk.append(dS_h); A_chunk.append(A_h)
    sh = lambda x: x.reshape((B, T) + x.shape[1:])  # noqa: E731
    out = dict(o=sh(o), dq=sh(dq), dk=sh(dk), dv=sh(dv), dg=sh(dg), db=sh(db), ht=ht, dh0=dh0, u=sh(U_all),
               S_chunk=np.array([np.stack(s) for s in S_chunk]) if S_chunk and S_chunk[0] else None,
               dS_chunk=np.array([np.stack(s) for s in dS_chunk]) if dS_chunk and dS_chunk[0] else None,
               A_chunk=A_chunk)
    if gate >= 1:
        out["dA_log"], out["ddt_bias"] = dA, ddt
    return out
