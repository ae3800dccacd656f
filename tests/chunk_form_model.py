"""fp64 model of the chunk-parallel algorithm the HIP chunk kernel implements.

Test-side only: it validates, against the oracle's recurrence, the algebra the
kernel is built on (sub-chunks, window unknowns, decay products, blocked
unit-lower-triangular solve, per-key folding, readout and carry).  It shares
no code with the kernel; it is the same sequence of steps written in numpy.

Within a sub-chunk of c steps starting from state S0 (per value row i):
  g_t = prod_{r<=t} a_r (g_{-1} = 1), zeta_t = eta_t / g_t
  unknowns u = (t, w), w = 0..B-1, key j(u) = t - w:
    e_u + g_{t-1} sum_{s<t, w'} G[j(u), j(s,w')] z_{(s,w')} = y_{j(u)} - g_{t-1} S0 x_{j(u)}
    z_u = zeta_t e_u   (inner-product family: e_u = y_{j(u)}, no solve)
  o_t   = g_t (S0 q_t + sum_{s<=t, w'} (q_t . x_{j(s,w')}) z_{(s,w')})
  S_c   = g_{c-1} (S0 + sum_j F_j x_j^T),  F_j = sum_{u: j(u)=j} z_u
(163.com section 02 (2): inside a chunk everything is parallel, only the fixed
size state crosses chunks; explainer §3 chunk-parallel form.)
"""
import numpy as np


def sub_chunk_size(chunk, window):
    c = chunk
    while c * window > 64:
        c //= 2
    return c


def chunk_forward(regression, per_row, q, k, v, *, beta, lam, eps, window, chunk,
                  beta_t=None, k_prev=None, S0=None, blk=16):
    """q, k [L, dk]; v [L, dv]; beta_t None, [L] or [L, dv].  One (batch, head)."""
    L, dk = q.shape
    dv = v.shape[1]
    B = window
    c = sub_chunk_size(chunk, B)
    U = c * B
    S = np.zeros((dv, dk)) if S0 is None else S0.astype(np.float64).copy()
    o = np.zeros((L, dv))

    def key(g):                      # x_g (0-based global step g)
        if g < 0:
            return np.zeros(dk)
        if g == 0:
            return np.zeros(dk) if k_prev is None else k_prev.astype(np.float64)
        return k[g - 1].astype(np.float64)

    def val(g):
        return np.zeros(dv) if g < 0 else v[g].astype(np.float64)

    c_full = c
    for t0 in range(0, L, c_full):
        c = min(c_full, L - t0)          # ragged tail
        U = c * B
        nx = c + B - 1
        X = np.stack([key(t0 - B + 1 + jj) for jj in range(nx)])      # [nx, dk]
        Y = np.stack([val(t0 - B + 1 + jj) for jj in range(nx)])      # [nx, dv]
        Q = q[t0:t0 + c].astype(np.float64)
        jof = lambda u: u // B - u % B + B - 1                         # local key of unknown
        # scalars
        nrm = np.sum(X * X, axis=1)
        eta = np.zeros((c, dv))
        a = np.zeros((c, dv))
        for t in range(c):
            n = sum(nrm[jof(t * B + w)] for w in range(B))
            if beta_t is None:
                b = np.full(dv, beta)
            elif beta_t.ndim == 2:
                b = beta_t[t0 + t].astype(np.float64)
            else:
                b = np.full(dv, float(beta_t[t0 + t]))
            if t0 + t == 0 and k_prev is None:
                eta[t], a[t] = 0.0, 1.0                                # fresh start
            else:
                eta[t] = b / (eps + n)
                a[t] = 1.0 - eta[t] * lam
        if not per_row:
            assert np.all(eta == eta[:, :1])
        g = np.cumprod(a, axis=0)                                      # [c, dv]
        gm1 = np.vstack([np.ones((1, dv)), g[:-1]])
        zeta = eta / g
        G = X @ X.T
        P = Q @ X.T
        # gathered, masked Gram over unknowns and readout weights
        Gt = np.zeros((U, U))
        Pt = np.zeros((c, U))
        for u in range(U):
            for u2 in range(U):
                if u2 // B < u // B:
                    Gt[u, u2] = G[jof(u), jof(u2)]
        for t in range(c):
            for u2 in range(U):
                if u2 // B <= t:
                    Pt[t, u2] = P[t, jof(u2)]
        step = np.arange(U) // B
        XS0 = X @ S.T                                                  # [nx, dv]
        if regression:
            R = np.stack([Y[jof(u)] - gm1[u // B] * XS0[jof(u)] for u in range(U)])  # [U, dv]
            Z = np.zeros((U, dv))
            for b0 in range(0, U, blk):
                b1 = min(U, b0 + blk)
                Rb = R[b0:b1] - gm1[step[b0:b1]] * (Gt[b0:b1, :b0] @ Z[:b0])
                if not per_row:
                    # shared diagonal block inverse T_bb = (I + A_bb)^-1
                    A = gm1[step[b0:b1], 0][:, None] * Gt[b0:b1, b0:b1] \
                        * zeta[step[b0:b1], 0][None, :]
                    T = np.linalg.inv(np.eye(b1 - b0) + A)
                    Eb = T @ Rb
                    Z[b0:b1] = zeta[step[b0:b1]] * Eb
                else:
                    # per-row forward substitution inside the block
                    for uu in range(b0, b1):
                        e = Rb[uu - b0] - gm1[step[uu]] * (Gt[uu, b0:uu] @ Z[b0:uu])
                        Z[uu] = zeta[step[uu]] * e
        else:
            Z = np.stack([zeta[u // B] * Y[jof(u)] for u in range(U)])
        F = np.zeros((nx, dv))
        for u in range(U):
            F[jof(u)] += Z[u]
        o[t0:t0 + c] = g * (Q @ S.T + Pt @ Z)
        S = g[-1][:, None] * (S + F.T @ X)
    return o, S


def chunk_forward_wy(regression, q, k, v, *, beta, lam, eps, chunk, beta_t=None, k_prev=None,
                     S0=None, blk=16):
    """Window 1, gains shared by the value rows (scalar or per token): the form in
    which every state-independent factor of a chunk is formed ahead of the state.

    With omega_t = zeta_t g_{t-1} (= eta_t / a_t) the chunk's equations become
      (I + diag(omega) L) z = diag(omega) (y / g_{t-1} - S0 x_t),  L = strictly lower Gram,
    so with N = (I + diag(omega) L)^-1 (unit lower triangular, the same for every
    value row) and Nw = N diag(omega):
      z = Ut - S0 Wt,  Ut[:, t] = sum_s Nw[t, s] y_s / g_{s-1},  Wt[:, t] = sum_s Nw[t, s] x_s
    N is built the way the kernel builds it: 16x16 diagonal blocks by forward
    substitution, then each block column downwards,
      N_bj = -T_bb sum_{m=j}^{b-1} (diag(omega) L)_bm N_mj.
    Readout and carry are those of chunk_forward; the inner-product family has
    z = zeta * y.
    """
    L_, dk = q.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else S0.astype(np.float64).copy()
    o = np.zeros((L_, dv))
    for t0 in range(0, L_, chunk):
        C = chunk                               # padded to the full chunk, like the kernel
        c = min(chunk, L_ - t0)
        X = np.zeros((C, dk))
        Y = np.zeros((C, dv))
        Q = np.zeros((C, dk))
        for t in range(c):
            g = t0 + t
            if g >= 1:
                X[t] = k[g - 1]
            elif k_prev is not None:
                X[t] = k_prev
            Y[t] = v[g]
            Q[t] = q[g]
        eta = np.zeros(C)
        a = np.ones(C)
        for t in range(c):
            if t0 + t == 0 and k_prev is None:
                continue
            b = beta if beta_t is None else float(beta_t[t0 + t])
            eta[t] = b / (eps + X[t] @ X[t])
            a[t] = 1.0 - eta[t] * lam
        g = np.cumprod(a)
        gm1 = np.concatenate([[1.0], g[:-1]])
        zeta = eta / g
        omega = zeta * gm1
        if regression:
            G = X @ X.T
            M = omega[:, None] * np.tril(G, -1)
            N = np.zeros((C, C))
            nb = C // blk
            T = []
            for bb in range(nb):                 # diagonal blocks: forward substitution
                u0 = bb * blk
                Tb = np.zeros((blk, blk))
                for cc in range(blk):
                    col = np.zeros(blk)
                    for r in range(blk):
                        col[r] = (1.0 if r == cc else 0.0) - M[u0 + r, u0:u0 + r] @ col[:r]
                    Tb[:, cc] = col
                T.append(Tb)
                N[u0:u0 + blk, u0:u0 + blk] = Tb
            for j in range(nb - 1):              # block columns, downwards
                for bb in range(j + 1, nb):
                    r0, c0 = bb * blk, j * blk
                    X1 = sum(M[r0:r0 + blk, m * blk:(m + 1) * blk] @ N[m * blk:(m + 1) * blk, c0:c0 + blk]
                             for m in range(j, bb))
                    N[r0:r0 + blk, c0:c0 + blk] = -T[bb] @ X1
            Nw = N * omega[None, :]
            Ut = (Y / gm1[:, None]).T @ Nw.T     # [dv, C]
            Wt = X.T @ Nw.T                      # [dk, C]
            Z = Ut - S @ Wt                      # [dv, C]
        else:
            Z = (zeta[:, None] * Y).T
        P = np.tril(Q @ X.T)                     # [C, C], s <= t
        O = (S @ Q.T + Z @ P.T) * g[None, :]     # [dv, C]
        o[t0:t0 + c] = O.T[:c]
        S = g[-1] * (S + Z @ X)
    return o, S


def chunk_forward_folded(regression, q, k, v, *, beta, lam, eps, window, beta_t=None,
                         k_prev=None, S0=None, cs=16, blk=16):
    """Key-folded form for a window B >= 1 with gains shared by the value rows.

    Sub-chunks of cs steps; the key tile of sub-chunk c is the 2 cs keys of
    sub-chunks c-1 and c (tile index m; key of unknown u = (t, w) is
    m(u) = cs + t - w).  With V = (I + M)^-1 (M over the unknowns, coupling only
    earlier steps) the state-independent matrices are
      F_x = V diag(omega_u) Gath,  F_y = V diag(zeta_u) Gath   (Gath[u, m] = [m(u) = m])
      H_x = Gath^T F_x,  H_y = Gath^T F_y,  Q_x = P' F_x,  Q_y = P' F_y
    (P'[t, u] = (q_t . x_m(u)) [t(u) <= t]); the inner-product family has
    F_x = 0 and F_y = diag(zeta_u) Gath.  Per value row the state enters only
    through XS = X S0^T:
      Fk = H_y Y - H_x XS,  o = g (Q S0^T + Q_y Y - Q_x XS),  S_c = g_last (S0 + Fk^T X).
    """
    L, dk = q.shape
    dv = v.shape[1]
    B = window
    S = np.zeros((dv, dk)) if S0 is None else S0.astype(np.float64).copy()
    o = np.zeros((L, dv))
    NXT = 2 * cs

    def key(g):
        if g < 0:
            return np.zeros(dk)
        if g == 0:
            return np.zeros(dk) if k_prev is None else k_prev.astype(np.float64)
        return k[g - 1].astype(np.float64)

    def val(g):
        return np.zeros(dv) if g < 0 or g >= L else v[g].astype(np.float64)

    for t0 in range(0, L, cs):
        c = min(cs, L - t0)
        U = cs * B
        X = np.stack([key(t0 - cs + m) if t0 - cs + m < t0 + c else np.zeros(dk)
                      for m in range(NXT)])                           # [2cs, dk]
        Y = np.stack([val(t0 - cs + m) if t0 - cs + m < t0 + c else np.zeros(dv)
                      for m in range(NXT)])
        Q = np.zeros((cs, dk))
        Q[:c] = q[t0:t0 + c]
        mof = lambda u: cs + u // B - u % B
        nrm = np.sum(X * X, axis=1)
        eta = np.zeros(cs)
        a = np.ones(cs)
        for t in range(c):
            n = sum(nrm[mof(t * B + w)] for w in range(B))
            b = beta if beta_t is None else float(beta_t[t0 + t])
            if not (t0 + t == 0 and k_prev is None):
                eta[t] = b / (eps + n)
                a[t] = 1.0 - eta[t] * lam
        g = np.cumprod(a)
        gm1 = np.concatenate([[1.0], g[:-1]])
        zeta = eta / g
        omega = zeta * gm1
        G = X @ X.T
        P = Q @ X.T
        tu = np.arange(U) // B
        Gath = np.zeros((U, NXT))
        Gath[np.arange(U), [mof(u) for u in range(U)]] = 1.0
        Pp = np.array([[P[t, mof(u)] if tu[u] <= t else 0.0 for u in range(U)] for t in range(cs)])
        if regression:
            Gp = Gath @ G @ Gath.T
            M = omega[tu][:, None] * Gp * (tu[None, :] < tu[:, None])
            # blocked forward solve of (I + M) V = I, blocks of blk unknowns
            V = np.zeros((U, U))
            for b0 in range(0, U, blk):
                b1 = b0 + blk
                T = np.linalg.inv(np.eye(blk) + M[b0:b1, b0:b1])
                rhs = np.zeros((blk, U))
                rhs[:, b0:b1] = np.eye(blk)
                V[b0:b1] = T @ (rhs - M[b0:b1, :b0] @ V[:b0])
            Fx = V @ (omega[tu][:, None] * Gath)
            Fy = V @ (zeta[tu][:, None] * Gath)
        else:
            Fx = np.zeros((U, NXT))
            Fy = zeta[tu][:, None] * Gath
        Hx, Hy = Gath.T @ Fx, Gath.T @ Fy
        Qx, Qy = Pp @ Fx, Pp @ Fy
        XS = X @ S.T                                                  # [2cs, dv]
        Fk = Hy @ Y - Hx @ XS
        o[t0:t0 + c] = (g[:, None] * (Q @ S.T + Qy @ Y - Qx @ XS))[:c]
        S = g[c - 1] * (S + Fk.T @ X)
    return o, S


def chunk_backward(regression, q, k, v, dO, *, beta, lam, eps, chunk, beta_t=None, k_prev=None,
                   S0=None, same_step=False, dS_L=None, dk_last=None):
    """Backward of the window-1 chunk form, per value row, one chain.

    q, k [L, dk]; v, dO [L, dv]; beta_t None, [L] or [L, dv] (per channel).  The
    derivation (chain rule through the chunk equations of the module docstring,
    0-based steps t of a chunk, row i implicit, gC = g_{c-1}):
      forward   r_t = y_t - g_{t-1} (s0.x_t); e = A^-1 r, A_ts = [t==s] + g_{t-1} G_ts zeta_s
                (s < t); z = zeta e; o_t = g_t (q_t.s0 + sum_{s<=t} P_ts z_s);
                s_end = gC (s0 + sum_s z_s x_s)
      backward  dz_s = sum_{t>=s} P_ts g_t do_t + gC (x_s.ds_end);  de = zeta dz
                dr = A^-T de:  dr_s = de_s - zeta_s sum_{t>s} G_ts w_t,  w_t = g_{t-1} dr_t
                ds0 = gC ds_end + sum_t g_t do_t q_t - sum_t w_t x_t
                dG_ts = -sum_i w_t z_s (t > s),  dP_ts = sum_i g_t do_t z_s (s <= t)
                dq_t = sum_i g_t do_t s0 + sum_s dP_ts x_s
                dx_t = sum_i (-w_t s0 + gC z_t ds_end) + sum_s (dG_ts + dG_st) x_s
                       + sum_t' dP_t't q_t' + 2 dn_t x_t
      scalars   dg_t += do_t o_t / g_t;  dg_{t-1} -= dr_t (h_t + s0.x_t), h_t = sum_{s<t} G_ts z_s;
                dzeta_t = dz_t e_t - e_t sum_{t'>t} G_t't w_t';  dgC += ds_end.s_end / gC;
                zeta = eta / g;  g_t = prod_{r<=t} a_r;  a = 1 - lambda eta;
                eta = beta / (eps + n):  dbeta = deta / (eps + n),  dn = -sum_i deta eta / (eps + n)
    Inner-product family: e = r = y (no solve, no terms through A or s0.x).
    """
    f64 = lambda a: None if a is None else np.asarray(a, dtype=np.float64)
    q, k, v, dO = f64(q), f64(k), f64(v), f64(dO)
    beta_t, k_prev, S0, dS_L, dk_last = f64(beta_t), f64(k_prev), f64(S0), f64(dS_L), f64(dk_last)
    L, dk = q.shape
    dv = v.shape[-1]
    x = np.zeros_like(k)
    if same_step:
        x[:] = k
    else:
        x[1:] = k[:-1]
        if k_prev is not None:
            x[0] = k_prev
    fresh = (k_prev is None) and not same_step
    nrm = np.sum(x * x, axis=-1)

    def scalars(t0, c):
        bt = np.empty((c, dv))
        for t in range(c):
            if beta_t is None:
                bt[t] = beta
            elif beta_t.ndim == 2:
                bt[t] = beta_t[t0 + t]
            else:
                bt[t] = beta_t[t0 + t]
        eta = bt / (eps + nrm[t0:t0 + c])[:, None]
        if fresh and t0 == 0:
            eta[0] = 0.0
        a = 1.0 - lam * eta
        g = np.cumprod(a, axis=0)                    # g_t, inclusive
        gm = np.vstack([np.ones((1, dv)), g[:-1]])    # g_{t-1}
        return eta, a, g, gm, eta / g

    def forward_chunk(t0, c, S):
        X, Q, Y = x[t0:t0 + c], q[t0:t0 + c], v[t0:t0 + c]
        G = X @ X.T
        P = np.tril(Q @ X.T)
        eta, a, g, gm, zeta = scalars(t0, c)
        XS = X @ S.T                                  # [c, dv] = s0 . x_t per row
        E = np.zeros((c, dv))
        Z = np.zeros((c, dv))
        for t in range(c):
            if regression:
                h = G[t, :t] @ Z[:t]
                E[t] = Y[t] - gm[t] * (XS[t] + h)
            else:
                E[t] = Y[t]
            Z[t] = zeta[t] * E[t]
        S_end = g[-1][:, None] * (S + Z.T @ X)
        return dict(X=X, Q=Q, G=G, P=P, eta=eta, a=a, g=g, gm=gm, zeta=zeta, XS=XS, E=E, Z=Z,
                    S=S, S_end=S_end)

    # forward sweep: chunk-start states
    starts = list(range(0, L, chunk))
    S = np.zeros((dv, dk)) if S0 is None else S0.copy()
    S_starts = []
    for t0 in starts:
        c = min(chunk, L - t0)
        S_starts.append(S)
        S = forward_chunk(t0, c, S)["S_end"]
    # backward sweep
    dq = np.zeros_like(q)
    dx = np.zeros_like(x)
    dy = np.zeros_like(v)
    dbeta = None if beta_t is None else np.zeros_like(beta_t)
    dS = np.zeros((dv, dk)) if dS_L is None else dS_L.copy()
    for ci in range(len(starts) - 1, -1, -1):
        t0 = starts[ci]
        c = min(chunk, L - t0)
        f = forward_chunk(t0, c, S_starts[ci])
        X, Q, G, P, S0c = f["X"], f["Q"], f["G"], f["P"], f["S"]
        eta, a, g, gm, zeta, E, Z = f["eta"], f["a"], f["g"], f["gm"], f["zeta"], f["E"], f["Z"]
        dOc = dO[t0:t0 + c]
        gC = g[-1]                                    # [dv]
        QS = Q @ S0c.T                                # q_t . s0
        ohat = QS + P @ Z                             # o_t / g_t
        gdo = g * dOc                                 # g_t do_t
        dg = dOc * ohat                               # from o_t = g_t ohat_t
        dgC = np.sum(dS * f["S_end"], axis=1) / gC
        XdS = X @ dS.T                                # x_s . ds_end  [c, dv]
        dZ = P.T @ gdo + gC * XdS
        dzeta = dZ * E
        dE = zeta * dZ
        if regression:
            W = np.zeros((c, dv))
            dR = np.zeros((c, dv))
            for s in range(c - 1, -1, -1):
                gs = G[s + 1:, s] @ W[s + 1:] if s + 1 < c else np.zeros(dv)
                dR[s] = dE[s] - zeta[s] * gs
                W[s] = gm[s] * dR[s]
                dzeta[s] -= E[s] * gs
            Hh = np.tril(G, -1) @ Z                   # h_t
            dgm = -dR * (Hh + f["XS"])
        else:
            dR = dE
            W = np.zeros((c, dv))
            dgm = np.zeros((c, dv))
        dy[t0:t0 + c] = dR
        dS_prev = gC[:, None] * dS + gdo.T @ Q - W.T @ X
        dG = -np.tril(W @ Z.T, -1)
        dP = np.tril(gdo @ Z.T)
        dq[t0:t0 + c] = gdo @ S0c + dP @ X
        dxc = -W @ S0c + (gC * Z) @ dS + (dG + dG.T) @ X + dP.T @ Q
        # scalars
        deta = dzeta / g
        dg = dg - dzeta * zeta / g
        dg[-1] += dgC
        dg[:-1] += dgm[1:]                            # g_{t-1} of step t is g_{t-1}
        # g_t = prod_{r<=t} a_r  ->  da_r = sum_{t>=r} dg_t g_t / a_r
        suffix = np.cumsum((dg * g)[::-1], axis=0)[::-1]
        da = suffix / a
        deta = deta - lam * da
        if fresh and t0 == 0:
            deta[0] = 0.0
        den = eps + nrm[t0:t0 + c]
        dn = -np.sum(deta * eta, axis=1) / den
        dxc += 2.0 * dn[:, None] * X
        dx[t0:t0 + c] += dxc
        if dbeta is not None:
            if dbeta.ndim == 2:
                dbeta[t0:t0 + c] = deta / den[:, None]
            else:
                dbeta[t0:t0 + c] = np.sum(deta, axis=1) / den
        dS = dS_prev
    dk_ = np.zeros_like(k)
    out = {}
    if same_step:
        dk_ += dx
    else:
        dk_[:-1] += dx[1:]
        if k_prev is not None:
            out["dk_prev"] = dx[0].copy()
    if dk_last is not None:
        dk_[-1] += dk_last
    out.update(dq=dq, dk=dk_, dv=dy)
    if dbeta is not None:
        out["dbeta_t"] = dbeta
    if S0 is not None:
        out["dS0"] = dS
    return out


def masked_blocked(regression, q, k, v, *, beta, lam, eps, beta_t=None, k_prev=None, S0=None,
                   same_step=False, rnd=None):
    """The masked-parallel form for one short call (L <= 64, window 1, gains shared
    by the value rows) in the blocked shape the matrix-core masked kernel uses.

    Steps t = 0..63 (padded steps: zero sample, eta = 0, a = 1), blocks of 16.
    With D[t][s] = prod_{s<r<=t} a_r and d_t = D[t][-1]:
      A[t][s] = eta_s D[t-1][s] (x_t . x_s)   (s < t; regression family)
      (I + A) E = Y - diag(d_{t-1}) X S0^T     (E = Y for the inner-product family)
      W[t][s] = eta_s D[t][s] (q_t . x_s)      (s <= t)
      O = diag(d_t) Q S0^T + W E
      S_L = d_63 S0 + E^T diag(eta_s D[63][s]) X
    Every decay factor is a product of a's (no division): inside a block a running
    product; across blocks  D[t-1][s] = suf_s * mid(k, b) * pin_t  with suf_s the
    product over the rest of s's block, mid the products of the whole blocks in
    between and pin_t the product over t's block before t (inclusive of t for W).
    The solve is blocked: T_bb = (I + A_bb)^-1, E_b = T_bb (R_b - sum_{k<b} A_bk E_k).
    ``rnd``: optional rounding applied to every product operand (precision study).
    """
    L, dk = q.shape
    dv = v.shape[1]
    N, NB = 64, 4
    f = (lambda a: a) if rnd is None else rnd
    X = np.zeros((N, dk))
    Q = np.zeros((N, dk))
    Y = np.zeros((N, dv))
    s = 0 if same_step else 1
    for t in range(L):
        g = t - s
        if g >= 0:
            X[t] = k[g]
        elif k_prev is not None:
            X[t] = k_prev
        Q[t] = q[t]
        Y[t] = v[t]
    fresh = (not same_step) and k_prev is None
    n = np.sum(X * X, axis=1)
    bt = np.full(N, beta if beta is not None else 0.0)
    if beta_t is not None:
        bt[:L] = beta_t
    live = np.arange(N) < L
    eta = np.zeros(N)
    eta[live] = bt[live] / (eps + n[live])
    if fresh:
        eta[0] = 0.0
    a = 1.0 - eta * lam
    a[np.arange(N) >= L] = 1.0
    if fresh:
        a[0] = 1.0
    G = f(X) @ f(X).T
    P = f(Q) @ f(X).T
    blk = np.arange(N) // 16
    # in-block products: pin_x[t] = prod_{16 b(t) <= r < t} a_r, pin_i[t] includes a_t,
    # suf[s] = prod_{s < r < 16 (b(s) + 1)} a_r, bp[b] = product of block b
    pin_x = np.ones(N)
    pin_i = np.ones(N)
    suf = np.ones(N)
    bp = np.ones(NB)
    for b in range(NB):
        run = 1.0
        for t in range(16 * b, 16 * b + 16):
            pin_x[t] = run
            run *= a[t]
            pin_i[t] = run
        bp[b] = run
        run = 1.0
        for t in range(16 * b + 15, 16 * b - 1, -1):
            suf[t] = run
            run *= a[t]

    def mid(kb, b):                 # product of the whole blocks strictly between
        return np.prod(bp[kb + 1:b]) if b > kb + 1 else 1.0

    def dec(t, s_, incl):           # D[t][s] (incl) or D[t-1][s]
        if blk[t] == blk[s_]:
            r = 1.0
            for q_ in range(s_ + 1, t + (1 if incl else 0)):
                r *= a[q_]
            return r
        return suf[s_] * mid(blk[s_], blk[t]) * (pin_i[t] if incl else pin_x[t])

    A = np.zeros((N, N))
    W = np.zeros((N, N))
    for t in range(N):
        for s_ in range(t + 1):
            if s_ < t:
                A[t, s_] = eta[s_] * dec(t, s_, False) * G[t, s_]
            W[t, s_] = eta[s_] * dec(t, s_, True) * P[t, s_]
    dprev = np.array([np.prod(bp[:blk[t]]) * pin_x[t] for t in range(N)])
    dincl = np.array([np.prod(bp[:blk[t]]) * pin_i[t] for t in range(N)])
    S0m = np.zeros((dv, dk)) if S0 is None else S0.astype(np.float64)
    R = Y - (dprev[:, None] * (f(X) @ f(S0m).T) if regression else 0.0)
    if regression:
        E = np.zeros((N, dv))
        for b in range(NB):
            sl = slice(16 * b, 16 * b + 16)
            Tbb = np.linalg.inv(np.eye(16) + A[sl, sl])
            acc = R[sl].copy()
            for kb in range(b):
                sk = slice(16 * kb, 16 * kb + 16)
                acc -= f(A[sl, sk]) @ f(E[sk])
            E[sl] = f(Tbb) @ f(acc)
    else:
        E = Y
    O = dincl[:, None] * (f(Q) @ f(S0m).T) + f(W) @ f(E)
    c = eta * suf * np.array([np.prod(bp[blk[s_] + 1:]) for s_ in range(N)])
    S_L = np.prod(bp) * S0m + (f(E * c[:, None])).T @ f(X)
    return O[:L], S_L
