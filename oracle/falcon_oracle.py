"""Plain fp64 CPU oracle for the Falcon fast-weight state update and readout.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only the
test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call it.  It shares no code with the HIP library
(no kernels, headers, helpers or constant tables) and imports nothing from it.

What it computes (sources: "Fast Weight Attention：用于持续学习的快速权重注意力",
papers.ananclaw.com explainer of arXiv 2608.27763, section 核心方法 §1 and the
variant table of §2; "借鉴40年前的设想！字节Seed提出快速权重注意力..." (163.com),
section 02 (1) and (2)):

* prefix-aligned sample pair (x_t, y_t) = (phi(k_{t-1}), v_t), phi = identity,
  x_1 = k_prev when the caller carries one, else the zero vector
  (explainer §1; 163.com section 01);
* one normalized first-order step per token on the online loss
  L(S) = sum_{j in W_t} l(S; x_j, y_j) + (lambda/2)||S||_F^2, with
  l = 1/2||S x - y||^2 (regression family: Falcon-1/2/3) or l = -y^T S x
  (inner-product family: Falcon-1A/2A/3A) (explainer §1; 163.com 02 (1));
  written out this is
      S_t = (1 - eta_t lambda) S_{t-1} + eta_t * sum_{j in W_t} e_j x_j^T,
      e_j = y_j - S_{t-1} x_j   (regression)   or   e_j = y_j   (inner product);
* eta_t = beta_t / (eps + n_t), n_t = sum_{j in W_t} ||x_j||^2 (NLMS step
  normalization, 163.com 02 (1)); granularity from the variant table
  (explainer §2; 163.com 02 (2)): one eta shared by every value channel
  (Falcon-1/1A), one eta per value channel = per row of S (Falcon-2/2A), or a
  sliding window W_t of the B latest causal samples (Falcon-3/3A; B = 1
  otherwise);
* read-after-write readout o_t = S_t q_t (163.com section 01: observe and
  write first, then predict with the updated state).

Readings where the pages leave a step open (each also listed in the design
notes of the repository):

* Falcon-3 window: the loss is the *sum* over the window, the normalizer is
  the summed squared norm of the window's inputs, the window holds the current
  sample and is truncated at the start of the sequence.  Parity against the
  authors' Falcon-3 is unpinned (no page prints the formula); what is pinned is
  that the step is exactly one normalized gradient step on that summed loss.
* Per-channel (Falcon-2): a value channel is a row of S (S maps key space to
  value space, S x); eta_{t,i} = beta_{t,i} / (eps + ||x_t||^2).
* A fresh sequence starts at S_0 = 0 with x_1 = 0; then S_1 = 0 exactly.  With
  eps = 0 the literal step is 0/0 there; the oracle defines S_1 = 0 and raises
  for a zero denominator on a non-zero state.
* Resuming a Falcon-3/3A sequence: besides S and the carried key, the window
  of the first B-1 steps reaches back into the previous call, so the caller
  carries the B-1 latest samples (x_j, y_j) as a history (oldest first).  The
  window is then "the B latest causal samples" over the joined sample list.
  A zero sample adds nothing to n_t or to the write, so a history of zeros is
  the same as none (a fresh sequence).

Functions
---------
``falcon_recurrence``   the recurrence, step by step (the plain definition).
``falcon_masked_parallel``  an independent second evaluation: every output as
                        an explicit sum over the causal mask of transition
                        products (the masked-parallel form of explainer §3),
                        tiny inputs only.
``falcon_decode_step``  exactly one step of the recurrence with x = k_prev.
``falcon_history``      the B-1 latest samples after a call (the history the
                        next call of a Falcon-3/3A sequence needs).
``falcon_decode_step_window``  one step with a carried window history.
``falcon_backward``     gradients of <dO, o> + <dS_L, S_L> + <dk_last, k_last>
                        with respect to every input, by reverse-mode
                        differentiation of the recurrence step by step (the
                        pages give no gradients; this is the chain rule applied
                        to the definition above).
"""
from __future__ import annotations

import numpy as np

# Variant ids (the same numbering as the C interface; defined here on their own).
FALCON_1, FALCON_2, FALCON_3, FALCON_1A, FALCON_2A, FALCON_3A = range(6)

_REGRESSION = {FALCON_1: True, FALCON_2: True, FALCON_3: True,
               FALCON_1A: False, FALCON_2A: False, FALCON_3A: False}
_WINDOWED = {FALCON_3, FALCON_3A}


def is_regression(variant: int) -> bool:
    return _REGRESSION[variant]


def _as64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def _shift_keys(k, k_prev, same_step):
    """x_t = k_{t-1} (x_1 = k_prev or 0); same_step: x_t = k_t (explainer §1 ⚠)."""
    if same_step:
        return k.copy()
    x = np.zeros_like(k)
    x[:, :, 1:] = k[:, :, :-1]
    if k_prev is not None:
        x[:, :, 0] = k_prev
    return x


def _beta_rows(beta, beta_t, t, shape_bh, dv):
    """beta for step t broadcast over value rows -> [B, H, dv]."""
    if beta_t is None:
        return np.full(shape_bh + (dv,), float(beta))
    if beta_t.ndim == 4:                       # per token and value channel
        return beta_t[:, :, t, :].copy()
    return np.repeat(beta_t[:, :, t][..., None], dv, axis=-1)   # per token


def _check_args(variant, window, q, k, v, beta_t):
    if variant not in _REGRESSION:
        raise ValueError("unknown variant %r" % (variant,))
    if window < 1:
        raise ValueError("window must be >= 1")
    if window != 1 and variant not in _WINDOWED:
        raise ValueError("window > 1 is Falcon-3/3A only")
    if q.shape != k.shape or q.shape[:3] != v.shape[:3]:
        raise ValueError("q, k, v shapes disagree")
    if beta_t is not None and beta_t.ndim == 4 and variant not in (FALCON_2, FALCON_2A):
        raise ValueError("per-channel beta is Falcon-2/2A only")


def _join_history(window, x, y, x_hist, y_hist):
    """Samples of the history (oldest first) followed by those of this call."""
    if x_hist is None and y_hist is None:
        return x, y, 0
    if x_hist is None or y_hist is None:
        raise ValueError("x_hist and y_hist go together")
    if window < 2:
        raise ValueError("a window history needs window > 1")
    if x_hist.shape != x.shape[:2] + (window - 1, x.shape[-1]) or \
            y_hist.shape != y.shape[:2] + (window - 1, y.shape[-1]):
        raise ValueError("history shapes must be [B, H, window-1, d]")
    return np.concatenate([x_hist, x], axis=2), np.concatenate([y_hist, y], axis=2), window - 1


def falcon_recurrence(variant, q, k, v, *, beta=0.5, lam=0.0, eps=1e-6, window=1,
                      beta_t=None, k_prev=None, S0=None, same_step=False,
                      x_hist=None, y_hist=None, return_states=False):
    """Run the Falcon recurrence in fp64, one token at a time.

    Shapes: q, k [B, H, L, dk]; v [B, H, L, dv]; beta_t None, [B, H, L] or
    [B, H, L, dv] (Falcon-2/2A); k_prev [B, H, dk]; S0 [B, H, dv, dk];
    x_hist [B, H, window-1, dk], y_hist [B, H, window-1, dv]: the samples
    before step 1 that the first windows reach (oldest first), or None.
    Returns (o [B, H, L, dv], S_L [B, H, dv, dk], k_last [B, H, dk]) and, with
    ``return_states``, also every S_t as [B, H, L, dv, dk].
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    beta_t, k_prev, S0 = _as64(beta_t), _as64(k_prev), _as64(S0)
    x_hist, y_hist = _as64(x_hist), _as64(y_hist)
    _check_args(variant, window, q, k, v, beta_t)
    Bz, H, L, dk = q.shape
    dv = v.shape[-1]
    regression = _REGRESSION[variant]
    x = _shift_keys(k, k_prev, same_step)
    y = v
    x, y, P = _join_history(window, x, y, x_hist, y_hist)   # sample P + t is step t's own
    S = np.zeros((Bz, H, dv, dk)) if S0 is None else S0.copy()
    o = np.zeros((Bz, H, L, dv))
    states = np.zeros((Bz, H, L, dv, dk)) if return_states else None
    for t in range(L):
        lo = max(0, P + t - window + 1)
        Xw = x[:, :, lo:P + t + 1]                  # [B, H, w, dk]
        Yw = y[:, :, lo:P + t + 1]                  # [B, H, w, dv]
        n = np.sum(Xw * Xw, axis=(-1, -2))          # [B, H]
        b = _beta_rows(beta, beta_t, t, (Bz, H), dv)  # [B, H, dv]
        denom = eps + n
        zero = denom == 0.0
        if np.any(zero):
            if np.any(np.abs(S[zero]) > 0):
                raise ZeroDivisionError("eps + ||x||^2 = 0 on a non-zero state")
            denom = np.where(zero, 1.0, denom)      # S stays 0 there (see below)
        eta = b / denom[..., None]                  # [B, H, dv]
        eta = np.where(zero[..., None], 0.0, eta)
        a = 1.0 - eta * lam
        if regression:
            # e_j = y_j - S_{t-1} x_j for every window sample, pre-update S
            E = Yw - np.matmul(Xw, np.swapaxes(S, -1, -2))   # [B, H, w, dv]
        else:
            E = Yw
        write = np.matmul(np.swapaxes(E, -1, -2), Xw)          # [B, H, dv, dk]
        S = a[..., None] * S + eta[..., None] * write
        o[:, :, t] = np.matmul(S, q[:, :, t][..., None])[..., 0]
        if return_states:
            states[:, :, t] = S
    k_last = k[:, :, -1].copy() if L > 0 else (k_prev.copy() if k_prev is not None else None)
    if return_states:
        return o, S, k_last, states
    return o, S, k_last


def falcon_history(k, v, window, *, k_prev=None, x_hist=None, y_hist=None, same_step=False):
    """The window-1 latest samples (x_j, y_j) after a call, oldest first.

    The joined sample list is the incoming history (if any) followed by this
    call's samples x_t (the shifted keys) and y_t = v_t; the result is its
    tail, padded in front with zero samples when the list is shorter.
    Returns (x_hist [B, H, window-1, dk], y_hist [B, H, window-1, dv]).
    """
    k, v = _as64(k), _as64(v)
    x = _shift_keys(k, _as64(k_prev), same_step)
    x, y, _ = _join_history(window, x, v, _as64(x_hist), _as64(y_hist))
    n = window - 1
    Bz, H, Lx, dk = x.shape
    dv = y.shape[-1]
    xo = np.zeros((Bz, H, n, dk))
    yo = np.zeros((Bz, H, n, dv))
    take = min(n, Lx)
    if take > 0:
        xo[:, :, n - take:] = x[:, :, Lx - take:]
        yo[:, :, n - take:] = y[:, :, Lx - take:]
    return xo, yo


def falcon_decode_step_window(variant, window, S, k_prev, x_hist, y_hist, q, k, v, *,
                              beta=0.5, lam=0.0, eps=1e-6, same_step=False):
    """One decode step of Falcon-3/3A with a carried window history.

    x = k_prev (x = k with same_step), y = v; the window is the history
    (window-1 samples, oldest first) plus this sample.  Shapes: S [N, H, dv, dk];
    k_prev, q, k [N, H, dk]; v [N, H, dv]; x_hist [N, H, window-1, dk]; y_hist
    [N, H, window-1, dv].  Returns (o, S_new, k_prev_new, x_hist_new, y_hist_new);
    with same_step k_prev plays no part and comes back unchanged.
    """
    q3, k3, v3 = _as64(q)[:, :, None], _as64(k)[:, :, None], _as64(v)[:, :, None]
    kp = None if same_step else _as64(k_prev)
    o, S_new, _ = falcon_recurrence(variant, q3, k3, v3, beta=beta, lam=lam, eps=eps,
                                    window=window, k_prev=kp, S0=_as64(S),
                                    x_hist=x_hist, y_hist=y_hist, same_step=same_step)
    xh, yh = falcon_history(k3, v3, window, k_prev=kp, x_hist=x_hist, y_hist=y_hist,
                            same_step=same_step)
    k_next = k_prev if same_step else _as64(k).copy()
    return o[:, :, 0], S_new, k_next, xh, yh


def falcon_decode_step(variant, S, k_prev, q, k, v, *, beta=0.5, lam=0.0, eps=1e-6,
                       beta_t=None, same_step=False):
    """One decode step: x = k_prev, y = v, update S, o = S_new q; k_prev <- k.
    With same_step: x = k, and k_prev plays no part (returned unchanged).

    Shapes: S [N, H, dv, dk]; k_prev, q, k [N, H, dk]; v [N, H, dv];
    beta_t None, [N, H] or [N, H, dv].  Returns (o, S_new, k_prev_new).
    """
    if variant in _WINDOWED:
        raise ValueError("Falcon-3/3A decode needs its window history: "
                         "use falcon_decode_step_window")
    bt = None
    if beta_t is not None:
        beta_t = _as64(beta_t)
        bt = beta_t[:, :, None] if beta_t.ndim == 2 else beta_t[:, :, None, :]
    o, S_new, _ = falcon_recurrence(
        variant, _as64(q)[:, :, None], _as64(k)[:, :, None], _as64(v)[:, :, None],
        beta=beta, lam=lam, eps=eps, beta_t=bt, k_prev=None if same_step else _as64(k_prev),
        S0=_as64(S), same_step=same_step)
    return o[:, :, 0], S_new, (k_prev if same_step else _as64(k).copy())


def falcon_masked_parallel(variant, q, k, v, *, beta=0.5, lam=0.0, eps=1e-6, window=1,
                           beta_t=None, k_prev=None, S0=None, same_step=False):
    """Independent evaluation by the causal-mask expansion (explainer §3).

    Unrolling S_t = S_{t-1} M_t + eta_t R_t per value row i gives
        o_{t,i} = s0_i^T M_1..M_t q_t + sum_{s<=t} eta_{s,i} r_{s,i}^T M_{s+1}..M_t q_t
    with R_s = sum_{j in W_s} y_j x_j^T and the transition
        M_r = a_r I - eta_r sum_{j in W_r} x_j x_j^T   (regression)
        M_r = a_r I                                    (inner product).
    No residual is ever formed.  Cost O(L^2 dk^2) per row: tiny inputs only.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    beta_t, k_prev, S0 = _as64(beta_t), _as64(k_prev), _as64(S0)
    _check_args(variant, window, q, k, v, beta_t)
    Bz, H, L, dk = q.shape
    dv = v.shape[-1]
    regression = _REGRESSION[variant]
    x = _shift_keys(k, k_prev, same_step)
    o = np.zeros((Bz, H, L, dv))
    eye = np.eye(dk)
    for bi in range(Bz):
        for hi in range(H):
            # per-step quantities
            eta = np.zeros((L, dv))
            M = np.zeros((L, dv, dk, dk))
            Rrow = np.zeros((L, dv, dk))
            for s in range(L):
                lo = max(0, s - window + 1)
                n = sum(float(x[bi, hi, j] @ x[bi, hi, j]) for j in range(lo, s + 1))
                for i in range(dv):
                    if beta_t is None:
                        b = beta
                    elif beta_t.ndim == 4:
                        b = beta_t[bi, hi, s, i]
                    else:
                        b = beta_t[bi, hi, s]
                    e_si = 0.0 if eps + n == 0.0 else b / (eps + n)
                    eta[s, i] = e_si
                    Ms = (1.0 - e_si * lam) * eye
                    r = np.zeros(dk)
                    for j in range(lo, s + 1):
                        if regression:
                            Ms = Ms - e_si * np.outer(x[bi, hi, j], x[bi, hi, j])
                        r = r + v[bi, hi, j, i] * x[bi, hi, j]
                    M[s, i] = Ms
                    Rrow[s, i] = r
            for t in range(L):
                for i in range(dv):
                    w = q[bi, hi, t].copy()          # M_{s+1}..M_t q_t, built backwards
                    acc = 0.0
                    for s in range(t, -1, -1):
                        acc += eta[s, i] * float(Rrow[s, i] @ w)
                        w = M[s, i] @ w
                    if S0 is not None:
                        acc += float(S0[bi, hi, i] @ w)
                    o[bi, hi, t, i] = acc
    return o


def falcon_backward(variant, q, k, v, dO, *, beta=0.5, lam=0.0, eps=1e-6, window=1,
                    beta_t=None, k_prev=None, S0=None, same_step=False, dS_L=None,
                    dk_last=None):
    """Reverse-mode gradients of the recurrence.

    The scalar being differentiated is  sum_t <dO_t, o_t> + <dS_L, S_L> +
    <dk_last, k_last>  (dS_L and dk_last optional: the gradients arriving from a
    later call of the same sequence).  Shapes as ``falcon_recurrence``; dO
    [B, H, L, dv].  Returns a dict with dq, dk, dv and, when the input was given,
    dbeta_t (same shape as beta_t), dk_prev and dS0.  A scalar beta gets no
    gradient (it is a hyper-parameter here).

    Each step S_t = a S_{t-1} + eta sum_j e_j x_j^T, o_t = S_t q_t is undone in
    reverse order with the stored S_{t-1}: the adjoint dS of S_t gains dO_t q_t^T,
    then flows to eta, to the window samples (x_j, y_j), to n_t and to S_{t-1}.
    """
    q, k, v, dO = _as64(q), _as64(k), _as64(v), _as64(dO)
    beta_t, k_prev, S0 = _as64(beta_t), _as64(k_prev), _as64(S0)
    _check_args(variant, window, q, k, v, beta_t)
    Bz, H, L, dk = q.shape
    dv = v.shape[-1]
    regression = _REGRESSION[variant]
    o, S_L, _, states = falcon_recurrence(variant, q, k, v, beta=beta, lam=lam, eps=eps,
                                          window=window, beta_t=beta_t, k_prev=k_prev, S0=S0,
                                          same_step=same_step, return_states=True)
    x = _shift_keys(k, k_prev, same_step)
    y = v
    dx = np.zeros_like(x)
    dy = np.zeros_like(y)
    dq = np.zeros_like(q)
    dbeta = None if beta_t is None else np.zeros_like(beta_t)
    dS = np.zeros((Bz, H, dv, dk)) if dS_L is None else _as64(dS_L).copy()
    S_init = np.zeros((Bz, H, dv, dk)) if S0 is None else S0
    for t in range(L - 1, -1, -1):
        S_t = states[:, :, t]
        S_prev = states[:, :, t - 1] if t > 0 else S_init
        # o_t = S_t q_t
        dq[:, :, t] = np.matmul(np.swapaxes(S_t, -1, -2), dO[:, :, t][..., None])[..., 0]
        dS = dS + dO[:, :, t][..., None] * q[:, :, t][:, :, None, :]
        # the step's own quantities, recomputed from S_{t-1} as in the forward
        lo = max(0, t - window + 1)
        Xw = x[:, :, lo:t + 1]
        Yw = y[:, :, lo:t + 1]
        n = np.sum(Xw * Xw, axis=(-1, -2))
        b = _beta_rows(beta, beta_t, t, (Bz, H), dv)
        denom = eps + n
        zero = denom == 0.0
        denom_s = np.where(zero, 1.0, denom)
        eta = np.where(zero[..., None], 0.0, b / denom_s[..., None])        # [B, H, dv]
        a = 1.0 - eta * lam
        E = Yw - np.matmul(Xw, np.swapaxes(S_prev, -1, -2)) if regression else Yw
        write = np.matmul(np.swapaxes(E, -1, -2), Xw)                       # sum_j e_j x_j^T
        # S_t = a S_prev + eta write   (a, eta per value row)
        d_eta = np.sum(dS * (-lam * S_prev + write), axis=-1)               # [B, H, dv]
        d_eta = np.where(zero[..., None], 0.0, d_eta)
        dE = np.swapaxes(np.matmul(dS, np.swapaxes(Xw, -1, -2)), -1, -2) * eta[:, :, None, :]
        dXw = np.matmul(E, eta[..., None] * dS)                              # from the write
        dS_prev = a[..., None] * dS
        if regression:   # E = Y - X S_prev^T
            dS_prev = dS_prev - np.matmul(np.swapaxes(dE, -1, -2), Xw)
            dXw = dXw - np.matmul(dE, S_prev)
        dy[:, :, lo:t + 1] += dE
        # eta = beta / (eps + n), n = sum of the window's squared norms
        dn = -np.sum(d_eta * eta, axis=-1) / denom_s                         # [B, H]
        dXw = dXw + 2.0 * dn[..., None, None] * Xw
        dx[:, :, lo:t + 1] += dXw
        if dbeta is not None:
            g = d_eta / denom_s[..., None]
            if dbeta.ndim == 4:
                dbeta[:, :, t] = g
            else:
                dbeta[:, :, t] = np.sum(g, axis=-1)
        dS = dS_prev
    # x_t = k_{t-1} (x_1 = k_prev) or, same-step, x_t = k_t
    dk_ = np.zeros_like(k)
    dk_prev = None
    if same_step:
        dk_ += dx
    else:
        dk_[:, :, :-1] += dx[:, :, 1:]
        if k_prev is not None:
            dk_prev = dx[:, :, 0].copy()
    if dk_last is not None and L > 0:
        dk_[:, :, -1] += _as64(dk_last)
    out = dict(dq=dq, dk=dk_, dv=dy)
    if dbeta is not None:
        out["dbeta_t"] = dbeta
    if k_prev is not None and not same_step:
        out["dk_prev"] = dk_prev
    if S0 is not None:
        out["dS0"] = dS
    return out
