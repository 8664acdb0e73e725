"""Independent numpy forms that pin the fp64 oracle.

TEST INFRASTRUCTURE ONLY (imported by the test suite).  Nothing here is
shared with the oracle's C code or with the HIP library.

* ``quadratic_form`` -- the SSD "dual" (attention-like) form of the Mamba-2
  recurrence: the whole sequence at once as a masked matrix product
  ``Y = (Lmask o C B^T) (dt * X) + D X + decay * C h0``, with
  ``Lmask[t, s] = exp(sum_{r=s+1..t} dt_r A)`` for ``s <= t`` in the same
  document and 0 otherwise.  It materialises the L x L matrix, so it is for
  tiny inputs only.  The recurrence and its matrix form compute the same
  function; agreement to ~1e-12 pins dt scaling, the write (B) and read (C)
  sides, the inclusive output, group sharing, the D skip, the initial state
  and the document mask of the sequential oracle.
* ``zero_decay_form`` -- with A = 0 the state is a plain running sum of
  ``dt_s x_s B_s^T`` (``np.cumsum``), and ``y_t = C_t . S_t + D x_t``.
* ``conv_reference`` -- a causal depthwise conv without documents or carried
  state, via ``np.convolve`` (a library routine the oracle does not use).
* ``s6_quadratic_form`` -- the Mamba-1 selective scan written out the same
  way: for each channel d and state index n the whole sequence at once,
  ``h_t[n] = sum_s Lmask_dn[t, s] dt_s B_s[n] x_s + decay_dn[t] h0[n]`` with
  ``Lmask_dn[t, s] = exp(A[d, n] sum_{r=s+1..t} dt_r)`` inside a document,
  then ``y_t = C_t . h_t + D x_t`` and the gate.
"""
from __future__ import annotations

import numpy as np


def _segments(doc_row, L):
    """Segment index per token: a new segment starts where the document id changes."""
    if doc_row is None:
        return np.zeros(L, dtype=np.int64)
    d = np.asarray(doc_row)
    starts = np.concatenate([[0], (d[1:] != d[:-1]).astype(np.int64)])
    return np.cumsum(starts)


def quadratic_form(x, Bm, Cm, dt, A, D=None, z=None, doc_ids=None, init_state=None, *, H, P, N, G):
    """Y for all (b, h) via the materialised masked matrix; also returns the final state.

    x [B,L,H*P], Bm/Cm [B,L,G*N], dt [B,L,H] (already activated), A [H].
    """
    x = np.asarray(x, np.float64)
    Bsz, L, _ = x.shape
    Bm = np.asarray(Bm, np.float64)
    Cm = np.asarray(Cm, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    y = np.zeros((Bsz, L, H * P))
    fin = np.zeros((Bsz, H, P, N))
    hpg = H // G
    for b in range(Bsz):
        seg = _segments(None if doc_ids is None else doc_ids[b], L)
        same = seg[:, None] == seg[None, :]
        causal = np.tril(np.ones((L, L), dtype=bool))
        for h in range(H):
            g = h // hpg
            X = x[b, :, h * P:(h + 1) * P]                      # [L, P]
            Bg = Bm[b, :, g * N:(g + 1) * N]                    # [L, N]
            Cg = Cm[b, :, g * N:(g + 1) * N]                    # [L, N]
            dA = dt[b, :, h] * A[h]
            # cumulative log-decay restarted at every segment start
            cs = np.zeros(L)
            for t in range(L):
                cs[t] = dA[t] + (cs[t - 1] if t > 0 and seg[t] == seg[t - 1] else 0.0)
            with np.errstate(over="ignore"):
                decay = np.exp(cs[:, None] - cs[None, :])
            Lmask = np.where(same & causal, decay, 0.0)
            Y = (Lmask * (Cg @ Bg.T)) @ (dt[b, :, h][:, None] * X)
            if D is not None:
                Y = Y + D[h] * X
            S_end = (np.exp(cs[-1] - cs) * dt[b, :, h] * (seg == seg[-1]))[:, None] * X
            S_end = S_end.T @ Bg                                # [P, N]
            if init_state is not None:
                h0 = np.asarray(init_state, np.float64)[b, h]   # [P, N]
                first = seg == 0
                Y = Y + (first * np.exp(cs))[:, None] * (Cg @ h0.T)
                if seg[-1] == 0:
                    S_end = S_end + np.exp(cs[-1]) * h0
            if z is not None:
                Z = np.asarray(z, np.float64)[b, :, h * P:(h + 1) * P]
                Y = Y * (Z / (1.0 + np.exp(-Z)))
            y[b, :, h * P:(h + 1) * P] = Y
            fin[b, h] = S_end
    return y, fin


def zero_decay_form(x, Bm, Cm, dt, D=None, *, H, P, N, G):
    """A = 0: S_t = sum_{s<=t} dt_s x_s B_s^T, y_t = C_t . S_t + D x_t (no documents, zero h0)."""
    x = np.asarray(x, np.float64)
    Bsz, L, _ = x.shape
    y = np.zeros((Bsz, L, H * P))
    hpg = H // G
    for b in range(Bsz):
        for h in range(H):
            g = h // hpg
            X = x[b, :, h * P:(h + 1) * P]
            Bg = np.asarray(Bm, np.float64)[b, :, g * N:(g + 1) * N]
            Cg = np.asarray(Cm, np.float64)[b, :, g * N:(g + 1) * N]
            outer = (np.asarray(dt, np.float64)[b, :, h][:, None, None] * X[:, :, None]) * Bg[:, None, :]
            S = np.cumsum(outer, axis=0)                        # [L, P, N]
            Y = np.einsum("tpn,tn->tp", S, Cg)
            if D is not None:
                Y = Y + D[h] * X
            y[b, :, h * P:(h + 1) * P] = Y
    return y


def conv_reference(raw, w, bias=None, act_silu=True):
    """Causal depthwise conv per channel with np.convolve; no documents, zero history."""
    raw = np.asarray(raw, np.float64)
    Bsz, L, C = raw.shape
    K = w.shape[1]
    out = np.empty_like(raw)
    for b in range(Bsz):
        for c in range(C):
            v = np.convolve(raw[b, :, c], np.asarray(w[c], np.float64)[::-1])[:L]
            if bias is not None:
                v = v + bias[c]
            out[b, :, c] = v
    if act_silu:
        out = out / (1.0 + np.exp(-out))
    return out


def s6_quadratic_form(x, dt, A, Bm, Cm, D=None, z=None, doc_ids=None, init_state=None):
    """Y and the final state of the Mamba-1 selective scan via materialised per-(d, n) decay matrices.

    x, dt [B,L,D] (dt already activated), A [D,N], Bm, Cm [B,L,N], init_state [B,D,N].
    """
    x = np.asarray(x, np.float64)
    Bsz, L, Dn = x.shape
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    N = A.shape[1]
    Bm = np.asarray(Bm, np.float64)
    Cm = np.asarray(Cm, np.float64)
    y = np.zeros((Bsz, L, Dn))
    fin = np.zeros((Bsz, Dn, N))
    causal = np.tril(np.ones((L, L), dtype=bool))
    for b in range(Bsz):
        seg = _segments(None if doc_ids is None else doc_ids[b], L)
        mask = causal & (seg[:, None] == seg[None, :])
        first = seg == 0                                    # tokens that still see the initial state
        for d in range(Dn):
            T = np.cumsum(dt[b, :, d])                      # sum_{r <= t} dt_r
            for n in range(N):
                # Lmask[t, s] = exp(A (T_t - T_s)) for s <= t in one document
                E = np.where(mask, np.exp(A[d, n] * (T[:, None] - T[None, :])), 0.0)
                h = E @ (dt[b, :, d] * Bm[b, :, n] * x[b, :, d])
                if init_state is not None:
                    h = h + np.where(first, np.exp(A[d, n] * T), 0.0) * init_state[b, d, n]
                y[b, :, d] += Cm[b, :, n] * h
                fin[b, d, n] = h[-1] if L else (0.0 if init_state is None else init_state[b, d, n])
            if D is not None:
                y[b, :, d] += D[d] * x[b, :, d]
            if z is not None:
                zz = np.asarray(z, np.float64)[b, :, d]
                y[b, :, d] *= zz / (1.0 + np.exp(-zz))
    return y, fin
