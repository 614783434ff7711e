"""Independent fp64 chunkwise evaluation of the gated delta rule (TEST INFRASTRUCTURE ONLY).

This module evaluates, chunk by chunk and literally, the formulas the pages
give for the chunked-prefill forward.  It shares nothing with the token
recurrence in ``recurrent.py`` except the inputs, so agreement between the two
pins both (tests/test_oracle_chunkwise.py).

Notation (one sequence, one value head, one chunk of c <= C tokens):
    g_c    chunk-local inclusive cumsum of the log-gates, resetting at every
           chunk and sequence start   (06 . Flash Linear Attention, section 3,
           "why pre-multiply RCP_LN2": chunk_local_cumsum; natural log here,
           the base-2 pre-scaling is an implementation detail of the kernels)
    gamma  exp(g_c);  Gamma_ij = gamma_i / gamma_j (i >= j)
    A      (I + strictLower(diag(beta)(Gamma (.) K K^T)))^{-1}
    W, U   A diag(beta) diag(gamma) K,   A diag(beta) V
    V'     U - W S
    S      S <- gamma_C S + K^T diag(gamma_C / gamma) V'       (gamma_C: last valid token)
    O      scale * (diag(gamma) Q S + (Lower(Gamma) (.) Q K^T) V')   (mask includes the diagonal)

Sources: FlashQLA announcement (Qwen), section "key problems of FLA GDN
chunked prefill", the four-step forward for chunk i; GDN-in-FLA notes, forward
Steps 1-5; 06 . Flash Linear Attention, sections 3-6.  The scale is applied to
both output terms as in 06 . Flash Linear Attention section 3 (the FlashQLA
statement omits it).  The tail chunk's gamma_C is taken at its last valid token
(KDA source walk-through, section 3.3, last_idx).

Per-channel gates (KDA, KDA source walk-through sections 3-5), with G the
chunk-local cumsum of gk ([c, D_k]):
    A_raw[i, j] = beta_i sum_d k_id k_jd exp(G_id - G_jd)        (j < i)
    Aqk[i, j]   = sum_d q_id k_jd exp(G_id - G_jd)               (j <= i)
    W = A diag(beta) (K (.) exp(G)),  U = A diag(beta) V,  kg = K (.) exp(G_C - G)
    S <- Diag(exp(G_C)) S + kg^T V',   O = scale * ((Q (.) exp(G)) S + Aqk V')

Context parallelism (FlashQLA announcement, the DeltaNet-style CP pre-process
and the rewritten X/Y/Z form): each segment of chunks is run from S = 0 to get
S*, and its transition M from M = I; the segment start states are then fixed up
serially, S_start(j) = S*_end(j-1) + M_end(j-1) S_start(j-1).
"""
import numpy as np
from scipy.linalg import solve_triangular

from .recurrent import flatten_batch


def chunk_local_cumsum(g, C):
    """Inclusive cumsum along axis 0 that restarts every C rows (one sequence)."""
    g = np.asarray(g, dtype=np.float64)
    out = np.empty_like(g)
    for s in range(0, g.shape[0], C):
        out[s:s + C] = np.cumsum(g[s:s + C], axis=0)
    return out


def unit_lower_inverse(A_raw):
    """Exact (I + A_raw)^{-1} for strictly lower A_raw: triangular solve against I."""
    c = A_raw.shape[0]
    return solve_triangular(np.eye(c) + A_raw, np.eye(c), lower=True, unit_diagonal=True)


def wy_factors(A, bc, Kw, Vc):
    """WY form of one chunk: W = A diag(beta) Kw and U = A diag(beta) V, Kw the gated keys
    (diag(gamma) K, or K (.) exp(G) per channel).  FlashQLA announcement, the second step of the
    chunk-i forward; KDA source walk-through section 3.3 (u = A (v * beta), w = A (k * beta * exp(g)))."""
    return A @ (bc[:, None] * Kw), A @ (bc[:, None] * Vc)


def intra_scalar(Kc, Vc, bc, gcs, erase=True):
    """One chunk, scalar gate: gcs is the chunk-local cumsum.  Returns dict of intermediates."""
    c = Kc.shape[0]
    gamma = np.exp(gcs)
    diff = gcs[:, None] - gcs[None, :]
    lower = np.tril(np.ones((c, c), dtype=bool))
    Gamma = np.where(lower, np.exp(np.where(lower, diff, 0.0)), 0.0)
    A_raw = np.tril(bc[:, None] * (Gamma * (Kc @ Kc.T)), -1)
    A = unit_lower_inverse(A_raw) if erase else np.eye(c)
    W, U = wy_factors(A, bc, gamma[:, None] * Kc, Vc)
    if not erase:
        W = np.zeros_like(Kc)
    gC = gamma[-1]
    return dict(A_raw=A_raw, A=A, W=W, U=U, gamma=gamma, Gamma=Gamma,
                decay=np.full(Kc.shape[1], gC), kd=(gC / gamma)[:, None] * Kc)


def intra_channel(Qc, Kc, Vc, bc, Gcs, erase=True):
    """One chunk, per-channel gate: Gcs [c, D_k] chunk-local cumsum."""
    c = Kc.shape[0]
    lower = np.tril(np.ones((c, c), dtype=bool))
    # E[i, j, d] = exp(G_id - G_jd) for j <= i, else 0 (never exponentiate the upper half)
    diff = Gcs[:, None, :] - Gcs[None, :, :]
    E = np.where(lower[:, :, None], np.exp(np.where(lower[:, :, None], diff, 0.0)), 0.0)
    KK = np.einsum("id,jd,ijd->ij", Kc, Kc, E)
    QK = np.einsum("id,jd,ijd->ij", Qc, Kc, E)
    A_raw = np.tril(bc[:, None] * KK, -1)
    A = unit_lower_inverse(A_raw) if erase else np.eye(c)
    W, U = wy_factors(A, bc, Kc * np.exp(Gcs), Vc)
    if not erase:
        W = np.zeros_like(Kc)
    GC = Gcs[-1]
    return dict(A_raw=A_raw, A=A, W=W, U=U, Aqk=np.tril(QK), qg=Qc * np.exp(Gcs),
                decay=np.exp(GC), kd=Kc * np.exp(GC[None, :] - Gcs))


def chunk_records(Q, K, V, beta, g, C, gate, erase=True):
    """Split one (sequence, head) into chunks and compute the per-chunk intermediates."""
    L = K.shape[0]
    gcs = chunk_local_cumsum(g, C)
    recs = []
    for s in range(0, L, C):
        e = min(s + C, L)
        if gate == "scalar":
            r = intra_scalar(K[s:e], V[s:e], beta[s:e], gcs[s:e], erase)
        else:
            r = intra_channel(Q[s:e], K[s:e], V[s:e], beta[s:e], gcs[s:e], erase)
        r.update(start=s, end=e, g_cumsum=gcs[s:e])
        recs.append(r)
    return recs


def state_step(S, r):
    """One chunk of the inter-chunk recurrence: V' = U - W S, then S_next (read -> residual -> write)."""
    Vp = r["U"] - r["W"] @ S
    S_next = r["decay"][:, None] * S + r["kd"].T @ Vp
    return Vp, S_next


def chunk_output(Qc, Kc, S_enter, Vp, r, scale, gate):
    if gate == "scalar":
        inter = r["gamma"][:, None] * (Qc @ S_enter)
        intra = (r["Gamma"] * (Qc @ Kc.T)) @ Vp
    else:
        inter = r["qg"] @ S_enter
        intra = r["Aqk"] @ Vp
    return scale * (inter + intra)


def run_sequence(Q, K, V, beta, g, scale, S0, C, gate, erase=True):
    """Chunkwise forward of one (sequence, head).  Returns (O, S_final, records with V' and S_enter)."""
    recs = chunk_records(Q, K, V, beta, g, C, gate, erase)
    O = np.zeros((K.shape[0], V.shape[1]))
    S = S0.copy()
    for r in recs:
        s, e = r["start"], r["end"]
        r["S_enter"] = S  # stored before the update (entering state of this chunk)
        Vp, S = state_step(S, r)
        r["Vp"] = Vp
        O[s:e] = chunk_output(Q[s:e], K[s:e], r["S_enter"], Vp, r, scale, gate)
    return O, S, recs


def chunkwise_fwd(q, k, v, g, beta, scale, h0=None, cu_seqlens=None, chunk_size=64, gate="scalar",
                  erase=True, return_records=False):
    """Whole forward.  Shapes as oracle.recurrent.gdn_recurrent.  Returns (o, final[, records])."""
    qf, kf, vf, gf, bf, cu, bt = flatten_batch(q, k, v, g, beta, cu_seqlens)
    qf, kf, vf, gf, bf = (np.asarray(a, dtype=np.float64) for a in (qf, kf, vf, gf, bf))
    Ttot, H_qk, Dk = qf.shape
    H_v, Dv = vf.shape[1:]
    G = H_v // H_qk
    N = len(cu) - 1
    o = np.zeros((Ttot, H_v, Dv))
    fin = np.zeros((N, H_v, Dk, Dv))
    records = {}
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(H_v):
            hq = h // G
            S0 = np.zeros((Dk, Dv)) if h0 is None else np.asarray(h0, dtype=np.float64)[n, h]
            O, S, recs = run_sequence(qf[a:b, hq], kf[a:b, hq], vf[a:b, h], bf[a:b, h], gf[a:b, h],
                                      scale, S0, chunk_size, gate, erase)
            o[a:b, h] = O
            fin[n, h] = S
            if return_records:
                records[(n, h)] = recs
    if bt is not None:
        o = o.reshape(bt + (H_v, Dv))
    return (o, fin, records) if return_records else (o, fin)


# ----------------------------------------------------------------------------------------------
# Context parallelism inside one sequence (FlashQLA announcement, CP pre-process and fix-up)
# ----------------------------------------------------------------------------------------------

def cp_segment_maps(recs, seg_chunks):
    """Direct form: per segment, S* (from S = 0) and M (from M = I) after its last chunk.

    S*_{i+1} = T_i S*_i + b_i and M_{i+1} = T_i M_i with the chunk's affine step
    S -> decay * S + kd^T (U - W S), i.e. T_i = diag(decay) - kd^T W.
    """
    Dk = recs[0]["W"].shape[1]
    Dv = recs[0]["U"].shape[1]
    out = []
    for s0 in range(0, len(recs), seg_chunks):
        Sx = np.zeros((Dk, Dv))
        M = np.eye(Dk)
        for r in recs[s0:s0 + seg_chunks]:
            _, Sx = state_step(Sx, r)
            M = r["decay"][:, None] * M - r["kd"].T @ (r["W"] @ M)
        out.append((Sx, M))
    return out


def cp_segment_maps_xyz(K_seq, V_seq, beta_seq, g_seq, C, seg_chunks):
    """FlashQLA's rewritten CP pre-process (scalar gate), from the ungated inverse A'.

    A' = (I + strictLower(diag(beta) K K^T))^{-1};  X = -diag(beta) A'^T K;
    Y = gamma_C K S* - diag(gamma_C / gamma) V;  Z = K M;
    S* <- gamma_C S* + X^T Y;   M <- gamma_C (M + X^T Z).
    """
    gcs = chunk_local_cumsum(g_seq, C)
    L, Dk = K_seq.shape
    Dv = V_seq.shape[1]
    chunks = list(range(0, L, C))
    out = []
    for s0 in range(0, len(chunks), seg_chunks):
        Sx = np.zeros((Dk, Dv))
        M = np.eye(Dk)
        for st in chunks[s0:s0 + seg_chunks]:
            e = min(st + C, L)
            Kc, Vc, bc = K_seq[st:e], V_seq[st:e], beta_seq[st:e]
            gamma = np.exp(gcs[st:e])
            gC = gamma[-1]
            Ap = unit_lower_inverse(np.tril(bc[:, None] * (Kc @ Kc.T), -1))
            X = -(bc[:, None] * (Ap.T @ Kc))
            Y = gC * (Kc @ Sx) - (gC / gamma)[:, None] * Vc
            Z = Kc @ M
            Sx = gC * Sx + X.T @ Y
            M = gC * (M + X.T @ Z)
        out.append((Sx, M))
    return out


def cp_fixup(S0, maps):
    """Serial fix-up of segment start states: S_start(j) = S*_end(j-1) + M_end(j-1) S_start(j-1)."""
    starts = [S0]
    for Sx, M in maps[:-1]:
        starts.append(Sx + M @ starts[-1])
    Sx, M = maps[-1]
    return starts, Sx + M @ starts[-1]
