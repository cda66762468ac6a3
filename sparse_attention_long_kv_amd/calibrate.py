"""Host-side basis calibration for the indexer, and a selection-recall check.

JSSA article (rit.work blog, Joint Subspace Sparse Attention), "How JSSA
preserves token order": each KV head gets one low-dimensional space shared by
its queries and keys, chosen to preserve their pairwise scores rather than to
reconstruct the vectors; calibration accumulates query and key statistics
once per head and layer and takes the basis from the eigenvectors of a
matrix (a more elaborate objective gave no measurable gain).  "When the work
changes the architecture plan" adds that the calibration sequences should be
about as long as the longest context served.

The pages do not name the matrix.  This module reads the aim literally: with
one orthonormal basis P (d x r) and Pi = P P^T, the indexer's score of key k
for group-mean query q is q^T Pi k, so the squared score error over
independent queries and keys is

    E(Pi) = E[(q^T (I - Pi) k)^2] = tr((I - Pi) C_k (I - Pi) C_q),

C_q = E[q q^T] (second moment of group-mean queries) and C_k the covariance
of the keys (a key mean shifts every score of a query alike and does not
change the ranking).  E has no closed-form minimiser in general, so three
eigen-solutions are formed -- the top-r eigenvectors of C_k alone, of the
trace-normalised joint moment C_q / tr C_q + C_k / tr C_k, and of the
symmetrised product (C_q C_k + C_k C_q) / 2 (exact when C_q and C_k share
eigenvectors: E is then the sum of the dropped eigenvalue products) -- and
the one with the smallest relative error E(Pi) / tr(C_k C_q) on the
calibration statistics is kept.  Off the decode path; numpy, fp64.

``python -m sparse_attention_long_kv_amd.calibrate`` measures, on the GPU
through the library, how much of the exact top-M a random basis and the
calibrated basis recover on anisotropic synthetic keys and queries.
"""

import argparse
import json
import sys

import numpy as np


def score_moments(q_means, keys):
    """C_q (second moment of the group-mean queries [n, d]) and C_k
    (covariance of the keys [m, d]), fp64."""
    q = np.asarray(q_means, dtype=np.float64)
    k = np.asarray(keys, dtype=np.float64)
    c_q = q.T @ q / q.shape[0]
    kc = k - k.mean(axis=0, keepdims=True)
    c_k = kc.T @ kc / k.shape[0]
    return c_q, c_k


def score_error(P, c_q, c_k):
    """Relative squared score error E(Pi) / tr(C_k C_q) of the basis P [d, r]."""
    P = np.asarray(P, dtype=np.float64)
    a = np.eye(P.shape[0]) - P @ P.T
    return float(np.trace(a @ c_k @ a @ c_q) / np.trace(c_k @ c_q))


def _top_eigvecs(m, r):
    m = 0.5 * (m + m.T)
    w, v = np.linalg.eigh(m)
    order = np.argsort(w, kind="stable")[::-1][:r]
    P = v[:, order]
    # fixed signs: the largest-magnitude entry of each column is positive
    s = np.sign(P[np.argmax(np.abs(P), axis=0), np.arange(r)])
    return P * np.where(s == 0, 1.0, s)[None, :]


def basis_candidates(c_q, c_k, r):
    """The three eigen-solutions, by name."""
    return {
        "key_moments": _top_eigvecs(c_k, r),
        "joint_moments": _top_eigvecs(c_q / np.trace(c_q) + c_k / np.trace(c_k), r),
        "symmetrised_product": _top_eigvecs(c_q @ c_k + c_k @ c_q, r),
    }


def calibrate_basis(q_means, keys, r):
    """Basis P [d, r] (fp64, orthonormal columns) for one KV head from
    calibration queries (group means) and keys, and a report of every
    candidate's relative score error."""
    c_q, c_k = score_moments(q_means, keys)
    return basis_from_moments(c_q, c_k, r)


def basis_from_moments(c_q, c_k, r):
    """The candidate with the smallest relative score error, and the report."""
    cands = basis_candidates(c_q, c_k, r)
    errs = {name: score_error(P, c_q, c_k) for name, P in cands.items()}
    best = min(errs, key=lambda n: (errs[n], n))
    return cands[best], {"chosen": best, "relative_score_error": errs}


# ------------------------------------------------------------------ recall

def _exact_top(scores, M):
    """Top-M positions by score, ties to the lower position, ascending."""
    order = np.lexsort((np.arange(scores.shape[0]), -scores))
    return np.sort(order[:M])


def _measure(args):
    import torch
    import sparse_attention_long_kv_amd as sa
    from workloads import make_aniso_inputs, default_scale

    if not torch.cuda.is_available():
        raise SystemExit("the recall measurement runs the library on a GPU")
    sa.load()
    B, Hq, Hkv, d, r, N, M = args.B, args.Hq, args.Hkv, 128, 32, args.N, args.M
    G = Hq // Hkv
    inp = make_aniso_inputs(B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, r=r, seed=args.seed, device="cuda")
    sh = sa.make_shape(B, Hq, Hkv, d, r, N)
    cal, reports = [], []
    for h in range(Hkv):
        P, rep = calibrate_basis(inp.cal_q[h], inp.cal_k[h], r)
        cal.append(P)
        reports.append(rep)
    bases = {"random": inp.P_random,
             "calibrated": torch.from_numpy(np.ascontiguousarray(np.stack(cal),
                                                                 dtype=np.float32)).cuda()}
    K64 = inp.K.double().cpu().numpy()
    q64 = inp.q.double().cpu().numpy()
    tau = default_scale(d)
    ws = sa.alloc_workspace(sh, N, M)
    out = {"workload": "aniso: B%d Hq%d Hkv%d d%d N%d r%d M%d" % (B, Hq, Hkv, d, N, r, M),
           "calibration": reports}
    for name, P in bases.items():
        kp = torch.empty(B, Hkv, N, r, dtype=torch.uint8, device="cuda")
        sa.sparse_attn_project_keys(sh, inp.K, P, 0, N, kp)
        idx = torch.empty(B, Hkv, M, dtype=torch.int32, device="cuda")
        sa.sparse_attn_index_topm(sh, inp.q, P, kp, None, N, M, idx, ws)
        torch.cuda.synchronize()
        gi = idx.cpu().numpy()
        rec, cov, cov_best = [], [], []
        for b in range(B):
            for h in range(Hkv):
                qg = q64[b, h * G:(h + 1) * G]
                s = K64[b, h] @ qg.mean(axis=0)
                rec.append(np.intersect1d(_exact_top(s, M), gi[b, h]).size / M)
                z = tau * (K64[b, h] @ qg.T)                   # [N, G] logits
                p = np.exp(z - z.max(axis=0, keepdims=True))
                p /= p.sum(axis=0, keepdims=True)
                cov.append(p[gi[b, h]].sum(axis=0).mean())
                cov_best.append(np.sort(p, axis=0)[-M:].sum(axis=0).mean())
        out[name] = {"recall_of_exact_top_M": round(float(np.mean(rec)), 4),
                     "attention_mass_covered": round(float(np.mean(cov)), 4),
                     "attention_mass_of_best_M_per_head": round(float(np.mean(cov_best)), 4)}
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--B", type=int, default=4)
    ap.add_argument("--Hq", type=int, default=16)
    ap.add_argument("--Hkv", type=int, default=4)
    ap.add_argument("--N", type=int, default=32768)
    ap.add_argument("--M", type=int, default=1024)
    ap.add_argument("--seed", type=int, default=0)
    args = ap.parse_args(argv)
    print(json.dumps(_measure(args)))
    return 0


if __name__ == "__main__":
    sys.exit(main())
