"""Host reference for the inverse-conductivity demonstration (test helper):
the loss and its gradient with respect to the node conductivities, from the
oracle's PCG and adjoint and an explicit Jacobian of the assembly, written
independently of the package's PyTorch assembly.

A(kappa) on an N x N node grid (spacing h = 1/(N+1), Dirichlet): for each
interior face (i, j) the entries a_ij = a_ji = -(k_i + k_j)/2; a_ii = k_i times
the number of boundary faces of node i plus (k_i + k_j)/2 over its interior
faces. Sources: Gaussian bumps of width 0.1 times h^2 at (0.25, 0.25),
(0.75, 0.25), (0.25, 0.75), (0.75, 0.75).
"""
import numpy as np

import oracle


def grid(N):
    h = 1.0 / (N + 1)
    faces = []
    for y in range(N):                    # horizontal faces, then vertical, in node order
        for x in range(N - 1):
            faces.append((y * N + x, y * N + x + 1))
    for y in range(N - 1):
        for x in range(N):
            faces.append((y * N + x, (y + 1) * N + x))
    faces = np.array(faces, dtype=np.int64)
    n = N * N
    nb = np.zeros(n)
    for i in range(n):
        y, x = divmod(i, N)
        nb[i] = (x == 0) + (x == N - 1) + (y == 0) + (y == N - 1)
    xs = (np.arange(n) % N + 1) * h
    ys = (np.arange(n) // N + 1) * h
    return {"N": N, "n": n, "h": h, "faces": faces, "nb": nb, "x": xs, "y": ys}


def coo(G, kappa):
    n, fc = G["n"], G["faces"]
    i, j = fc[:, 0], fc[:, 1]
    face = (kappa[i] + kappa[j]) / 2
    diag = kappa * G["nb"]
    for f in range(fc.shape[0]):
        diag[i[f]] += face[f]
        diag[j[f]] += face[f]
    rows = np.concatenate([np.arange(n), i, j])
    cols = np.concatenate([np.arange(n), j, i])
    return rows, cols, np.concatenate([diag, -face, -face])


def true_kappa(G):
    return 1.0 + 0.5 * np.sin(2 * np.pi * G["x"]) * np.sin(np.pi * G["y"])


def sources(G, S=4):
    centres = [(0.25, 0.25), (0.75, 0.25), (0.25, 0.75), (0.75, 0.75)][:S]
    return np.stack([G["h"] ** 2 * np.exp(-((G["x"] - a) ** 2 + (G["y"] - b) ** 2) / (2 * 0.01))
                     for a, b in centres])


def loss_and_grad(G, kappa, F, U_obs, tol=1e-12, maxit=20000):
    """L = sum_s ||u_s - u_obs,s||^2 / sum_s ||u_obs,s||^2 and dL/dkappa."""
    rows, cols, vals = coo(G, kappa)
    ref = oracle.coo_to_csr(G["n"], rows, cols, vals)
    nrm = float((U_obs * U_obs).sum())
    L = 0.0
    g_coo = np.zeros(vals.shape[0])
    for f, uo in zip(F, U_obs):
        u, *_ = oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], f, tol, maxit)
        res = u - uo
        L += float(res @ res) / nrm
        _, gv, *_ = oracle.adjoint(ref["row_ptr"], ref["col"], ref["vals"], u, 2 * res / nrm, tol,
                                   maxit)
        g_coo += gv[ref["slot"]]
    # chain through the assembly: d a_ii/d k_i = nb_i + (faces of i)/2,
    # d a_ii/d k_j = 1/2 for a face (i, j), d a_ij/d k_i = d a_ij/d k_j = -1/2
    n, fc = G["n"], G["faces"]
    nf = fc.shape[0]
    dk = g_coo[:n] * G["nb"]
    for f in range(nf):
        i, j = fc[f]
        gd = 0.5 * (g_coo[i] + g_coo[j])          # both diagonals hold (k_i + k_j)/2
        go = -0.5 * (g_coo[n + f] + g_coo[n + nf + f])
        dk[i] += gd + go
        dk[j] += gd + go
    return L, dk


def observations(G, F, tol=1e-12):
    rows, cols, vals = coo(G, true_kappa(G))
    ref = oracle.coo_to_csr(G["n"], rows, cols, vals)
    return np.stack([oracle.pcg(ref["row_ptr"], ref["col"], ref["vals"], f, tol, 20000)[0]
                     for f in F])
