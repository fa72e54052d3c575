"""Error bounds and exact references used to pin the oracle and to judge the
GPU results.  Everything here is float64 / integer numpy and independent of
both the oracle and the HIP library."""
import numpy as np

U32 = 2.0 ** -24


def gamma(n, u=U32):
    return n * u / (1.0 - n * u)


def linear_magnitude(x, A, B, idx, slot_rank, scale, y0, y_col_offset=0):
    """M[t, c] = |y0| + |scale| * sum_j (sum_i |x_i A_ji|) |B_nj| in float64,
    the magnitude an a-priori rounding bound for one token's delta uses."""
    M = np.abs(np.asarray(y0, np.float64)).copy()
    T = x.shape[0]
    L = A[0].shape[0]
    ax = np.abs(np.asarray(x, np.float64))
    for t in range(T):
        s = int(idx[t])
        if s < 0 or s >= L or slot_rank[s] <= 0:
            continue
        r = int(slot_rank[s])
        off = y_col_offset
        for a, b in zip(A, B):
            sa = ax[t] @ np.abs(a[s, :r, :].astype(np.float64)).T        # [r]
            M[t, off:off + b.shape[1]] += abs(float(scale[s])) * (
                np.abs(b[s, :, :r].astype(np.float64)) @ sa)
            off += b.shape[1]
    return M


def linear_exact_f64(x, A, B, idx, slot_rank, scale, y0, y_col_offset=0):
    """Dense float64 reference with a different association from the oracle:
    W_s = scale_s * B_s[:, :r] @ A_s[:r, :] first, then y += W_s x."""
    y = np.asarray(y0, np.float64).copy()
    L = A[0].shape[0]
    for t in range(x.shape[0]):
        s = int(idx[t])
        if s < 0 or s >= L or slot_rank[s] <= 0:
            continue
        r = int(slot_rank[s])
        off = y_col_offset
        for a, b in zip(A, B):
            W = float(scale[s]) * (b[s, :, :r].astype(np.float64) @ a[s, :r, :].astype(np.float64))
            y[t, off:off + b.shape[1]] += W @ np.asarray(x[t], np.float64)
            off += b.shape[1]
    return y


def linear_exact_int(x, A, B, idx, slot_rank, scale, y0):
    """Exact integer reference for integer-valued inputs (scale must be an
    integer too): int64 matrix products."""
    y = np.asarray(y0).astype(np.int64).copy()
    L = A[0].shape[0]
    xi = np.asarray(x).astype(np.int64)
    for t in range(x.shape[0]):
        s = int(idx[t])
        if s < 0 or s >= L or slot_rank[s] <= 0:
            continue
        r = int(slot_rank[s])
        off = 0
        for a, b in zip(A, B):
            ai = a[s, :r, :].astype(np.int64)
            bi = b[s, :, :r].astype(np.int64)
            y[t, off:off + b.shape[1]] += int(scale[s]) * (bi @ (ai @ xi[t]))
            off += b.shape[1]
    return y


def linear_exact_int_by_slot(x, A, B, idx, slot_rank, scale, y0):
    """Exact reference for integer-valued inputs at large sizes: the tokens of
    each slot as one float64 matrix product (BLAS).  Every product and partial
    sum is an integer far below 2^53, so float64 holds it exactly whatever the
    summation order; the result equals linear_exact_int's."""
    y = np.asarray(y0, np.float64).copy()
    L = A[0].shape[0]
    idx = np.asarray(idx)
    xf = np.asarray(x, np.float64)
    for s in range(L):
        r = int(slot_rank[s])
        toks = np.nonzero(idx == s)[0]
        if r <= 0 or toks.size == 0:
            continue
        off = 0
        for a, b in zip(A, B):
            h = xf[toks] @ a[s, :r, :].astype(np.float64).T              # [n, r]
            y[toks, off:off + b.shape[1]] += float(scale[s]) * (h @ b[s, :, :r].astype(np.float64).T)
            off += b.shape[1]
    return y


def moe_exact_f64(kind, y0, x, A, B, topk_ids, topk_w, idx, slot_rank, scale, E, reduce_k=False):
    """Dense float64 fused-MoE LoRA reference (W = coef * B @ A, then W x)."""
    T, k = topk_ids.shape
    L, E_a, R, K = A[0].shape
    E_b = B[0].shape[1]
    y = np.asarray(y0, np.float64).copy()
    for t in range(T):
        s = int(idx[t])
        if s < 0 or s >= L or slot_rank[s] <= 0:
            continue
        r = int(slot_rank[s])
        for j in range(k):
            p = t * k + j
            e = int(topk_ids[t, j])
            if e < 0 or e >= E:
                continue
            ea = 0 if E_a == 1 else e
            eb = 0 if E_b == 1 else e
            xr = np.asarray(x[t if kind == 0 else p], np.float64)
            row = t if (kind == 1 and reduce_k) else p
            coef = float(scale[s])
            if kind == 1 and topk_w is not None:
                coef *= float(topk_w[t, j])
            off = 0
            for a, b in zip(A, B):
                W = coef * (b[s, eb, :, :r].astype(np.float64) @ a[s, ea, :r, :].astype(np.float64))
                y[row, off:off + b.shape[2]] += W @ xr
                off += b.shape[2]
    return y


def moe_magnitude(kind, y0, x, A, B, topk_ids, topk_w, idx, slot_rank, scale, E, reduce_k=False):
    T, k = topk_ids.shape
    L, E_a, R, K = A[0].shape
    E_b = B[0].shape[1]
    M = np.abs(np.asarray(y0, np.float64)).copy()
    for t in range(T):
        s = int(idx[t])
        if s < 0 or s >= L or slot_rank[s] <= 0:
            continue
        r = int(slot_rank[s])
        for j in range(k):
            p = t * k + j
            e = int(topk_ids[t, j])
            if e < 0 or e >= E:
                continue
            ea = 0 if E_a == 1 else e
            eb = 0 if E_b == 1 else e
            xr = np.abs(np.asarray(x[t if kind == 0 else p], np.float64))
            row = t if (kind == 1 and reduce_k) else p
            coef = abs(float(scale[s]))
            if kind == 1 and topk_w is not None:
                coef *= abs(float(topk_w[t, j]))
            off = 0
            for a, b in zip(A, B):
                sa = np.abs(a[s, ea, :r, :].astype(np.float64)) @ xr
                M[row, off:off + b.shape[2]] += coef * (np.abs(b[s, eb, :, :r].astype(np.float64)) @ sa)
                off += b.shape[2]
    return M


def fp32_bound(M, K, R, extra=4):
    """Order-independent a-priori bound on |fp32 result - exact| for results
    built from a length-K and a length-R dot product plus scale and add."""
    return 2.0 * gamma(K + R + extra) * M


def check_bf16_tolerance(g, r, abs_tol=2e-2, rel_tol=1e-2, block_rows=1024):
    """bf16 GPU output g vs fp32 oracle r: max abs error <= abs_tol and
    max abs error / max |r| <= rel_tol (normwise).  Returns (err, rel).
    Works through row blocks, so full-size outputs need little extra memory."""
    g = np.asarray(g)
    r = np.asarray(r)
    assert g.shape == r.shape, (g.shape, r.shape)
    if g.size == 0:
        return 0.0, 0.0
    g2 = g.reshape(g.shape[0], -1) if g.ndim > 1 else g.reshape(-1, 1)
    r2 = r.reshape(r.shape[0], -1) if r.ndim > 1 else r.reshape(-1, 1)
    err = ref = 0.0
    for lo in range(0, g2.shape[0], block_rows):
        gb = g2[lo:lo + block_rows].astype(np.float64)
        rb = r2[lo:lo + block_rows].astype(np.float64)
        err = max(err, float(np.max(np.abs(gb - rb))))
        ref = max(ref, float(np.max(np.abs(rb))))
    rel = err / ref if ref > 0 else err
    assert err <= abs_tol, f"max abs err {err} > {abs_tol}"
    assert rel <= rel_tol, f"normwise rel err {rel} > {rel_tol}"
    return err, rel
