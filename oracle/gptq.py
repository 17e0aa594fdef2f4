"""O9: the GPTQ quantizer, producing the packed format of O1 (plain numpy, fp64).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Page: [Lab5] "Lab 5: Gemma4 端到端推理优化", section "从 RTN 到 GPTQ":
  - objective: min_Q ||X W^T - X Q^T||_F^2 over the calibration activations X [N][d_in];
  - Hessian H = (2/N) X^T X; a column that is zero in every calibration row (diag H = 0) is a
    dead column: its weights are set to zero and H[i][i] to 1; then damping H += lambda I with
    lambda = alpha * mean(diag H);
  - H^-1 = U^T U with U upper triangular; columns are quantized in order; after column i is
    rounded to q_i, e_i = (w_i - q_i) / U_ii and W[:, i:] -= e_i U[i, i:];
  - the predicted loss L_pred = 1/2 sum_i ||w_i - q_i||^2 / U_ii^2.
The page builds H, factors it and propagates the error in fp32; this reference does all of that in
fp64 (numpy, with numpy's Cholesky and inverse as library steps) so that it is the more exact of
the two.

Readings (the page leaves them open):
  - groups: a group's scale (and zero point) is computed by O1's rule from the current, already
    error-updated weights of the group's columns when the first column of the group is reached,
    and kept for the rest of the group; per-row packing (group_size 0) uses one group per row;
  - a column's code is decided as O1 decides it, on the weight rounded to fp32:
    code = clip(rint(w / s + z), 0, 15) in fp32 operations (a zero scale gives the zero code);
    q = s (code - z);
  - columns are taken in their natural order; alpha defaults to 0.01;
  - padded columns carry the zero code (O1's format).
"""
import numpy as np

from . import ASYM, SYM, bf16_to_f32, k_pad, n_groups, pack


def hessian(x_bits, d_in=None):
    """H = (2/N) X^T X in fp64 from bf16 activations X [N][ldx] (first d_in columns)."""
    x = bf16_to_f32(np.asarray(x_bits, dtype=np.uint16)).astype(np.float64)
    if d_in is not None:
        x = x[:, :d_in]
    return (2.0 / x.shape[0]) * (x.T @ x)


def prepare(h, w, alpha=0.01):
    """Dead columns and damping.  Returns (H_damped, W with dead columns zeroed, lambda, dead)."""
    h = np.array(h, dtype=np.float64)
    w = np.array(w, dtype=np.float64)
    dead = np.diag(h) == 0.0
    w[:, dead] = 0.0
    idx = np.flatnonzero(dead)
    h[idx, idx] = 1.0
    lam = alpha * float(np.mean(np.diag(h)))
    h[np.diag_indices_from(h)] += lam
    return h, w, lam, dead


def inverse_factor(h):
    """U upper triangular with H^-1 = U^T U."""
    hinv = np.linalg.inv(h)
    hinv = 0.5 * (hinv + hinv.T)
    return np.linalg.cholesky(hinv).T


def _code(w_col, s_bits, z_bits, mode):
    """O1's code decision for one column, in fp32 operations (a zero scale gives the zero code,
    which O1 stores as 8 for symmetric and 0 for asymmetric groups). Also returns the value
    before rounding, v = w / s + z (fp32), whose distance to the nearest half-integer says how
    close the decision was."""
    s = bf16_to_f32(s_bits)
    z = bf16_to_f32(z_bits) if mode == ASYM else np.full(s.shape, 8.0, np.float32)
    v = np.asarray(w_col).astype(np.float32)
    nz = s != 0.0
    t = np.divide(v, s, out=np.zeros_like(v), where=nz)
    t = t + z
    pre = t.copy()
    t = np.clip(np.rint(t), 0.0, 15.0)
    code = np.where(nz, t, z).astype(np.uint8)
    return code, s.astype(np.float64), z.astype(np.float64), pre


def _group_stats(block, span, s_bits, mode):
    """The fp32 values that O1's scale and zero decisions round (the same fp32 operations, on the
    group padded with zeros): symmetric max|w| / 7; asymmetric (max - min) / 15 and -min / s with
    the stored bf16 s. Diagnostics only: they say how close each decision was to a rounding tie."""
    blk = np.zeros((block.shape[0], span), dtype=np.float32)
    blk[:, :block.shape[1]] = block
    if mode == SYM:
        s32 = np.max(np.abs(blk), axis=1).astype(np.float32) / np.float32(7.0)
        return s32, np.zeros_like(s32)
    mx = np.max(blk, axis=1).astype(np.float32)
    mn = np.min(blk, axis=1).astype(np.float32)
    s32 = (mx - mn) / np.float32(15.0)
    s = bf16_to_f32(s_bits)
    zp = np.divide(-mn, s, out=np.zeros_like(mn), where=s != 0.0)
    return s32.astype(np.float32), zp.astype(np.float32)


def gptq(w, x_bits, group_size, mode, alpha=0.01, d_in=None):
    """GPTQ of an fp32 weight [d_out][d_in] with bf16 calibration activations [N][>= d_in].
    Returns dict(qweight, scales, zeros (None for SYM), L_pred, H (damped), U, lam, dead,
    w (the weight after the dead-column step), codes [d_out][k_pad], v [d_out][d_in]: each
    column's value w / s + z before rounding, fp32; s_pre, z_pre [d_out][n_groups]: each group's
    fp32 scale before its bf16 rounding and (asymmetric) -min / s before its rounding to an
    integer -- O1's statistics of the updated weights at the group's first column)."""
    w = np.asarray(w, dtype=np.float32)
    d_out = w.shape[0]
    d_in = w.shape[1] if d_in is None else d_in
    h, W, lam, dead = prepare(hessian(x_bits, d_in), w[:, :d_in], alpha)
    U = inverse_factor(h)
    W0 = W.copy()
    kp, ng = k_pad(d_in, group_size), n_groups(d_in, group_size)
    span = kp // ng
    codes = np.zeros((d_out, kp), dtype=np.uint8)
    vpre = np.zeros((d_out, d_in), dtype=np.float32)
    s_pre = np.zeros((d_out, ng), dtype=np.float32)
    z_pre = np.zeros((d_out, ng), dtype=np.float32)
    scales = np.zeros((d_out, ng), dtype=np.uint16)
    zeros = np.zeros((d_out, ng), dtype=np.uint16) if mode == ASYM else None
    L = 0.0
    s_bits = z_bits = None
    for i in range(d_in):
        G = i // span
        if i % span == 0:
            block = W[:, G * span:min((G + 1) * span, d_in)].astype(np.float32)
            _, sc, zr = pack(block, group_size if group_size else 0, mode)
            s_bits = sc[:, 0]
            z_bits = zr[:, 0] if mode == ASYM else None
            scales[:, G] = s_bits
            if mode == ASYM:
                zeros[:, G] = z_bits
            s_pre[:, G], z_pre[:, G] = _group_stats(block, span, s_bits, mode)
        code, s, z, vpre[:, i] = _code(W[:, i], s_bits, z_bits, mode)
        q = s * (code.astype(np.float64) - z)
        codes[:, i] = code
        err = W[:, i] - q
        L += 0.5 * float(np.sum(err * err)) / (U[i, i] * U[i, i])
        e = err / U[i, i]
        W[:, i:] -= np.outer(e, U[i, i:])
    # pads: the code O1 gives a 0.0 of the group
    for G in range(ng):
        lo, hi = max(G * span, d_in), (G + 1) * span
        if lo < hi:
            zc, _, _, _ = _code(np.zeros(d_out), scales[:, G],
                                zeros[:, G] if mode == ASYM else None, mode)
            codes[:, lo:hi] = zc[:, None]
    qweight = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return dict(qweight=qweight, scales=scales, zeros=zeros, L_pred=L, H=h, U=U, lam=lam,
                dead=dead, w=W0, codes=codes, v=vpre, s_pre=s_pre, z_pre=z_pre)


__all__ = ["hessian", "prepare", "inverse_factor", "gptq", "SYM", "ASYM"]
