"""Dense brute-force attention in numpy (tiny shapes only): an independent
formulation used to pin the oracle.

Rotation is written with complex numbers (pair (x, y) -> (x + iy) * e^{i angle}),
GQA by materialising repeated KV heads, the mask as an explicit boolean matrix and
the softmax as a dense row operation.  Shares no code with ``oracle/``.
"""
import numpy as np


def rotate(x, pos, theta, n_rot):
    """x [..., S, H, d] float64, pos [..., S]: rotate pairs t < n_rot."""
    d = x.shape[-1]
    z = x[..., 0::2] + 1j * x[..., 1::2]
    t = np.arange(d // 2)
    freq = np.where(t < n_rot, np.power(float(theta), -2.0 * t / d), 0.0)
    ph = np.exp(1j * pos[..., :, None, None].astype(np.float64) * freq)
    z = z * ph
    y = np.empty_like(x)
    y[..., 0::2] = z.real
    y[..., 1::2] = z.imag
    return y


def mask_matrix(S, window):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    m = j <= i
    if window > 0:
        m &= (i - j) < window
    return m


def probabilities(q, k, pos, window, theta, n_rot):
    """Dense softmax weights [B, Hq, S(query), S(key)], 0 where masked."""
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    qr = rotate(q, pos, theta, n_rot)
    kr = np.repeat(rotate(k, pos, theta, n_rot), G, axis=2)
    sc = np.einsum("bihd,bjhd->bhij", qr, kr) / np.sqrt(d)
    m = mask_matrix(S, window)
    sc = np.where(m[None, None], sc, -np.inf)
    sc = sc - sc.max(axis=-1, keepdims=True)
    w = np.exp(sc)
    return w / w.sum(axis=-1, keepdims=True)


def attention(q, k, v, pos, window, theta, n_rot):
    """q [B,S,Hq,d], k/v [B,S,Hkv,d] float64; returns [B,S,Hq,d]."""
    G = q.shape[2] // k.shape[2]
    w = probabilities(q, k, pos, window, theta, n_rot)
    vv = np.repeat(v, G, axis=2)
    return np.einsum("bhij,bjhd->bihd", w, vv)


def vision_attention(q, k, v, pos2, theta, lengths=None):
    """Bidirectional attention with 2D RoPE: half c of the head dims is an
    ordinary RoPE of dim d/2 driven by position component c; keys past
    lengths[b] are masked and those rows are zero.  pos2 [B,S,2]."""
    B, S, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    half = d // 2

    def rot2(x):
        y = np.empty_like(x)
        y[..., :half] = rotate(x[..., :half], pos2[..., 0], theta, half // 2)
        y[..., half:] = rotate(x[..., half:], pos2[..., 1], theta, half // 2)
        return y

    n = np.full(B, S) if lengths is None else np.clip(np.asarray(lengths), 0, S)
    qr = rot2(np.nan_to_num(q))
    kr = np.repeat(rot2(np.nan_to_num(k)), G, axis=2)
    vv = np.repeat(np.nan_to_num(v), G, axis=2)
    sc = np.einsum("bihd,bjhd->bhij", qr, kr) / np.sqrt(d)
    valid = np.arange(S)[None, :] < n[:, None]  # [B, S] keys
    sc = np.where(valid[:, None, None, :], sc, -np.inf)
    out = np.zeros((B, S, Hq, d))
    for b in range(B):
        if n[b] == 0:
            continue
        s = sc[b, :, :n[b]]
        s = s - s.max(axis=-1, keepdims=True)
        w = np.exp(s)
        w = w / w.sum(axis=-1, keepdims=True)
        out[b, :n[b]] = np.einsum("hij,jhd->ihd", w[:, :n[b]], vv[b])
    return out
