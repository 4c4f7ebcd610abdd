"""fp64 CPU oracle for DeepSeek-V2 Multi-head Latent Attention (MLA).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module.  The product path (the HIP
library and its Python binding) never imports it, and it imports nothing from
the product path: the two share no code.  Inputs come from the seeded
generators in `mla_synth` (random draws and input rounding only).

What it computes is the definition on the page "DeepSeek-V2 paper summary"
(7shi.hateblo.jp):
  * section 2.1.1: standard MHA, q = W^Q h, k = W^K h, v = W^V h;
  * section 2.1.2: joint KV compression, c_KV = W^DKV h, k = W^UK c_KV, v = W^UV c_KV;
  * section 2.1.3: decoupled RoPE, a multi-head rope query and ONE shared rope key;
  * App. C "Full Formulas of MLA": the whole layer, the causal sum over j = 1..t,
    the softmax scale 1/sqrt(d_h + d_e), the output projection W^O, and the
    statement that only c^kv_t and the rope key are cached.
It is written in the explicit, un-absorbed form (keys and values rebuilt per
head from the cached latent).  The absorbed form (W^UK folded into the query,
W^UV applied after the softmax; App. C, associativity of matrix products) is a
second function used only to cross-check and for sampled checks at large sizes.

Readings where the page leaves a step open (each is also listed in the design
notes):
  * RoPE: rotation of interleaved pairs (x_2k, x_2k+1) by angle m * base^(-2k/d_e),
    m = the 0-based token position (the pages only say "apply the RoPE matrix" and
    cite RoFormer).  Angles are formed in fp64.
  * The rope key has no head index (section 2.1.3 calls it shared); the per-head
    query/key order [rope ; content] does not change a dot product, so the cache
    entry is laid out [c_KV | k_R].
  * "No query compression" (App. B.1, V2-Lite) means c^q := h.
  * Softmax over j in [1, t], inclusive of the token itself.
  * YaRN (section 3.1.4: s = 40, alpha = 1, beta = 32, sqrt(t) = 0.0707 ln s + 1; the page
    cites the YaRN paper for the rest), when the layer sets rope_scale s > 1: the "NTK-by-parts"
    frequencies of that paper, measured against the original context length L.  For the pair
    k with frequency theta_k, wavelength lambda_k = 2 pi / theta_k and r_k = L / lambda_k
    rotations over L; gamma_k = 0 for r_k < alpha, 1 for r_k > beta, linear in between; the
    pair rotates by (1 - gamma_k) theta_k / s + gamma_k theta_k.  Short wavelengths keep their
    frequency, long ones are interpolated by s.  The logits are multiplied by
    t = (0.0707 ln s + 1)^2 (the page names only sqrt(t) and says it adjusts the attention
    entropy; applying it to the logit scale is the plain reading).  Both rope parts (q^R and the
    shared k^R) use the same frequencies.
  * RMSNorm after the compressed latents (section 3.1.2), when the weights carry the gains
    g_cq / g_ckv: c^q <- g_cq * c^q / sqrt(mean(c^q^2) + eps) before W_UQ and W_QR, and
    c^KV <- g_ckv * c^KV / sqrt(mean(c^KV^2) + eps) before it is cached (so W_UK and W_UV see
    the normalised latent); the rope key is not normalised.  The page also multiplies
    "additional scaling factors" at the width bottlenecks without giving them; a constant factor
    folds into the gains, so none is modelled apart from them.

Parity pins: every function here is checked by tests that do not reuse this
code (a scalar brute-force layer on tiny inputs, reduction to textbook MHA, a
library attention routine, the RoPE closed form via complex numbers,
absorbed == un-absorbed, softmax/convexity invariants, causality, relative
position invariance and the cache element count).
"""
from __future__ import annotations

import numpy as np


# ----------------------------------------------------------------------------- RoPE
def yarn_frequencies(theta, s: float, orig_ctx: int, alpha: float, beta: float) -> np.ndarray:
    """YaRN frequencies (NTK-by-parts) of the plain RoPE frequencies theta (fp64), scale s,
    original context length orig_ctx, ramp bounds alpha < beta (see the module notes)."""
    theta = np.asarray(theta, dtype=np.float64)
    wavelength = 2.0 * np.pi / theta
    rotations = np.float64(orig_ctx) / wavelength
    gamma = np.clip((rotations - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / s + gamma * theta


def yarn_of(dims):
    """The layer's YaRN parameters (s, L, alpha, beta), or None for plain RoPE."""
    s = float(getattr(dims, "rope_scale", 1.0))
    if s <= 1.0:
        return None
    return s, int(dims.rope_orig_ctx), float(dims.yarn_alpha), float(dims.yarn_beta)


def rope_angles(pos, d_hr: int, base: float, yarn=None) -> np.ndarray:
    """Angles m * theta_k, theta_k = base^(-2k/d_hr), k = 0..d_hr/2-1, in fp64 (with yarn =
    (s, L, alpha, beta): the YaRN frequencies of those).
    pos: int or int array [...]; returns [..., d_hr/2]."""
    k = np.arange(d_hr // 2, dtype=np.float64)
    theta = np.power(np.float64(base), -2.0 * k / d_hr)
    if yarn is not None:
        theta = yarn_frequencies(theta, *yarn)
    return np.asarray(pos, dtype=np.float64)[..., None] * theta


def apply_rope(x: np.ndarray, pos, base: float, yarn=None) -> np.ndarray:
    """Rotate interleaved pairs of the last axis of x by the angles of position(s) pos.
    x: [..., d_hr]; pos broadcastable to x.shape[:-1]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = rope_angles(pos, d, base, yarn)
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


# ----------------------------------------------------------------------------- projections
def _w(W: dict, name: str) -> np.ndarray:
    return np.asarray(W[name], dtype=np.float64)


def rms_norm(x: np.ndarray, gain, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: gain * x / sqrt(mean(x^2) + eps), fp64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gain, dtype=np.float64)


def query(W: dict, dims, h: np.ndarray, pos) -> tuple:
    """App. C query side.  h [n, d] -> (q^C [n, n_h, d_h], rotated q^R [n, n_h, d_hr]).
    c^q = W_DQ h (or h itself without query compression); q^C = W_UQ c^q;
    q^R = RoPE(W_QR c^q), head i = rows [i*d_hr, (i+1)*d_hr)."""
    h = np.asarray(h, dtype=np.float64)
    cq = h @ _w(W, "W_DQ").T if dims.d_cq > 0 else h
    if dims.d_cq > 0 and "g_cq" in W:
        cq = rms_norm(cq, _w(W, "g_cq"), dims.rms_eps)
    qc = (cq @ _w(W, "W_UQ").T).reshape(h.shape[0], dims.n_h, dims.d_h)
    qr = (cq @ _w(W, "W_QR").T).reshape(h.shape[0], dims.n_h, dims.d_hr)
    qr = apply_rope(qr, np.asarray(pos)[:, None], dims.rope_base, yarn_of(dims))
    return qc, qr


def latent_entries(W: dict, dims, h: np.ndarray, pos) -> np.ndarray:
    """App. C cached vectors: [c^kv_t | RoPE(W_KR h_t)] per token, [n, d_c + d_hr]."""
    h = np.asarray(h, dtype=np.float64)
    ckv = h @ _w(W, "W_DKV").T
    if "g_ckv" in W:
        ckv = rms_norm(ckv, _w(W, "g_ckv"), dims.rms_eps)
    kr = apply_rope(h @ _w(W, "W_KR").T, np.asarray(pos), dims.rope_base, yarn_of(dims))
    return np.concatenate([ckv, kr], axis=1)


def softmax_rows(s: np.ndarray):
    """Max-subtracted softmax over the last axis, fp64; also returns the log-sum-exp."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = np.sum(e, axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


# ----------------------------------------------------------------------------- attention
def yarn_logit_factor(dims) -> float:
    """YaRN's attention-entropy factor t = (c ln s + 1)^2 (section 3.1.4: c = 0.0707), 1 without YaRN."""
    if yarn_of(dims) is None:
        return 1.0
    root_t = np.float64(dims.yarn_mscale) * np.log(np.float64(dims.rope_scale)) + 1.0
    return float(root_t * root_t)


def softmax_scale(dims) -> float:
    """The logit scale of App. C, 1/sqrt(d_h + d_e) (times YaRN's t), unless the layer fixes
    another value."""
    if dims.softmax_scale > 0:
        return float(dims.softmax_scale)
    return yarn_logit_factor(dims) * _app_c_scale(dims)


def _app_c_scale(dims) -> float:
    return 1.0 / np.sqrt(np.float64(dims.d_h + dims.d_hr))


def attend_unabsorbed(W: dict, dims, qc, qr, cache: np.ndarray, kv_len) -> tuple:
    """Un-absorbed attention of queries against cached entries.
    qc [n, n_h, d_h], qr [n, n_h, d_hr]; cache [L, d_c + d_hr] ([c_KV | k_R]);
    kv_len [n]: query r attends to cache rows 0..kv_len[r]-1.
    Per head i: K^C_i = c W_UK_i^T, V_i = c W_UV_i^T (W_UK_i = rows [i*d_h,(i+1)*d_h)),
    s = scale * ([q^C_i ; q^R_i] . [K^C_i ; k_R]), o_i = softmax(s) V_i.
    Returns o [n, n_h, d_h] and lse [n, n_h]."""
    cache = np.asarray(cache, dtype=np.float64)
    c, kr = cache[:, : dims.d_c], cache[:, dims.d_c:]
    n = qc.shape[0]
    L = cache.shape[0]
    kv_len = np.asarray(kv_len)
    mask = np.arange(L)[None, :] < kv_len[:, None]  # [n, L]
    WUK, WUV = _w(W, "W_UK"), _w(W, "W_UV")
    o = np.zeros((n, dims.n_h, dims.d_h))
    lse = np.zeros((n, dims.n_h))
    for i in range(dims.n_h):
        rows = slice(i * dims.d_h, (i + 1) * dims.d_h)
        Kc = c @ WUK[rows].T  # [L, d_h]
        V = c @ WUV[rows].T  # [L, d_h]
        s = (qc[:, i, :] @ Kc.T + qr[:, i, :] @ kr.T) * softmax_scale(dims)  # [n, L]
        s = np.where(mask, s, -np.inf)
        p, lse[:, i] = softmax_rows(s)
        o[:, i, :] = p @ V
    return o, lse


def latent_attention(qcat: np.ndarray, cache: np.ndarray, kv_len, scale: float, d_c: int) -> tuple:
    """The attention step of the absorbed form (App. C, associativity): every head attends over
    the cached entries themselves.  qcat [n, n_h, d_c + d_hr] = [q_hat_i | q^R_i] per head,
    cache [L, d_c + d_hr] = [c_KV | k_R]; query r sees rows 0..kv_len[r]-1.
    s_ij = scale * (qcat_i . entry_j), o_hat_i = sum_j softmax_j(s_ij) c_KV,j.
    Returns o_hat [n, n_h, d_c] and lse [n, n_h]."""
    cache = np.asarray(cache, dtype=np.float64)
    qcat = np.asarray(qcat, dtype=np.float64)
    L = cache.shape[0]
    kv_len = np.asarray(kv_len)
    mask = np.arange(L)[None, :] < kv_len[:, None]
    s = (qcat @ cache.T) * scale  # [n, n_h, L]
    s = np.where(mask[:, None, :], s, -np.inf)
    p, lse = softmax_rows(s)
    return p @ cache[:, :d_c], lse


def absorb_query(W: dict, dims, qc, qr) -> np.ndarray:
    """[q_hat_i | q^R_i] per head with q_hat_i = W_UK_i^T q^C_i (App. C, associativity)."""
    WUK = _w(W, "W_UK").reshape(dims.n_h, dims.d_h, dims.d_c)
    qhat = np.einsum("nik,ikc->nic", qc, WUK)  # [n, n_h, d_c]
    return np.concatenate([qhat, qr], axis=-1)


def attend_absorbed(W: dict, dims, qc, qr, cache: np.ndarray, kv_len) -> tuple:
    """Absorbed form (App. C, associativity): q_hat_i = W_UK_i^T q^C_i in R^{d_c},
    s = scale * (q_hat_i . c_j + q^R_i . k_R,j), o_hat_i = sum_j p_ij c_j,
    o_i = W_UV_i o_hat_i.  Same outputs as attend_unabsorbed in exact arithmetic."""
    ohat, lse = latent_attention(absorb_query(W, dims, qc, qr), cache, kv_len, softmax_scale(dims), dims.d_c)
    WUV = _w(W, "W_UV").reshape(dims.n_h, dims.d_h, dims.d_c)
    o = np.einsum("nic,idc->nid", ohat, WUV)
    return o, lse


def output(W: dict, dims, o: np.ndarray) -> np.ndarray:
    """u_t = W_O [o_t,1 ; ... ; o_t,n_h]  (App. C)."""
    return o.reshape(o.shape[0], dims.n_h * dims.d_h) @ _w(W, "W_O").T


# ----------------------------------------------------------------------------- whole layer
def mla_prefill(W: dict, dims, h: np.ndarray, start_pos: int = 0, prefix_cache=None,
                absorbed: bool = False, rope_positions=None) -> dict:
    """One sequence through the MLA layer, causal (App. C, sum over j <= t).
    h [T, d] are the tokens at sequence indices start_pos..start_pos+T-1; prefix_cache
    [start_pos, d_c+d_hr] holds the entries of the earlier tokens (None when start_pos == 0).
    rope_positions (optional, [T]) overrides the RoPE positions of the new tokens (default:
    their sequence indices); causality always follows the sequence index.
    Returns u [T, d], o [T, n_h, d_h], cache [start_pos+T, d_c+d_hr], lse [T, n_h], q^C, q^R."""
    h = np.asarray(h, dtype=np.float64)
    T = h.shape[0]
    idx = np.arange(start_pos, start_pos + T)
    pos = idx if rope_positions is None else np.asarray(rope_positions)
    new = latent_entries(W, dims, h, pos)
    cache = new if prefix_cache is None else np.concatenate([np.asarray(prefix_cache, np.float64), new])
    assert cache.shape[0] == start_pos + T
    qc, qr = query(W, dims, h, pos)
    attend = attend_absorbed if absorbed else attend_unabsorbed
    o, lse = attend(W, dims, qc, qr, cache, idx + 1)
    return {"u": output(W, dims, o), "o": o, "cache": cache, "lse": lse, "qc": qc, "qr": qr}


def mla_decode(W: dict, dims, h_new: np.ndarray, caches, absorbed: bool = False) -> dict:
    """One decode step for a batch.  h_new [B, d]; caches[b] = [L_b, d_c+d_hr] entries of
    the L_b tokens already cached (positions 0..L_b-1).  The new token sits at position
    L_b, its entry is appended, and it attends over all L_b + 1 tokens.
    Returns u [B, d], o [B, n_h, d_h], entry [B, d_c+d_hr], lse [B, n_h]."""
    h_new = np.asarray(h_new, dtype=np.float64)
    B = h_new.shape[0]
    u = np.zeros((B, dims.d_model))
    o = np.zeros((B, dims.n_h, dims.d_h))
    lse = np.zeros((B, dims.n_h))
    entry = np.zeros((B, dims.entry))
    attend = attend_absorbed if absorbed else attend_unabsorbed
    for b in range(B):
        L = int(np.asarray(caches[b]).shape[0])
        e = latent_entries(W, dims, h_new[b:b + 1], np.array([L]))
        full = np.concatenate([np.asarray(caches[b], np.float64).reshape(L, dims.entry), e])
        qc, qr = query(W, dims, h_new[b:b + 1], np.array([L]))
        ob, lb = attend(W, dims, qc, qr, full, np.array([L + 1]))
        o[b], lse[b], entry[b] = ob[0], lb[0], e[0]
        u[b] = output(W, dims, ob)[0]
    return {"u": u, "o": o, "entry": entry, "lse": lse}


def mla_prefill_rows(W: dict, dims, h: np.ndarray, rows, cache=None) -> dict:
    """mla_prefill's u, o and lse for the query rows `rows` of one sequence only (positions
    0..T-1), through the absorbed form so that no per-head key/value rebuild over all T tokens is
    needed (sampled checks at large sizes).  cache: the sequence's entries if already known."""
    h = np.asarray(h)
    rows = np.asarray(rows)
    if cache is None:
        cache = latent_entries(W, dims, h[: int(rows.max()) + 1], np.arange(int(rows.max()) + 1))
    qc, qr = query(W, dims, h[rows], rows)
    o, lse = attend_absorbed(W, dims, qc, qr, cache, rows + 1)
    return {"u": output(W, dims, o), "o": o, "lse": lse}


def cache_values_per_token(dims) -> int:
    """Values cached per token per layer by MLA: d_c + d_hr (App. C boxed vectors)."""
    return dims.d_c + dims.d_hr


def mha_cache_values_per_token(dims) -> int:
    """Values cached per token per layer by standard MHA: keys and values, 2 n_h d_h."""
    return 2 * dims.n_h * dims.d_h
