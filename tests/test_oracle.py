"""Pins of the fp64 oracle against things other than itself (CPU only).

Each check names what fixes the expected value:
  * a scalar brute-force of the App. C formulas ("Full Formulas of MLA", DeepSeek-V2
    paper summary, 7shi.hateblo.jp) on tiny inputs, written with Python loops;
  * the special case that turns MLA into textbook multi-head attention (section 2.1.1),
    checked against a triple-loop MHA and against torch's fp64 attention routine;
  * the RoPE rotation checked against complex multiplication (RoFormer's closed form);
  * absorbed == un-absorbed (App. C: associativity of matrix products);
  * softmax rows sum to one, outputs are convex combinations, closed forms for q = 0 and
    for a one-token context;
  * causality, relative-position invariance of the scores, decode == prefill row;
  * the cache element count per token (App. C boxed vectors; section 2.1.4's GQA with
    2.25 groups).
"""
import math

import numpy as np
import pytest
import torch

import mla_synth as S
import oracle.mla_oracle as O

TINY_BF = S.Dims(d_model=6, n_h=2, d_h=3, d_c=4, d_cq=5, d_hr=4, dtype=S.F32, rope_base=7.0)


def _rand_weights(dims, seed, std=0.5):
    rng = np.random.default_rng(seed)
    return {k: rng.standard_normal(s) * std for k, s in dims.weight_shapes().items()}


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


# ----------------------------------------------------------------------------- brute force
def _brute_layer(W, dims, h, positions):
    """Scalar loops over App. C, term by term, for every token t of one sequence."""
    T, d = len(h), dims.d_model
    nh, dh, dc, dr = dims.n_h, dims.d_h, dims.d_c, dims.d_hr

    def mv(M, x):  # y_r = sum_c M[r][c] x[c]
        return [sum(M[r][c] * x[c] for c in range(len(x))) for r in range(len(M))]

    def rot(x, m):  # RoFormer: pair (2k, 2k+1) rotated by m * base^(-2k/len)
        y = list(x)
        for k in range(len(x) // 2):
            a = m * dims.rope_base ** (-2.0 * k / len(x))
            y[2 * k] = x[2 * k] * math.cos(a) - x[2 * k + 1] * math.sin(a)
            y[2 * k + 1] = x[2 * k] * math.sin(a) + x[2 * k + 1] * math.cos(a)
        return y

    q, qt, k, kt, v = [], [], [], [], []
    for t in range(T):
        cq = mv(W["W_DQ"], h[t]) if dims.d_cq else list(h[t])
        q.append(mv(W["W_UQ"], cq))
        qt.append(mv(W["W_QR"], cq))
        qt[t] = sum((rot(qt[t][i * dr:(i + 1) * dr], positions[t]) for i in range(nh)), [])
        ckv = mv(W["W_DKV"], h[t])
        k.append(mv(W["W_UK"], ckv))
        kt.append(rot(mv(W["W_KR"], h[t]), positions[t]))
        v.append(mv(W["W_UV"], ckv))
    u = []
    for t in range(T):
        o = []
        for i in range(nh):
            sc = []
            for j in range(t + 1):
                s = sum(qt[t][i * dr + e] * kt[j][e] for e in range(dr))
                s += sum(q[t][i * dh + e] * k[j][i * dh + e] for e in range(dh))
                sc.append(s / math.sqrt(dh + dr))
            mx = max(sc)
            ex = [math.exp(s - mx) for s in sc]
            z = sum(ex)
            for e in range(dh):
                o.append(sum(ex[j] / z * v[j][i * dh + e] for j in range(t + 1)))
        u.append(mv(W["W_O"], o))
    return np.array(u)


@pytest.mark.parametrize("d_cq", [5, 0])
def test_bruteforce_scalar_layer(d_cq):
    dims = TINY_BF if d_cq else S.Dims(d_model=6, n_h=2, d_h=3, d_c=4, d_cq=0, d_hr=4,
                                       dtype=S.F32, rope_base=7.0)
    W = _rand_weights(dims, 11)
    h = np.random.default_rng(12).standard_normal((5, dims.d_model))
    ref = _brute_layer({k: v.tolist() for k, v in W.items()}, dims, h.tolist(), list(range(5)))
    got = O.mla_prefill(W, dims, h)["u"]
    assert _rel(got, ref) < 1e-12


# ----------------------------------------------------------------------------- textbook MHA
def _reduce_to_mha(seed):
    """W_QR = W_KR = 0, d_c = d, W_DKV = I: MLA is MHA with W^Q = W_UQ W_DQ,
    W^K = W_UK, W^V = W_UV."""
    dims = S.Dims(d_model=8, n_h=3, d_h=4, d_c=8, d_cq=6, d_hr=2, dtype=S.F32)
    W = _rand_weights(dims, seed)
    W["W_QR"][:] = 0
    W["W_KR"][:] = 0
    W["W_DKV"] = np.eye(8)
    return dims, W


def _mha_triple_loop(WQ, WK, WV, WO, h, n_h, d_h, scale):
    T = len(h)
    q = h @ WQ.T
    k = h @ WK.T
    v = h @ WV.T
    o = np.zeros((T, n_h * d_h))
    for t in range(T):
        for i in range(n_h):
            sl = slice(i * d_h, (i + 1) * d_h)
            s = np.array([np.dot(q[t, sl], k[j, sl]) * scale for j in range(t + 1)])
            p = np.exp(s - s.max())
            p /= p.sum()
            for j in range(t + 1):
                o[t, sl] += p[j] * v[j, sl]
    return o @ WO.T, o


def test_reduces_to_textbook_mha():
    dims, W = _reduce_to_mha(3)
    h = np.random.default_rng(4).standard_normal((7, dims.d_model))
    ref_u, ref_o = _mha_triple_loop(W["W_UQ"] @ W["W_DQ"], W["W_UK"], W["W_UV"], W["W_O"], h,
                                    dims.n_h, dims.d_h, 1 / math.sqrt(dims.d_h + dims.d_hr))
    got = O.mla_prefill(W, dims, h)
    assert _rel(got["u"], ref_u) < 1e-12
    assert _rel(got["o"].reshape(7, -1), ref_o) < 1e-12


def test_attention_matches_torch_sdpa_fp64():
    """Full MLA (rope parts on): per-head q, k, v built from the definition feed torch's
    fp64 scaled_dot_product_attention (causal); o must agree."""
    dims = S.Dims(d_model=16, n_h=4, d_h=8, d_c=8, d_cq=12, d_hr=4, dtype=S.F32)
    W = _rand_weights(dims, 5)
    T = 9
    h = np.random.default_rng(6).standard_normal((T, dims.d_model))
    pos = np.arange(T)
    cq = h @ W["W_DQ"].T
    qc = (cq @ W["W_UQ"].T).reshape(T, 4, 8)
    qr = O.apply_rope((cq @ W["W_QR"].T).reshape(T, 4, 4), pos[:, None], dims.rope_base)
    ckv = h @ W["W_DKV"].T
    kc = (ckv @ W["W_UK"].T).reshape(T, 4, 8)
    kr = O.apply_rope(h @ W["W_KR"].T, pos, dims.rope_base)
    v = (ckv @ W["W_UV"].T).reshape(T, 4, 8)
    Q = torch.from_numpy(np.concatenate([qr, qc], -1)).permute(1, 0, 2)  # rope part first
    K = torch.from_numpy(np.concatenate([np.broadcast_to(kr[:, None, :], (T, 4, 4)), kc], -1)).permute(1, 0, 2)
    V = torch.from_numpy(v).permute(1, 0, 2)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True,
                                                           scale=1 / math.sqrt(12)).permute(1, 0, 2)
    got = O.mla_prefill(W, dims, h)["o"]
    assert _rel(got, ref.numpy()) < 1e-12


# ----------------------------------------------------------------------------- RoPE
def test_rope_complex_closed_form():
    rng = np.random.default_rng(7)
    d, base = 16, 10000.0
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 17, 4096, 131072])
    z = x[:, 0::2] + 1j * x[:, 1::2]
    theta = np.exp(-(2.0 * np.arange(d // 2) / d) * np.log(base))
    zr = z * np.exp(1j * pos[:, None] * theta[None, :])
    ref = np.empty_like(x)
    ref[:, 0::2], ref[:, 1::2] = zr.real, zr.imag
    # theta computed two ways differs by an ulp; at m = 131072 that is ~3e-11 rad
    assert _rel(O.apply_rope(x, pos, base), ref) < 1e-10
    assert _rel(O.apply_rope(x[:3], pos[:3], base), ref[:3]) < 1e-14
    # one pair, angle 1 rad: (1, 0) -> (cos 1, sin 1)
    assert np.allclose(O.apply_rope(np.array([1.0, 0.0]), 1, 3.0), [math.cos(1), math.sin(1)], atol=1e-15)


def test_rope_identity_norm_and_relative():
    rng = np.random.default_rng(8)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    assert np.array_equal(O.apply_rope(q, 0, 1e4), q)
    for m in (1, 77, 131072):
        assert abs(np.linalg.norm(O.apply_rope(q, m, 1e4)) - np.linalg.norm(q)) < 1e-12
    m, n = 33, 5
    ref = np.dot(O.apply_rope(q, m, 1e4), O.apply_rope(k, n, 1e4))
    for delta in (1, 1000, 100000):
        got = np.dot(O.apply_rope(q, m + delta, 1e4), O.apply_rope(k, n + delta, 1e4))
        assert abs(got - ref) < 1e-10 * max(1.0, abs(ref))


def test_position_shift_leaves_layer_unchanged():
    W = _rand_weights(S.TINY, 9, std=0.3)
    h = np.random.default_rng(10).standard_normal((12, S.TINY.d_model))
    ref = O.mla_prefill(W, S.TINY, h)["u"]
    for delta in (1, 1000, 100000):
        got = O.mla_prefill(W, S.TINY, h, rope_positions=np.arange(12) + delta)["u"]
        assert _rel(got, ref) < 1e-10


# ----------------------------------------------------------------------------- absorbed form
@pytest.mark.parametrize("dims,L", [(S.TINY, 20), (S.V2_LITE, 40), (S.V2, 24)])
def test_absorbed_equals_unabsorbed(dims, L):
    W = S.make_weights(dims, std=0.05)
    h = S.hidden_history(dims, 0, L, "rmsnorm")
    a = O.mla_prefill(W, dims, h)
    b = O.mla_prefill(W, dims, h, absorbed=True)
    assert _rel(b["o"], a["o"]) < 1e-10
    assert _rel(b["u"], a["u"]) < 1e-10
    assert _rel(b["lse"], a["lse"]) < 1e-10


# ----------------------------------------------------------------------------- softmax
def test_softmax_rows_sum_to_one_and_overflow():
    rng = np.random.default_rng(13)
    s = rng.standard_normal((6, 50)) * np.array([[1e-3], [1.0], [30.0], [1e3], [1e5], [0.0]])
    p, lse = O.softmax_rows(s)
    assert np.all(np.isfinite(p)) and np.all(p >= 0)
    assert np.max(np.abs(p.sum(-1) - 1)) < 1e-12
    # lse closed form on rows that cannot overflow
    ref = np.log(np.sum(np.exp(s[:3]), axis=-1))
    assert np.max(np.abs(lse[:3] - ref)) < 1e-12
    # uniform logits: p = 1/L
    assert np.max(np.abs(p[5] - 1 / 50)) < 1e-15


def test_outputs_are_convex_combinations_of_values():
    dims = S.TINY
    W = _rand_weights(dims, 14, std=0.4)
    h = np.random.default_rng(15).standard_normal((10, dims.d_model))
    r = O.mla_prefill(W, dims, h)
    V = (r["cache"][:, :dims.d_c] @ W["W_UV"].T).reshape(10, dims.n_h, dims.d_h)
    for t in range(10):
        lo, hi = V[: t + 1].min(0), V[: t + 1].max(0)
        assert np.all(r["o"][t] >= lo - 1e-12) and np.all(r["o"][t] <= hi + 1e-12)


def test_zero_query_gives_running_mean_and_first_token_gives_own_value():
    dims = S.TINY
    W = _rand_weights(dims, 16, std=0.4)
    h = np.random.default_rng(17).standard_normal((8, dims.d_model))
    # ctx = 1: the first token attends only to itself, o_0 = W_UV c_0
    r = O.mla_prefill(W, dims, h)
    own = (r["cache"][0, :dims.d_c] @ W["W_UV"].T).reshape(dims.n_h, dims.d_h)
    assert _rel(r["o"][0], own) < 1e-13
    # q = 0 (W_UQ = W_QR = 0): uniform weights, o_t = mean_{j<=t} V_j
    W0 = dict(W)
    W0["W_UQ"] = np.zeros_like(W["W_UQ"])
    W0["W_QR"] = np.zeros_like(W["W_QR"])
    r0 = O.mla_prefill(W0, dims, h)
    V = (r0["cache"][:, :dims.d_c] @ W["W_UV"].T).reshape(8, dims.n_h, dims.d_h)
    mean = np.cumsum(V, 0) / np.arange(1, 9)[:, None, None]
    assert _rel(r0["o"], mean) < 1e-13


# ----------------------------------------------------------------------------- causality etc.
def test_causality_bit_identical():
    dims = S.TINY
    W = _rand_weights(dims, 18, std=0.3)
    h = np.random.default_rng(19).standard_normal((12, dims.d_model))
    a = O.mla_prefill(W, dims, h)
    h2 = h.copy()
    h2[7:] = np.random.default_rng(20).standard_normal((5, dims.d_model))
    b = O.mla_prefill(W, dims, h2)
    assert np.array_equal(a["u"][:7], b["u"][:7])
    assert not np.allclose(a["u"][7:], b["u"][7:])


@pytest.mark.parametrize("dims", [S.TINY, S.V2_LITE])
def test_decode_step_equals_prefill_row(dims):
    W = S.make_weights(dims, std=0.05)
    T = 9
    h = S.hidden_history(dims, 0, T, "rmsnorm")
    pre = O.mla_prefill(W, dims, h)
    for t in (0, 4, 8):
        dec = O.mla_decode(W, dims, h[t:t + 1], [pre["cache"][:t]])
        assert _rel(dec["u"][0], pre["u"][t]) < 1e-12
        assert _rel(dec["entry"][0], pre["cache"][t]) < 1e-14


def test_prefill_rows_equals_prefill():
    dims = S.TINY
    W = _rand_weights(dims, 24, std=0.3)
    h = np.random.default_rng(25).standard_normal((11, dims.d_model))
    whole = O.mla_prefill(W, dims, h)
    rows = np.array([0, 3, 10])
    sub = O.mla_prefill_rows(W, dims, h, rows)
    assert _rel(sub["u"], whole["u"][rows]) < 1e-12
    assert _rel(sub["o"], whole["o"][rows]) < 1e-12
    sub2 = O.mla_prefill_rows(W, dims, h, rows, cache=whole["cache"])
    assert _rel(sub2["u"], whole["u"][rows]) < 1e-12


def test_chunked_prefill_equals_whole():
    dims = S.TINY
    W = _rand_weights(dims, 21, std=0.3)
    h = np.random.default_rng(22).standard_normal((10, dims.d_model))
    whole = O.mla_prefill(W, dims, h)
    first = O.mla_prefill(W, dims, h[:6])
    rest = O.mla_prefill(W, dims, h[6:], start_pos=6, prefix_cache=first["cache"])
    assert _rel(np.concatenate([first["u"], rest["u"]]), whole["u"]) < 1e-12


# ----------------------------------------------------------------------------- cache size
def test_cache_element_count():
    assert O.cache_values_per_token(S.V2) == 576
    assert O.mha_cache_values_per_token(S.V2) == 32768
    # GQA with 2.25 groups caches 2 * 2.25 * d_h values: the same as MLA (section 2.1.4)
    assert O.cache_values_per_token(S.V2) == 2 * 2.25 * S.V2.d_h
    assert O.cache_values_per_token(S.V2_LITE) == 2 * 2.25 * S.V2_LITE.d_h
    assert abs(O.cache_values_per_token(S.V2) / O.mha_cache_values_per_token(S.V2) - 0.017578125) < 1e-12
    assert abs(O.cache_values_per_token(S.V2_LITE) / O.mha_cache_values_per_token(S.V2_LITE) - 0.140625) < 1e-12
    W = S.make_weights(S.TINY)
    r = O.mla_prefill(W, S.TINY, S.hidden_history(S.TINY, 0, 3, "normal002"))
    assert r["cache"].shape == (3, S.TINY.d_c + S.TINY.d_hr)


# ----------------------------------------------------------------------------- generator
def test_bf16_rounding_matches_torch_cast():
    x = np.random.default_rng(23).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 65504.0]  # ties and a large value
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(S.round_bf16(x), ref)
    assert np.array_equal(S.bits_to_f32(S.bf16_bits(ref)), ref)
