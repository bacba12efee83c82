"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: a value
worked by hand from the recurrence, a closed form, an invariant, a number the
pages print, or an independent library routine.  Together they are meant to
catch a dropped term, a wrong sign or index, or a transposed operand anywhere
in the oracle.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

RNG = np.random.default_rng(1234)


def f32_bits_to_bf16_torch(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def identity_taps(C):
    """Conv taps (0, 0, 0, 1): the conv passes the current token through."""
    w = np.zeros((C, 4), dtype=np.float32)
    w[:, 3] = 1.0
    return f32_bits_to_bf16_torch(w)


def pack_x(q, k, v):
    """[T,H,K],[T,H,K],[T,H,V] float -> x bf16 bits [T, C] in q|k|v head-major order."""
    T = q.shape[0]
    x = np.concatenate([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], axis=1)
    return f32_bits_to_bf16_torch(x)


# ---------------------------------------------------------------- helpers ----

def test_bf16_round_matches_torch_rne():
    """The oracle's double->bf16 rounding agrees with torch's float->bf16 RNE on
    float inputs, including exact ties, subnormals and overflow."""
    vals = np.concatenate([
        RNG.standard_normal(4000).astype(np.float32) * np.float32(10.0) ** RNG.integers(-40, 38, 4000),
        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 1e-40, -3e-39,
                  3.39e38, 3.4e38, 0.0, -0.0], dtype=np.float32),
    ]).astype(np.float32)
    got = oracle.bf16_round(vals.astype(np.float64))
    want = f32_bits_to_bf16_torch(vals)
    assert np.array_equal(got, want)


def test_bf16_round_no_double_rounding():
    """A double just above a bf16 tie must round up, which float-first rounding gets wrong."""
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40   # float rounds to the exact tie, then to even (down)
    assert oracle.bf16_round(np.array([x]))[0] == 0x3F81


# ----------------------------------------------------- hand-worked steps ----

def _full_path_single_token(case, precision):
    """Run a hand case through oracle_prefill (conv taps identity, no norm)."""
    K, V = case["K"], case["V"]
    pool = oracle.Pool(1, 2, 1, K, V, oracle.SSM_F32)
    pool.ssm()[0, 1, 0] = np.array(case["S0"], dtype=np.float32)
    q = np.array(case["q"], dtype=np.float32)[None, None]
    k = np.array(case["k"], dtype=np.float32)[None, None]
    v = np.array(case["v"], dtype=np.float32)[None, None]
    alpha = np.array(case["alpha"], dtype=np.float32).reshape(1, 1, K)
    beta = np.array([[case["beta"]]], dtype=np.float32)
    out, err = oracle.prefill(pool, 0, [0, 1], [1], pack_x(q, k, v), identity_taps(2 * K + V),
                              alpha, oracle.ALPHA_PER_CHANNEL, beta, has_initial_state=[1],
                              scale=case["scale"], flags=0, precision=precision)
    assert err == 0
    return out, pool


@pytest.mark.parametrize("name", ["rank1_step_2x2.json", "rank1_step_3x2.json"])
@pytest.mark.parametrize("precision", ["f64", "f32"])
def test_hand_worked_step(golden_dir, name, precision):
    case = json.load(open(os.path.join(golden_dir, name)))
    out, pool = _full_path_single_token(case, precision)
    assert np.array_equal(pool.ssm()[0, 1, 0], np.array(case["S1"], dtype=np.float32))
    assert np.array_equal(oracle.bf16_widen(out[0, 0]), np.array(case["o"]))
    # bare recurrence agrees as well
    o, S = oracle.recurrence_head(np.array([case["q"]]), np.array([case["k"]]),
                                  np.array([case["v"]]), np.array([case["alpha"]]),
                                  np.array([case["beta"]]), np.array(case["S0"], dtype=np.float64),
                                  scale=case["scale"], precision=precision)
    assert np.array_equal(S, np.array(case["S1"], dtype=np.float64))
    assert np.array_equal(o[0], np.array(case["o"]))


def test_key_is_l2_normalised_after_conv():
    """Raw key (3, 4) is normalised to (0.6, 0.8) (eps 1e-6 inside the sqrt)."""
    K = V = 2
    pool = oracle.Pool(1, 2, 1, K, V, oracle.SSM_F32)
    q = np.array([[[1.0, 0.0]]], dtype=np.float32)
    k = np.array([[[3.0, 4.0]]], dtype=np.float32)
    v = np.array([[[1.0, 2.0]]], dtype=np.float32)
    alpha = np.ones((1, 1, K), dtype=np.float32)
    beta = np.ones((1, 1), dtype=np.float32)
    out, err, oe, se = oracle.prefill(pool, 0, [0, 1], [1], pack_x(q, k, v), identity_taps(6),
                                      alpha, oracle.ALPHA_PER_CHANNEL, beta, has_initial_state=[0],
                                      flags=oracle.L2NORM_K, exact=True)
    khat = np.array([3.0, 4.0]) / np.sqrt(25.0 + 1e-6)
    # zero start, beta = 1: S = v khat^T, o = S q = v * khat[0]
    np.testing.assert_allclose(se[0, 0], np.outer([1.0, 2.0], khat), rtol=1e-14)
    np.testing.assert_allclose(oe[0, 0], np.array([1.0, 2.0]) * khat[0], rtol=1e-14)


# ------------------------------------------------------ closed forms ----

def _rand_head(T, K, V, alpha_per_channel=True, unit_k=True):
    q = RNG.standard_normal((T, K))
    k = RNG.standard_normal((T, K))
    if unit_k:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = RNG.standard_normal((T, V))
    alpha = 1 / (1 + np.exp(-(RNG.standard_normal((T, K) if alpha_per_channel else (T,)) + 3)))
    beta = 1 / (1 + np.exp(-RNG.standard_normal(T)))
    S0 = 0.25 * RNG.standard_normal((V, K))
    return q, k, v, alpha, beta, S0


def test_beta0_alpha1_leaves_state_unchanged_bitexact():
    """beta = 0 and alpha = 1: the state is untouched (bit-exact through the pool)."""
    H, K, V, T = 2, 16, 16, 70
    pool = oracle.Pool(1, 4, H, K, V, oracle.SSM_F32)
    pool.ssm()[:] = (0.25 * RNG.standard_normal(pool.ssm().shape)).astype(np.float32)
    pool.conv()[:] = f32_bits_to_bf16_torch(RNG.standard_normal(pool.conv().shape))
    before = pool.ssm()[0, 2].copy()
    g = wl.generator(7)
    inp = wl.projected_inputs(g, T, H, K, V, wl.ALPHA_PER_CHANNEL)
    alpha = np.ones((T, H, K), dtype=np.float32)
    beta = np.zeros((T, H), dtype=np.float32)
    w = wl.bf16_bits(wl.conv_weights(g, pool.channels))
    out, err = oracle.prefill(pool, 0, [0, T], [2], wl.bf16_bits(inp["x"]), w, alpha,
                              oracle.ALPHA_PER_CHANNEL, beta, has_initial_state=[1])
    assert err == 0
    assert np.array_equal(pool.ssm()[0, 2], before)


def test_beta0_pure_decay_closed_form():
    """beta = 0: S_T = S0 Diag(prod_t alpha_t)."""
    T, K, V = 50, 8, 6
    q, k, v, alpha, beta, S0 = _rand_head(T, K, V)
    o, S = oracle.recurrence_head(q, k, v, alpha, np.zeros(T), S0)
    np.testing.assert_allclose(S, S0 * np.prod(alpha, axis=0)[None, :], rtol=1e-12)
    # outputs from the decayed state
    gam = np.cumprod(alpha, axis=0)
    np.testing.assert_allclose(o, np.einsum("rk,tk,tk->tr", S0, gam, q), rtol=1e-10, atol=1e-14)


def test_delta_rule_exact_write():
    """beta = 1 and a unit key: the updated state maps k to v exactly."""
    K, V = 16, 12
    q, k, v, alpha, beta, S0 = _rand_head(1, K, V)
    _, S = oracle.recurrence_head(q, k, v, alpha, np.ones(1), S0)
    np.testing.assert_allclose(S @ k[0], v[0], rtol=1e-12, atol=1e-12)


def test_orthonormal_keys_store_columns():
    """Keys e_1..e_K, alpha = beta = 1, zero start: column i of S is v_i."""
    K = V = 8
    k = np.eye(K)
    v = RNG.standard_normal((K, V))
    q = RNG.standard_normal((K, K))
    _, S = oracle.recurrence_head(q, k, v, np.ones((K, K)), np.ones(K), np.zeros((V, K)))
    assert np.array_equal(S, v.T)


def test_affine_in_initial_state():
    """The map S0 -> (o, S_T) is affine: f(A) + f(B) - f(0) = f(A + B)."""
    T, K, V = 40, 8, 8
    q, k, v, alpha, beta, A = _rand_head(T, K, V)
    B = 0.25 * RNG.standard_normal((V, K))
    fa = oracle.recurrence_head(q, k, v, alpha, beta, A)
    fb = oracle.recurrence_head(q, k, v, alpha, beta, B)
    f0 = oracle.recurrence_head(q, k, v, alpha, beta, np.zeros((V, K)))
    fab = oracle.recurrence_head(q, k, v, alpha, beta, A + B)
    for i in range(2):
        np.testing.assert_allclose(fa[i] + fb[i] - f0[i], fab[i], rtol=1e-9, atol=1e-12)


def test_value_rows_are_independent():
    """Permuting the value channels permutes the rows of S and of o (bit-exact)."""
    T, K, V = 30, 8, 10
    q, k, v, alpha, beta, S0 = _rand_head(T, K, V)
    perm = RNG.permutation(V)
    o1, S1 = oracle.recurrence_head(q, k, v, alpha, beta, S0)
    o2, S2 = oracle.recurrence_head(q, k, v[:, perm], alpha, beta, S0[perm])
    assert np.array_equal(S1[perm], S2)
    assert np.array_equal(o1[:, perm], o2)


def test_gdn_equals_kda_with_broadcast_alpha():
    """A per-head decay equals the per-channel decay with that value in every channel."""
    cfg = wl.TINY
    g = wl.generator(11)
    T = 100
    inp = wl.projected_inputs(g, T, cfg.heads, cfg.head_k, cfg.head_v, wl.ALPHA_PER_HEAD)
    w = wl.bf16_bits(wl.conv_weights(g, cfg.channels))
    a_head = inp["alpha"].numpy()
    a_chan = np.repeat(a_head[:, :, None], cfg.head_k, axis=2)
    res = []
    for a, mode in ((a_head, oracle.ALPHA_PER_HEAD), (a_chan, oracle.ALPHA_PER_CHANNEL)):
        pool = oracle.Pool(1, 3, cfg.heads, cfg.head_k, cfg.head_v, oracle.SSM_F32)
        out, err = oracle.prefill(pool, 0, [0, T], [1], wl.bf16_bits(inp["x"]), w, a, mode,
                                  inp["beta"].numpy(), has_initial_state=[0])
        res.append((out, pool.ssm_bytes.copy(), pool.conv_bytes.copy()))
    for i in range(3):
        assert np.array_equal(res[0][i], res[1][i])


# ------------------------------------------------------------- the conv ----

def test_conv_impulse_response_and_tap_order():
    """With beta = 1, alpha = 1 and k = q = 1 the delta rule overwrites the state
    with the conv output of the v channel, so o_t is the conv output itself.
    An impulse at t = 0 gives the taps in reverse order: w3, w2, w1, w0, 0."""
    C = 3   # H = 1, K = V = 1 -> channels q, k, v
    taps = np.array([[0, 0, 0, 1], [0, 0, 0, 1], [0.5, -0.25, 2.0, 1.5]], dtype=np.float32)
    T = 6
    q = np.ones((T, 1, 1)); k = np.ones((T, 1, 1)); v = np.zeros((T, 1, 1)); v[0] = 1.0
    pool = oracle.Pool(1, 2, 1, 1, 1, oracle.SSM_F32)
    out, err, oe, se = oracle.prefill(
        pool, 0, [0, T], [1], pack_x(q, k, v), f32_bits_to_bf16_torch(taps),
        np.ones((T, 1), np.float32), oracle.ALPHA_PER_HEAD, np.ones((T, 1), np.float32),
        has_initial_state=[0], flags=0, exact=True)
    np.testing.assert_array_equal(oe[:, 0, 0], [1.5, 2.0, -0.25, 0.5, 0.0, 0.0])


def test_conv_uses_warm_rows_oldest_first():
    """Warm conv rows (r0, r1, r2) = (1, 2, 4) and x = 8 on the v channel give
    y = w0*1 + w1*2 + w2*4 + w3*8 for the first token."""
    taps = np.array([[0, 0, 0, 1], [0, 0, 0, 1], [1.0, 0.0625, 2.0 ** -8, 2.0 ** -12]], np.float32)
    pool = oracle.Pool(1, 2, 1, 1, 1, oracle.SSM_F32)
    conv = pool.conv()
    conv[0, 1, :, 2] = f32_bits_to_bf16_torch([1.0, 2.0, 4.0])
    conv[0, 1, :, 0] = f32_bits_to_bf16_torch([0.0, 0.0, 0.0])
    conv[0, 1, :, 1] = f32_bits_to_bf16_torch([0.0, 0.0, 0.0])
    x = pack_x(np.ones((1, 1, 1)), np.ones((1, 1, 1)), np.full((1, 1, 1), 8.0))
    out, err, oe, se = oracle.prefill(pool, 0, [0, 1], [1], x, f32_bits_to_bf16_torch(taps),
                                      np.ones((1, 1), np.float32), oracle.ALPHA_PER_HEAD,
                                      np.ones((1, 1), np.float32), has_initial_state=[1],
                                      flags=0, exact=True)
    assert oe[0, 0, 0] == 1.0 + 0.125 + 4 * 2.0 ** -8 + 8 * 2.0 ** -12
    # state afterwards holds the last three raw rows: (2, 4, 8)
    np.testing.assert_array_equal(oracle.bf16_widen(pool.conv()[0, 1, :, 2]), [2.0, 4.0, 8.0])


def test_conv_silu_flag():
    """SiLU after the conv: o_t / silu(1) = silu(y_t) for the impulse setup."""
    taps = np.array([[0, 0, 0, 1], [0, 0, 0, 1], [0.5, -0.25, 2.0, 1.5]], dtype=np.float32)
    T = 5
    q = np.ones((T, 1, 1)); k = np.ones((T, 1, 1)); v = np.zeros((T, 1, 1)); v[0] = 1.0
    pool = oracle.Pool(1, 2, 1, 1, 1, oracle.SSM_F32)
    out, err, oe, se = oracle.prefill(
        pool, 0, [0, T], [1], pack_x(q, k, v), f32_bits_to_bf16_torch(taps),
        np.ones((T, 1), np.float32), oracle.ALPHA_PER_HEAD, np.ones((T, 1), np.float32),
        has_initial_state=[0], flags=oracle.CONV_SILU | oracle.L2NORM_K, exact=True)
    silu = lambda z: z / (1 + np.exp(-z))
    y = np.array([1.5, 2.0, -0.25, 0.5, 0.0])
    # K = V = 1: khat = silu(1)/sqrt(silu(1)^2 + 1e-6) is just below 1, so the
    # delta rule keeps S (1 - khat^2) of the old state and writes silu(y) khat.
    s1 = silu(1.0)
    khat = s1 / np.sqrt(s1 * s1 + 1e-6)
    S, want = 0.0, []
    for yt in y:
        S = S * (1 - khat * khat) + silu(yt) * khat
        want.append(S * s1)
    np.testing.assert_allclose(oe[:, 0, 0], want, rtol=1e-12, atol=1e-15)


def test_conv_state_is_last_three_raw_rows():
    """After a call the conv rows equal the last three raw x rows (bit-exact), also
    when the call has fewer than three tokens (rows shift in from the old state)."""
    cfg = wl.TINY
    g = wl.generator(21)
    pool = oracle.Pool(1, 4, cfg.heads, cfg.head_k, cfg.head_v, oracle.SSM_F32)
    ssm, conv = wl.warm_pool(g, 1, 4, cfg.heads, cfg.head_k, cfg.head_v, False)
    pool.ssm()[:] = ssm.numpy(); pool.conv()[:] = wl.bf16_bits(conv)
    w = wl.bf16_bits(wl.conv_weights(g, cfg.channels))
    lens = [9, 2]
    inp = wl.projected_inputs(g, sum(lens), cfg.heads, cfg.head_k, cfg.head_v, cfg.alpha_mode)
    x = wl.bf16_bits(inp["x"])
    old = pool.conv()[0, 3].copy()
    oracle.prefill(pool, 0, wl.cu_seqlens(lens), [1, 3], x, w, inp["alpha"].numpy(),
                   cfg.alpha_mode, inp["beta"].numpy(), has_initial_state=[1, 1])
    assert np.array_equal(pool.conv()[0, 1], x[6:9])
    assert np.array_equal(pool.conv()[0, 3], np.stack([old[2], x[9], x[10]]))


# --------------------------------------------- indexing of the full path ----

def test_full_path_matches_bare_recurrence_per_head():
    """oracle_prefill on several heads, tokens, requests and layers, with identity
    conv taps and no norm, equals the bare recurrence run per head on numpy
    slices; the result lands in the named (layer, slot, head) block and nothing
    else in the pool changes."""
    L, N, H, K, V = 2, 6, 3, 8, 4
    lens = [37, 5]
    T = sum(lens)
    g = wl.generator(31)
    q = torch.randn(T, H, K, generator=g).numpy()
    k = torch.randn(T, H, K, generator=g).numpy()
    v = torch.randn(T, H, V, generator=g).numpy()
    x = pack_x(q, k, v)
    xq = oracle.bf16_widen(x)  # the values the oracle actually sees
    qw = xq[:, :H * K].reshape(T, H, K)
    kw = xq[:, H * K:2 * H * K].reshape(T, H, K)
    vw = xq[:, 2 * H * K:].reshape(T, H, V)
    alpha = torch.sigmoid(torch.randn(T, H, K, generator=g) + 3).numpy()
    beta = torch.sigmoid(torch.randn(T, H, generator=g)).numpy()
    pool = oracle.Pool(L, N, H, K, V, oracle.SSM_F32)
    pool.ssm()[:] = (0.25 * RNG.standard_normal(pool.ssm().shape)).astype(np.float32)
    before = pool.copy()
    slots = [4, 2]
    out, err, oe, se = oracle.prefill(pool, 1, wl.cu_seqlens(lens), slots, x,
                                      identity_taps(H * (2 * K + V)), alpha,
                                      oracle.ALPHA_PER_CHANNEL, beta, has_initial_state=[1, 1],
                                      scale=0.7, flags=0, exact=True)
    cu = wl.cu_seqlens(lens).numpy()
    for b, s in enumerate(slots):
        t0, t1 = cu[b], cu[b + 1]
        for h in range(H):
            o, S = oracle.recurrence_head(qw[t0:t1, h], kw[t0:t1, h], vw[t0:t1, h],
                                          alpha[t0:t1, h], beta[t0:t1, h],
                                          before.ssm()[1, s, h].astype(np.float64),
                                          scale=float(np.float32(0.7)))  # the ABI's scale is a float
            np.testing.assert_array_equal(oe[t0:t1, h], o)
            np.testing.assert_array_equal(se[b, h], S)
            np.testing.assert_array_equal(pool.ssm()[1, s, h], S.astype(np.float32))
    untouched = np.ones((L, N), bool)
    untouched[1, slots] = False
    assert np.array_equal(pool.ssm()[untouched], before.ssm()[untouched])
    assert np.array_equal(pool.conv()[untouched], before.conv()[untouched])


def test_bad_slots_are_skipped_and_flagged():
    cfg = wl.TINY
    g = wl.generator(41)
    pool = oracle.Pool(1, 4, cfg.heads, cfg.head_k, cfg.head_v, oracle.SSM_F32)
    inp = wl.projected_inputs(g, 8, cfg.heads, cfg.head_k, cfg.head_v, cfg.alpha_mode)
    w = wl.bf16_bits(wl.conv_weights(g, cfg.channels))
    before = pool.copy()
    out, err = oracle.prefill(pool, 0, [0, 3, 5, 8], [0, -1, 9], wl.bf16_bits(inp["x"]), w,
                              inp["alpha"].numpy(), cfg.alpha_mode, inp["beta"].numpy())
    assert err == 1
    assert not out.any()
    assert np.array_equal(pool.ssm_bytes, before.ssm_bytes)


# ------------------------------------------------------- chunked algebra ----

@pytest.mark.parametrize("per_channel", [True, False])
@pytest.mark.parametrize("T", [64, 200, 7])
def test_chunked_wy_form_equals_sequential(per_channel, T):
    K, V = 16, 12
    q, k, v, alpha, beta, S0 = _rand_head(T, K, V, alpha_per_channel=per_channel)
    o1, S1 = oracle.recurrence_head(q, k, v, alpha, beta, S0, scale=0.3)
    o2, S2 = oracle.chunked_head_f64(q, k, v, alpha, beta, S0, chunk=64, scale=0.3)
    assert np.linalg.norm(o1 - o2) <= 1e-12 * np.linalg.norm(o1)
    assert np.linalg.norm(S1 - S2) <= 1e-12 * np.linalg.norm(S1)


def test_chunked_wy_form_extreme_decay():
    """Channels with alpha down to 1e-3 (products far below float range) stay finite."""
    T, K, V = 130, 16, 16
    q, k, v, alpha, beta, S0 = _rand_head(T, K, V)
    alpha[:, :4] = 1e-3
    o1, S1 = oracle.recurrence_head(q, k, v, alpha, beta, S0)
    o2, S2 = oracle.chunked_head_f64(q, k, v, alpha, beta, S0, chunk=64)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(S2))
    assert np.linalg.norm(o1 - o2) <= 1e-12 * np.linalg.norm(o1)


# ------------------------------------------------ split and restore ----

def _tiny_setup(seed, ssm_dtype=oracle.SSM_F32):
    cfg = wl.TINY
    g = wl.generator(seed)
    pool = oracle.Pool(1, cfg.slots, cfg.heads, cfg.head_k, cfg.head_v, ssm_dtype)
    ssm, conv = wl.warm_pool(g, 1, cfg.slots, cfg.heads, cfg.head_k, cfg.head_v,
                             ssm_dtype == oracle.SSM_BF16)
    if ssm_dtype == oracle.SSM_F32:
        pool.ssm()[:] = ssm.numpy()
    else:
        pool.ssm()[:] = wl.bf16_bits(ssm)
    pool.conv()[:] = wl.bf16_bits(conv)
    inp = wl.projected_inputs(g, 256, cfg.heads, cfg.head_k, cfg.head_v, cfg.alpha_mode)
    w = wl.bf16_bits(wl.conv_weights(g, cfg.channels))
    return cfg, pool, inp, w


@pytest.mark.parametrize("warm", [0, 1])
def test_split_invariance_bitexact_fp32(warm):
    """One call over 256 tokens equals calls split at 64-token boundaries
    (fp32 oracle, fp32 pool: bit-exact, outputs included)."""
    cfg, pool, inp, w = _tiny_setup(51)
    x, a, b = wl.bf16_bits(inp["x"]), inp["alpha"].numpy(), inp["beta"].numpy()
    p1 = pool.copy()
    o1, _ = oracle.prefill(p1, 0, [0, 256], [3], x, w, a, cfg.alpha_mode, b,
                           has_initial_state=[warm], precision="f32")
    p2 = pool.copy()
    outs = []
    bounds = [0, 64, 192, 256]
    for i in range(3):
        s, e = bounds[i], bounds[i + 1]
        o, _ = oracle.prefill(p2, 0, [0, e - s], [3], x[s:e], w, a[s:e], cfg.alpha_mode, b[s:e],
                              has_initial_state=[warm if i == 0 else 1], start_len=[s],
                              precision="f32")
        outs.append(o)
    assert np.array_equal(o1, np.concatenate(outs))
    assert np.array_equal(p1.ssm_bytes, p2.ssm_bytes)
    assert np.array_equal(p1.conv_bytes, p2.conv_bytes)


def test_restore_then_continue_equals_from_scratch():
    """Snapshot every 64 tokens into ping-pong slots, then restore the snapshot
    taken at 128 into a fresh live slot and continue: the result equals the
    uninterrupted run (fp32 oracle and pool: bit-exact)."""
    cfg, pool, inp, w = _tiny_setup(61)
    x, a, b = wl.bf16_bits(inp["x"]), inp["alpha"].numpy(), inp["beta"].numpy()
    full = pool.copy()
    o_full, _ = oracle.prefill(full, 0, [0, 256], [1], x, w, a, cfg.alpha_mode, b,
                               has_initial_state=[0], precision="f32")
    run = pool.copy()
    # 0..128 with snapshots at 64 (track[0] = slot 2) and 128 (track[1] = slot 3)
    oracle.prefill(run, 0, [0, 128], [1], x[:128], w, a[:128], cfg.alpha_mode, b[:128],
                   has_initial_state=[0], snap_interval=64, track_slots=[[2, 3]],
                   next_track_idx=[0], precision="f32")
    # the snapshot at 128 equals the live slot after 128 tokens
    assert np.array_equal(run.ssm()[0, 3], run.ssm()[0, 1])
    # preemption: the live slot is lost (garbage), restore 3 -> 5 and continue
    run.ssm()[0, 5] = np.float32(np.nan)
    hi = np.array([0], dtype=np.int64)
    oracle.restore_slots(run, [(5, 1, 3)], hi)
    assert hi[0] == 1
    o2, _ = oracle.prefill(run, 0, [0, 128], [5], x[128:], w, a[128:], cfg.alpha_mode, b[128:],
                           has_initial_state=[int(hi[0])], start_len=[128], precision="f32")
    assert np.array_equal(o2, o_full[128:])
    assert np.array_equal(run.ssm()[0, 5], full.ssm()[0, 1])
    assert np.array_equal(run.conv()[0, 5], full.conv()[0, 1])


def test_f32_oracle_close_to_f64_on_tiny_workload():
    cfg, pool, inp, w = _tiny_setup(71)
    x, a, b = wl.bf16_bits(inp["x"]), inp["alpha"].numpy(), inp["beta"].numpy()
    res = {}
    for prec in ("f32", "f64"):
        p = pool.copy()
        out, err, oe, se = oracle.prefill(p, 0, [0, 128, 256], [1, 4], x, w, a, cfg.alpha_mode, b,
                                          has_initial_state=[1, 0], exact=True, precision=prec)
        res[prec] = (oe, se)
    for i in range(2):
        d = np.linalg.norm(res["f32"][i] - res["f64"][i]) / np.linalg.norm(res["f64"][i])
        assert d < 1e-5


# ----------------------------------------------- snapshots and restores ----

def _tiny_model(H=1, K=4, V=4):
    g = wl.generator(81)
    w = wl.bf16_bits(wl.conv_weights(g, H * (2 * K + V)))
    return g, w


def test_decode_track_points_from_the_page(golden_dir):
    """Prompt 1000, interval 256: decode snapshots land at 1024, 1280 and 1536."""
    spec = json.load(open(os.path.join(golden_dir, "page_numbers.json")))["decode_track"]
    H, K, V = 1, 4, 4
    g, w = _tiny_model(H, K, V)
    pool = oracle.Pool(1, 4, H, K, V, oracle.SSM_F32)
    hits = []
    nxt = 0
    for step in range(spec["steps"]):
        seq_after = spec["prompt"] + step + 1
        inp = wl.projected_inputs(g, 1, H, K, V, wl.ALPHA_PER_CHANNEL)
        probe = pool.ssm()[0, 2:4].copy()
        oracle.decode_step(pool, 0, [1], wl.bf16_bits(inp["x"]), w, inp["alpha"].numpy(),
                           oracle.ALPHA_PER_CHANNEL, inp["beta"].numpy(),
                           seq_len_after=[seq_after], track_interval=spec["interval"],
                           track_slots=[[2, 3]], next_track_idx=[nxt])
        if not np.array_equal(probe, pool.ssm()[0, 2:4]):
            hits.append(seq_after)
            assert np.array_equal(pool.ssm()[0, 2 + nxt], pool.ssm()[0, 1])
            nxt ^= 1   # the caller flips after the step
    assert hits == spec["checkpoints"]


@pytest.mark.parametrize("alpha_mode", [oracle.ALPHA_PER_CHANNEL, oracle.ALPHA_PER_HEAD])
@pytest.mark.parametrize("ssm_dtype", [oracle.SSM_F32, oracle.SSM_BF16])
def test_batched_decode_equals_single_request_calls(alpha_mode, ssm_dtype):
    """oracle_decode_step over B requests in one call equals B calls of one
    request each, and a one-token oracle_prefill per request (page
    "企业官网建设流程全解析", "--mamba-track-interval": the step folds one
    token per request; a request whose length reaches a multiple of the interval
    snapshots into track_slots[b][next_track_idx[b]]).  The pool has K != V, two
    layers and three heads, so a wrong per-request stride of x, alpha, beta, out,
    the slot table, the track pairs or the next index lands on another request's
    data or slot.  Covered: a reserved slot (0), a slot past the pool (flagged),
    a request that snapshots into track index 1, one into index 0, one whose
    designated track entry is masked (0), and requests that do not snapshot.
    fp32 build, bit-exact."""
    L, N, H, K, V = 2, 24, 3, 8, 4
    g = wl.generator(1212)
    pool = oracle.Pool(L, N, H, K, V, ssm_dtype)
    ssm, conv = wl.warm_pool(g, L, N, H, K, V, ssm_dtype == oracle.SSM_BF16)
    pool.ssm()[:] = ssm.numpy() if ssm_dtype == oracle.SSM_F32 else wl.bf16_bits(ssm)
    pool.conv()[:] = wl.bf16_bits(conv)
    w = wl.bf16_bits(wl.conv_weights(g, H * (2 * K + V)))
    slots = np.array([5, 0, 9, 2, 30, 14, 7], np.int32)
    B = len(slots)
    seq_after = np.array([512, 300, 257, 768, 1024, 1280, 9], np.int32)
    track = np.array([[17, 18], [19, 20], [21, 22], [3, 4], [11, 12], [0, 23], [15, 16]], np.int32)
    nxt = np.array([1, 0, 0, 0, 1, 0, 1], np.int32)
    inp = wl.projected_inputs(g, B, H, K, V, alpha_mode)
    x, a, b = wl.bf16_bits(inp["x"]), inp["alpha"].numpy(), inp["beta"].numpy()
    kw = dict(scale=0.75, flags=oracle.L2NORM_K, track_interval=256, precision="f32")

    batched = pool.copy()
    out, err = oracle.decode_step(batched, 1, slots, x, w, a, alpha_mode, b,
                                  seq_len_after=seq_after, track_slots=track,
                                  next_track_idx=nxt, **kw)
    assert err == 1                                   # slot 30 is past the pool
    single = pool.copy()
    for i in range(B):
        o1, e1 = oracle.decode_step(single, 1, slots[i:i + 1], x[i:i + 1], w, a[i:i + 1],
                                    alpha_mode, b[i:i + 1], seq_len_after=seq_after[i:i + 1],
                                    track_slots=track[i:i + 1], next_track_idx=nxt[i:i + 1], **kw)
        assert e1 == (1 if slots[i] >= N else 0)
        np.testing.assert_array_equal(out[i], o1[0])
    assert np.array_equal(batched.ssm_bytes, single.ssm_bytes)
    assert np.array_equal(batched.conv(), single.conv())

    # One-token prefill calls with the same snapshot rule give the same pool
    # and outputs (the prefill indexing is pinned by the per-head test above).
    pre = pool.copy()
    for i in range(B):
        if not 0 < slots[i] < N:
            continue
        o1, e1 = oracle.prefill(pre, 1, [0, 1], slots[i:i + 1], x[i:i + 1], w, a[i:i + 1],
                                alpha_mode, b[i:i + 1], has_initial_state=[1],
                                start_len=seq_after[i:i + 1] - 1, scale=0.75,
                                flags=oracle.L2NORM_K, snap_interval=256,
                                track_slots=track[i:i + 1], next_track_idx=nxt[i:i + 1],
                                precision="f32")
        assert e1 == 0
        np.testing.assert_array_equal(out[i], o1[0])
    assert np.array_equal(batched.ssm_bytes, pre.ssm_bytes)
    assert np.array_equal(batched.conv(), pre.conv())

    # What landed where: live slots changed, snapshots in the designated track
    # slots only, the masked entry and the skipped requests wrote nothing.
    changed = lambda p, l, s: not np.array_equal(p.ssm()[l, s], pool.ssm()[l, s])
    for i, s in enumerate(slots):
        if 0 < s < N:
            assert changed(batched, 1, s) and not changed(batched, 0, s)
    snaps = {18: 5, 3: 2}                             # track slot -> the live slot it copies
    for t, s in snaps.items():
        assert np.array_equal(batched.ssm()[1, t], batched.ssm()[1, s])
        assert np.array_equal(batched.conv()[1, t], batched.conv()[1, s])
    untouched = [n for n in range(1, N) if n not in set(slots.tolist()) | set(snaps)]
    for n in untouched:
        assert not changed(batched, 1, n), n
    assert not out[1].any() and not out[4].any()


def test_prefill_walkthrough_from_the_page(golden_dir):
    """1200 tokens in calls of 512/512/176 with snapshot interval 512: slot B
    (track[0]) holds the state at 512, slot C (track[1]) the state at 1024, and
    one single 1200-token call places them identically."""
    spec = json.load(open(os.path.join(golden_dir, "page_numbers.json")))["prefill_walkthrough"]
    H, K, V = 1, 4, 4
    g, w = _tiny_model(H, K, V)
    n = spec["length"]
    inp = wl.projected_inputs(g, n, H, K, V, wl.ALPHA_PER_CHANNEL)
    x, a, b = wl.bf16_bits(inp["x"]), inp["alpha"].numpy(), inp["beta"].numpy()
    A, B, C = 1, 2, 3
    # reference states at the track points (f32 oracle, fp32 pool: exact under splitting)
    ref = {}
    for pt in spec["track_points"]:
        p = oracle.Pool(1, 4, H, K, V, oracle.SSM_F32)
        oracle.prefill(p, 0, [0, pt], [A], x[:pt], w, a[:pt], 1, b[:pt], has_initial_state=[0],
                       precision="f32")
        ref[pt] = p.ssm()[0, A].copy()
    # chunked calls, flipping next_track_idx after each call that took a snapshot
    p = oracle.Pool(1, 4, H, K, V, oracle.SSM_F32)
    nxt, start, nexts = 0, 0, []
    for i, m in enumerate(spec["calls"]):
        before = p.ssm()[0, [B, C]].copy()
        oracle.prefill(p, 0, [0, m], [A], x[start:start + m], w, a[start:start + m], 1,
                       b[start:start + m], has_initial_state=[1 if i else 0], start_len=[start],
                       snap_interval=spec["chunk"], track_slots=[[B, C]], next_track_idx=[nxt],
                       precision="f32")
        if not np.array_equal(before, p.ssm()[0, [B, C]]):
            nxt ^= 1
        nexts.append(nxt)
        start += m
    assert nexts == spec["next_idx_after"]
    for pt, bi in zip(spec["track_points"], spec["track_buffer_index"]):
        assert np.array_equal(p.ssm()[0, [B, C][bi]], ref[pt])
    # one call, the j-th boundary alternating from next_track_idx
    q = oracle.Pool(1, 4, H, K, V, oracle.SSM_F32)
    oracle.prefill(q, 0, [0, n], [A], x, w, a, 1, b, has_initial_state=[0], snap_interval=spec["chunk"],
                   track_slots=[[B, C]], next_track_idx=[0], precision="f32")
    assert np.array_equal(q.ssm()[0, B], ref[512]) and np.array_equal(q.ssm()[0, C], ref[1024])


def test_chunked_prefill_state_count_from_the_page(golden_dir):
    """13600 tokens in chunked-prefill passes of 6144: boundaries at 6144 and
    12288 are snapshotted and the live slot holds the third state."""
    spec = json.load(open(os.path.join(golden_dir, "page_numbers.json")))["chunked_prefill_states"]
    n, cps = spec["length"], spec["chunk"]
    bounds = [m for m in range(1, n + 1) if m % cps == 0]
    assert len(bounds) + 1 == spec["states"]
    assert [min(cps, n - i) for i in range(0, n, cps)] == spec["calls"]


def test_pool_sizes_from_the_page(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "page_numbers.json")))["pool_sizes"]
    for e in spec:
        dt = oracle.SSM_F32 if e["ssm_dtype"] == "f32" else oracle.SSM_BF16
        s, c = oracle.pool_bytes(e["layers"], e["slots"], e["heads"], e["head_k"], e["head_v"], dt)
        if "ssm_gib_2dp" in e:
            assert round(s / 2 ** 30, 2) == e["ssm_gib_2dp"]
            assert round(c / 2 ** 30, 2) == e["conv_gib_2dp"]
        if "ssm_bytes" in e:
            assert s == e["ssm_bytes"]
        if "conv_bytes" in e:
            assert c == e["conv_bytes"]


def test_restore_rules():
    """restore_linear_state_slots: not requested -> unchanged; bad or missing
    source -> COLD_START (0) and no copy; src == dst -> RESTORED, no copy;
    otherwise copy every layer -> RESTORED."""
    pool = oracle.Pool(3, 6, 1, 4, 4, oracle.SSM_BF16)
    pool.ssm_bytes[:] = RNG.integers(0, 256, pool.ssm_bytes.size, dtype=np.uint8)
    pool.conv_bytes[:] = RNG.integers(0, 256, pool.conv_bytes.size, dtype=np.uint8)
    before = pool.copy()
    ops = [(1, 0, 2), (2, 1, -1), (3, 1, 6), (4, 1, 4), (5, 1, 3), (0, 1, 3)]
    hi = np.array([7, 7, 7, 7, 7, 7], dtype=np.int64)
    oracle.restore_slots(pool, ops, hi)
    assert hi.tolist() == [7, 0, 0, 1, 1, 0]
    exp_ssm, exp_conv = before.ssm().copy(), before.conv().copy()
    exp_ssm[:, 5] = before.ssm()[:, 3]
    exp_conv[:, 5] = before.conv()[:, 3]
    assert np.array_equal(pool.ssm(), exp_ssm)
    assert np.array_equal(pool.conv(), exp_conv)


def test_track_snapshot_copies_layer_range():
    pool = oracle.Pool(4, 6, 2, 4, 4, oracle.SSM_F32)
    pool.ssm_bytes[:] = RNG.integers(0, 256, pool.ssm_bytes.size, dtype=np.uint8)
    pool.conv_bytes[:] = RNG.integers(0, 256, pool.conv_bytes.size, dtype=np.uint8)
    before = pool.copy()
    err = oracle.track_snapshot(pool, 1, 3, [1, 2, 3], [4, 0, 5])
    assert err == 0
    exp = before.ssm().copy(); expc = before.conv().copy()
    exp[1:3, 4] = before.ssm()[1:3, 1]; expc[1:3, 4] = before.conv()[1:3, 1]
    exp[1:3, 5] = before.ssm()[1:3, 3]; expc[1:3, 5] = before.conv()[1:3, 3]
    # random bytes include NaN patterns: compare bit patterns, not float values
    assert np.array_equal(pool.ssm().view(np.uint32), exp.view(np.uint32))
    assert np.array_equal(pool.conv(), expc)


def test_cold_start_ignores_slot_contents():
    """has_initial_state = 0 starts from zero state and zero conv rows, whatever
    the live slot held (page "Qwen3.5 Linear-State Prefix Cache", 6.4: cold)."""
    cfg, pool, inp, w = _tiny_setup(91)
    x, a, b = wl.bf16_bits(inp["x"]), inp["alpha"].numpy(), inp["beta"].numpy()
    zero = oracle.Pool(1, cfg.slots, cfg.heads, cfg.head_k, cfg.head_v, oracle.SSM_F32)
    o1, _ = oracle.prefill(pool, 0, [0, 100], [2], x[:100], w, a[:100], cfg.alpha_mode, b[:100],
                           has_initial_state=[0])
    o2, _ = oracle.prefill(zero, 0, [0, 100], [2], x[:100], w, a[:100], cfg.alpha_mode, b[:100],
                           has_initial_state=[1])
    assert np.array_equal(o1, o2)
    assert np.array_equal(pool.ssm()[0, 2], zero.ssm()[0, 2])
    assert np.array_equal(pool.conv()[0, 2], zero.conv()[0, 2])


# ------------------------------------------------ speculative verify ----

def _spec_setup(seed, B, T, ssm_dtype=oracle.SSM_F32, H=2, K=8, V=8, slots=12):
    """Warm pool, conv taps and per-node inputs x [B][T][C], alpha [B][T][H][K],
    beta [B][T][H]."""
    g = wl.generator(seed)
    pool = oracle.Pool(1, slots, H, K, V, ssm_dtype)
    ssm, conv = wl.warm_pool(g, 1, slots, H, K, V, ssm_dtype == oracle.SSM_BF16)
    pool.ssm()[:] = ssm.numpy() if ssm_dtype == oracle.SSM_F32 else wl.bf16_bits(ssm)
    pool.conv()[:] = wl.bf16_bits(conv)
    w = wl.bf16_bits(wl.conv_weights(g, H * (2 * K + V)))
    inp = wl.projected_inputs(g, B * T, H, K, V, wl.ALPHA_PER_CHANNEL)
    x = wl.bf16_bits(inp["x"]).reshape(B, T, -1)
    a = inp["alpha"].numpy().reshape(B, T, H, K)
    b = inp["beta"].numpy().reshape(B, T, H)
    return pool, w, x, a, b


def _path(parent, n):
    p = []
    while n >= 0:
        p.append(n)
        n = parent[n]
    return p[::-1]


def _decode_path(pool, slot, path, x, w, a, b, precision, **track):
    """Decode the path's tokens one by one into ``slot`` of a copy of the pool;
    returns (copy, outputs per step)."""
    p = pool.copy()
    outs = []
    for i, n in enumerate(path):
        kw = {k: (v[i] if k == "seq_len_after" else v) for k, v in track.items()}
        o, err = oracle.decode_step(p, 0, [slot], x[None, n], w, a[None, n],
                                    oracle.ALPHA_PER_CHANNEL, b[None, n], precision=precision, **kw)
        assert err == 0
        outs.append(o[0])
    return p, outs


@pytest.mark.parametrize("ssm_dtype", [oracle.SSM_F32, oracle.SSM_BF16])
def test_verify_page_tree_equals_decodes_along_each_path(golden_dir, ssm_dtype):
    """Every node of the pages' 9-node tree equals decoding the tokens on its
    root path one at a time from the live slot: same output bits, same state
    and conv rows (each decode stores its state in the pool dtype, as a node
    does).  The live slot is left as it was."""
    spec = json.load(open(os.path.join(golden_dir, "eagle_tree.json")))
    parent = np.array(spec["parent"], dtype=np.int32)
    T = parent.shape[0]
    pool, w, x, a, b = _spec_setup(91, 1, T, ssm_dtype)
    before = pool.copy()
    out, ns, nc, err = oracle.verify_tree(pool, 0, [5], parent[None], x, w, a,
                                          oracle.ALPHA_PER_CHANNEL, b, precision="f32")
    assert err == 0
    assert np.array_equal(pool.ssm_bytes, before.ssm_bytes)
    assert np.array_equal(pool.conv_bytes, before.conv_bytes)
    # the reads the page lists: roots from the main state, the rest from a node
    for src, nodes in spec["reads"].items():
        for n in nodes:
            assert parent[n] == (-1 if src == "main" else int(src))
    for n in range(T):
        p, outs = _decode_path(pool, 5, _path(parent, n), x[0], w, a[0], b[0], "f32")
        assert np.array_equal(out[0, n], outs[-1])
        assert np.array_equal(ns[0, n], p.ssm()[0, 5])
        assert np.array_equal(nc[0, n], p.conv()[0, 5])


def test_verify_chain_and_star_trees():
    """A chain (parent n-1) equals sequential decodes; a star (all -1) equals
    independent one-token decodes from the live slot.  Two requests at once,
    in different slots."""
    T = 5
    pool, w, x, a, b = _spec_setup(92, 2, T)
    parent = np.array([np.arange(T) - 1, -np.ones(T)], dtype=np.int32)
    out, ns, nc, err = oracle.verify_tree(pool, 0, [3, 7], parent, x, w, a,
                                          oracle.ALPHA_PER_CHANNEL, b, precision="f32")
    assert err == 0
    p, outs = _decode_path(pool, 3, list(range(T)), x[0], w, a[0], b[0], "f32")
    assert np.array_equal(out[0], np.stack(outs))
    assert np.array_equal(ns[0, T - 1], p.ssm()[0, 3])
    for n in range(T):
        p, outs = _decode_path(pool, 7, [n], x[1], w, a[1], b[1], "f32")
        assert np.array_equal(out[1, n], outs[0])
        assert np.array_equal(ns[1, n], p.ssm()[0, 7])
        assert np.array_equal(nc[1, n], p.conv()[0, 7])


def test_verify_f64_node_states_follow_the_recurrence():
    """Conv off (identity taps), f64: a chain's last node state equals the bare
    recurrence over the same prepared tokens from the live state."""
    H, K, V, T = 1, 4, 4, 4
    g = wl.generator(93)
    pool = oracle.Pool(1, 4, H, K, V, oracle.SSM_F32)
    S0 = (0.25 * torch.randn(V, K, generator=g)).numpy()
    pool.ssm()[0, 2, 0] = S0
    q = torch.randn(T, K, generator=g).to(torch.bfloat16)
    k = torch.randn(T, K, generator=g)
    k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
    v = torch.randn(T, V, generator=g).to(torch.bfloat16)
    x = wl.bf16_bits(torch.cat([q, k, v], dim=1)).reshape(1, T, -1)
    a = torch.sigmoid(torch.randn(1, T, H, K, generator=g) + 3).numpy()
    b = torch.sigmoid(torch.randn(1, T, H, generator=g)).numpy()
    parent = (np.arange(T, dtype=np.int32) - 1)[None]
    out, ns, nc, err, oe = oracle.verify_tree(pool, 0, [2], parent, x, identity_taps(H * (2 * K + V)),
                                              a, oracle.ALPHA_PER_CHANNEL, b, flags=0, exact=True)
    assert err == 0
    o, S = oracle.recurrence_head(q.float().numpy(), k.float().numpy(), v.float().numpy(),
                                  a[0, :, 0], b[0, :, 0], S0.astype(np.float64))
    # node 0 starts from the live state itself; each later node starts from its
    # parent's state as stored (fp32 here), so agreement is to fp32 rounding
    assert np.allclose(oe[0, 0, 0], o[0], rtol=0, atol=1e-12)
    assert np.allclose(oe[0, :, 0], o, rtol=0, atol=1e-6)
    assert np.allclose(ns[0, T - 1, 0], S, rtol=0, atol=1e-6)


def test_verify_rejects_bad_trees_and_slots():
    """A parent that is not -1 or an earlier node flags bit 8 and the request
    gets zero outputs and no node writes; a live slot past the pool flags bit
    1; the other requests are unaffected."""
    T = 3
    pool, w, x, a, b = _spec_setup(94, 3, T)
    good = [-1, 0, 0]
    parent = np.array([good, [-1, 2, 0], good], dtype=np.int32)   # node 1 reads a later node
    out, ns, nc, err = oracle.verify_tree(pool, 0, [1, 2, 99], parent, x, w, a,
                                          oracle.ALPHA_PER_CHANNEL, b, precision="f32")
    assert err == 8 | 1
    assert not out[1].any() and not ns[1].any() and not nc[1].any()
    assert not out[2].any() and not ns[2].any()
    ref, _, _, e0 = oracle.verify_tree(pool, 0, [1], parent[:1], x[:1], w, a[:1],
                                       oracle.ALPHA_PER_CHANNEL, b[:1], precision="f32")
    assert e0 == 0 and np.array_equal(out[0], ref[0]) and out[0].any()
    for bad in ([-2, -1, 0], [0, -1, -1]):
        _, _, _, e = oracle.verify_tree(pool, 0, [1], np.array([bad], dtype=np.int32), x[:1], w,
                                        a[:1], oracle.ALPHA_PER_CHANNEL, b[:1], precision="f32")
        assert e == 8


def test_verify_buffer_is_nodes_times_the_state(golden_dir):
    """The per-node buffers hold one state and one set of conv rows per tree
    node: T times a slot's bytes (the pages' 3x, 7x, 63x)."""
    spec = json.load(open(os.path.join(golden_dir, "eagle_tree.json")))
    pool = oracle.Pool(1, 2, 2, 8, 8, oracle.SSM_BF16)
    slot_bytes = pool.ssm()[0, 0].nbytes
    for topk, steps, nodes in spec["buffer_ratio"]:
        ns, nc = oracle.node_buffers(pool, 1, nodes)
        assert ns.nbytes == nodes * slot_bytes
        assert nc.nbytes == nodes * pool.conv()[0, 0].nbytes


@pytest.mark.parametrize("ssm_dtype", [oracle.SSM_F32, oracle.SSM_BF16])
def test_accept_scatter_equals_decoding_the_accepted_path(golden_dir, ssm_dtype):
    """After verify, scattering accepted node n leaves the live slot exactly as
    decoding n's root path token by token would; accepted -1 changes nothing."""
    spec = json.load(open(os.path.join(golden_dir, "eagle_tree.json")))
    parent = np.array([spec["parent"]] * 2, dtype=np.int32)
    T = parent.shape[1]
    pool, w, x, a, b = _spec_setup(95, 2, T, ssm_dtype)
    _, ns, nc, err = oracle.verify_tree(pool, 0, [4, 6], parent, x, w, a,
                                        oracle.ALPHA_PER_CHANNEL, b, precision="f32")
    assert err == 0
    run = pool.copy()
    assert oracle.accept_scatter(run, 0, [4, 6], parent, [7, -1], ns, nc) == 0
    p, _ = _decode_path(pool, 4, _path(parent[0], 7), x[0], w, a[0], b[0], "f32")
    assert np.array_equal(run.ssm_bytes, p.ssm_bytes)
    assert np.array_equal(run.conv_bytes, p.conv_bytes)


@pytest.mark.parametrize("before,hit_depth", [(254, 2), (255, 1), (253, 3), (250, None)])
def test_accept_scatter_tracks_the_interval_crossing(before, hit_depth):
    """Accepting a depth-3 node whose tokens cross a multiple of 256 copies the
    node at the crossing depth into the track slot, exactly as decode steps with
    tracking place the snapshot (replay-with-tracking rule of the pages)."""
    T = 4
    parent = np.array([[-1, 0, 1, 0]], dtype=np.int32)   # node 2 at depth 3
    pool, w, x, a, b = _spec_setup(96, 1, T)
    _, ns, nc, err = oracle.verify_tree(pool, 0, [1], parent, x, w, a,
                                        oracle.ALPHA_PER_CHANNEL, b, precision="f32")
    run = pool.copy()
    err = oracle.accept_scatter(run, 0, [1], parent, [2], ns, nc, seq_len_before=[before],
                                track_interval=256, track_slots=[[9, 10]], next_track_idx=[1])
    assert err == 0
    path = _path(parent[0], 2)
    p, _ = _decode_path(pool, 1, path, x[0], w, a[0], b[0], "f32",
                        seq_len_after=[[before + i + 1] for i in range(3)], track_interval=256,
                        track_slots=[[9, 10]], next_track_idx=[1])
    assert np.array_equal(run.ssm_bytes, p.ssm_bytes)
    assert np.array_equal(run.conv_bytes, p.conv_bytes)
    if hit_depth is None:
        assert np.array_equal(run.ssm()[0, 10], pool.ssm()[0, 10])
    else:
        assert np.array_equal(run.ssm()[0, 10], ns[0, path[hit_depth - 1]])
    assert np.array_equal(run.ssm()[0, 9], pool.ssm()[0, 9])


def test_accept_scatter_rejects_bad_input():
    T = 3
    pool, w, x, a, b = _spec_setup(97, 2, T)
    parent = np.array([[-1, 0, 1], [-1, 0, 1]], dtype=np.int32)
    _, ns, nc, _ = oracle.verify_tree(pool, 0, [1, 2], parent, x, w, a,
                                      oracle.ALPHA_PER_CHANNEL, b, precision="f32")
    run = pool.copy()
    assert oracle.accept_scatter(run, 0, [1, 2], parent, [3, -2], ns, nc) == 8
    assert np.array_equal(run.ssm_bytes, pool.ssm_bytes)
    assert oracle.accept_scatter(run, 0, [99, 2], parent, [0, 2], ns, nc) == 1
    assert np.array_equal(run.ssm()[0, 2], ns[1, 2])
    assert oracle.accept_scatter(run, 0, [1, 2], parent, [2, -1], ns, nc, seq_len_before=[254],
                                 track_interval=256, track_slots=[[99, 99], [0, 0]]) == 2


# ------------------------------------------------------ ReplaySSM ring ----

def test_replay_ring_sizes_from_the_page(golden_dir):
    """The ring arrays the commit replays from (rawk, rawv, g, beta) have the
    sizes the pages print; with the pages' two further rings (d, k) the total
    and the per-slot figure match too."""
    spec = json.load(open(os.path.join(golden_dir, "replay_ring.json")))
    pool = oracle.Pool(spec["layers"], spec["slots"], spec["heads"], spec["head_k"], spec["head_v"],
                       oracle.SSM_BF16)
    rk, rv, g, beta, xrow = oracle.ring_bytes(pool, spec["positions"], oracle.ALPHA_PER_CHANNEL)
    assert (rk, rv, g, beta) == (spec["rawk_bytes"], spec["rawv_bytes"], spec["g_per_channel_bytes"],
                                 spec["beta_bytes"])
    _, _, g_head, _, _ = oracle.ring_bytes(pool, spec["positions"], oracle.ALPHA_PER_HEAD)
    assert g_head * 128 == g
    total = rk + rv + g + beta + spec["d_bytes"] + spec["k_bytes"]
    # the printed GiB total (1.539063) is one unit of its last decimal above the
    # exact 1.5390623 of its own byte figures; the per-slot byte count is exact
    assert abs(total / 2 ** 30 - spec["total_gib_6dp"]) <= 1e-6
    assert total == spec["per_slot_bytes"] * spec["slots"]
    # the conv input rows the commit needs in addition: one row of C per position
    assert xrow == spec["layers"] * spec["slots"] * spec["positions"] * pool.channels * 2


def _replay_setup(seed, B, D, ssm_dtype=oracle.SSM_F32, identity=True, H=2, K=8, V=8, slots=12,
                  positions=8, amode=oracle.ALPHA_PER_CHANNEL):
    pool, w, x, a, b = _spec_setup(seed, B, D, ssm_dtype, H, K, V, slots)
    if identity:
        w = identity_taps(H * (2 * K + V))
    if amode == oracle.ALPHA_PER_HEAD:
        a = np.ascontiguousarray(a[..., 0])
    ring = oracle.Ring(pool, positions, amode)
    return pool, w, x, a, b, ring


@pytest.mark.parametrize("identity", [True, False])
def test_replay_verify_equals_chain_of_decodes(identity):
    """Verify with the ring gives the outputs of consecutive decode steps (bit-exact,
    fp32 build), leaves the live slots as they are, and records the conv outputs
    k and v (bf16), the decay, beta and the conv input rows."""
    B, D = 2, 5
    pool, w, x, a, b, ring = _replay_setup(101, B, D, identity=identity)
    before = pool.copy()
    out, err = oracle.replay_verify(pool, ring, 0, [3, 7], x, w, a, oracle.ALPHA_PER_CHANNEL, b,
                                    precision="f32")
    assert err == 0
    assert np.array_equal(pool.ssm_bytes, before.ssm_bytes)
    assert np.array_equal(pool.conv_bytes, before.conv_bytes)
    for i, s in enumerate((3, 7)):
        _, outs = _decode_path(before, s, list(range(D)), x[i], w, a[i], b[i], "f32")
        assert np.array_equal(out[i], np.stack(outs))
        assert np.array_equal(ring.g[0, s, :, :D], a[i].transpose(1, 0, 2))
        assert np.array_equal(ring.beta[0, s, :, :D], b[i].T)
        assert np.array_equal(ring.xrow[0, s, :D], x[i])
        if identity:   # taps (0, 0, 0, 1): the conv outputs are the inputs, exactly
            H, K, V = pool.heads, pool.head_k, pool.head_v
            xk = x[i][:, H * K:2 * H * K].reshape(D, H, K).transpose(1, 0, 2)
            xv = x[i][:, 2 * H * K:].reshape(D, H, V).transpose(1, 0, 2)
            assert np.array_equal(ring.rawk[0, s, :, :D], xk)
            assert np.array_equal(ring.rawv[0, s, :, :D], xv)
    assert not ring.rawk[0, 5].any()   # other slots' rings untouched


@pytest.mark.parametrize("ssm_dtype", [oracle.SSM_F32, oracle.SSM_BF16])
@pytest.mark.parametrize("n", [0, 1, 3, 5])
def test_replay_commit_equals_decoding_the_accepted_prefix(ssm_dtype, n):
    """With identity taps (so the ring's bf16 k and v are exact), committing n
    accepted tokens leaves the slot exactly as n decode steps would (fp32
    build; the state is rounded to the pool dtype once, at the end)."""
    B, D = 2, 5
    pool, w, x, a, b, ring = _replay_setup(102, B, D, ssm_dtype)
    oracle.replay_verify(pool, ring, 0, [3, 7], x, w, a, oracle.ALPHA_PER_CHANNEL, b,
                         precision="f32")
    run = pool.copy()
    assert oracle.replay_commit(run, ring, 0, [3, 7], [n, 2], oracle.ALPHA_PER_CHANNEL,
                                precision="f32") == 0
    want = pool.copy()
    # decode steps store the state every step; with an fp32 pool that is exact,
    # with a bf16 pool the fold (one rounding) is compared with tolerance
    for i, (s, m) in enumerate(((3, n), (7, 2))):
        if m:
            p, _ = _decode_path(pool, s, list(range(m)), x[i], w, a[i], b[i], "f32")
            want.ssm()[0, s] = p.ssm()[0, s]
            want.conv()[0, s] = p.conv()[0, s]
    assert np.array_equal(run.conv_bytes, want.conv_bytes)
    if ssm_dtype == oracle.SSM_F32:
        assert np.array_equal(run.ssm_bytes, want.ssm_bytes)
    else:
        got, exp = oracle.bf16_widen(run.ssm()), oracle.bf16_widen(want.ssm())
        assert np.linalg.norm(got - exp) <= 1e-2 * np.linalg.norm(exp)
        untouched = [s for s in range(pool.slots) if s not in (3, 7)]
        assert np.array_equal(run.ssm()[0, untouched], pool.ssm()[0, untouched])


def test_replay_commit_with_conv_taps_folds_the_ring_values():
    """With real conv taps the ring holds k and v rounded to bf16 (the pages' ring
    dtype).  The fold is the bare recurrence on exactly those values (k
    normalised, decay g, beta), and it lies within bf16-level distance of
    decoding the same tokens."""
    H, K, V = 2, 16, 16
    pool, w, x, a, b, ring = _replay_setup(103, 1, 6, identity=False, K=K, V=V)
    oracle.replay_verify(pool, ring, 0, [4], x, w, a, oracle.ALPHA_PER_CHANNEL, b)
    run = pool.copy()
    oracle.replay_commit(run, ring, 0, [4], [6], oracle.ALPHA_PER_CHANNEL)
    for h in range(H):
        k = oracle.bf16_widen(ring.rawk[0, 4, h, :6])
        k = k / np.sqrt((k * k).sum(axis=1, keepdims=True) + 1e-6)
        v = oracle.bf16_widen(ring.rawv[0, 4, h, :6])
        _, S = oracle.recurrence_head(np.zeros((6, K)), k, v, ring.g[0, 4, h, :6].astype(np.float64),
                                      ring.beta[0, 4, h, :6].astype(np.float64),
                                      pool.ssm()[0, 4, h].astype(np.float64))
        got = run.ssm()[0, 4, h].astype(np.float64)
        assert np.linalg.norm(got - S) <= 1e-6 * np.linalg.norm(S)   # fp32 pool rounding
    p, _ = _decode_path(pool, 4, list(range(6)), x[0], w, a[0], b[0], "f64")
    got, want = run.ssm()[0, 4].astype(np.float64), p.ssm()[0, 4].astype(np.float64)
    d = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert 0 < d < 1e-2
    assert np.array_equal(run.conv()[0, 4], p.conv()[0, 4])


@pytest.mark.parametrize("before,interval,hits", [(254, 256, [2]), (255, 256, [1]), (250, 256, []),
                                                   (3, 2, [1, 3])])
def test_replay_commit_tracks_crossings(before, interval, hits):
    """The state after the token that completes a multiple of the interval goes
    to the track slot, the j-th crossing to (next + j) & 1 (decode-with-tracking
    and prefill rules; identity taps, bit-exact)."""
    pool, w, x, a, b, ring = _replay_setup(104, 1, 4, identity=True)
    oracle.replay_verify(pool, ring, 0, [1], x, w, a, oracle.ALPHA_PER_CHANNEL, b, precision="f32")
    run = pool.copy()
    track = np.array([[9, 10]], dtype=np.int32)
    assert oracle.replay_commit(run, ring, 0, [1], [4], oracle.ALPHA_PER_CHANNEL,
                                seq_len_before=[before], track_interval=interval, track_slots=track,
                                next_track_idx=[1], precision="f32") == 0
    for j, i in enumerate(hits):
        p, _ = _decode_path(pool, 1, list(range(i)), x[0], w, a[0], b[0], "f32")
        dst = int(track[0, (1 + j) & 1])
        assert np.array_equal(run.ssm()[0, dst], p.ssm()[0, 1])
        assert np.array_equal(run.conv()[0, dst], p.conv()[0, 1])
    if not hits:
        assert np.array_equal(run.ssm()[0, 9:11], pool.ssm()[0, 9:11])


def test_replay_gdn_scalar_decay_and_errors():
    """Per-head decay rings hold one g per position; accepted beyond the ring
    flags bit 8 and writes nothing; bad live and track slots flag bits 1 and 2."""
    pool, w, x, a, b, ring = _replay_setup(105, 2, 3, amode=oracle.ALPHA_PER_HEAD, positions=4)
    out, err = oracle.replay_verify(pool, ring, 0, [2, 5], x, w, a, oracle.ALPHA_PER_HEAD, b,
                                    precision="f32")
    assert err == 0 and ring.g.shape == (1, pool.slots, pool.heads, 4)
    _, outs = _decode_path_head(pool, 2, 3, x[0], w, a[0], b[0])
    assert np.array_equal(out[0], np.stack(outs))
    run = pool.copy()
    assert oracle.replay_commit(run, ring, 0, [2, 5], [5, 1], oracle.ALPHA_PER_HEAD) == 8
    assert np.array_equal(run.ssm()[0, 2], pool.ssm()[0, 2])
    assert not np.array_equal(run.ssm()[0, 5], pool.ssm()[0, 5])
    assert oracle.replay_commit(pool.copy(), ring, 0, [99, 5], [1, 1], oracle.ALPHA_PER_HEAD) == 1
    assert oracle.replay_commit(pool.copy(), ring, 0, [2, 5], [2, 0], oracle.ALPHA_PER_HEAD,
                                seq_len_before=[0, 0], track_interval=1,
                                track_slots=[[99, 0], [0, 0]]) == 2


def _decode_path_head(pool, slot, n, x, w, a, b):
    """n decode steps with per-head decay (a [D][H])."""
    p = pool.copy()
    outs = []
    for t in range(n):
        o, err = oracle.decode_step(p, 0, [slot], x[None, t], w, a[None, t], oracle.ALPHA_PER_HEAD,
                                    b[None, t], precision="f32")
        assert err == 0
        outs.append(o[0])
    return p, outs
