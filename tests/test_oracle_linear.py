"""Pins for the fp64 definition of the multi-adapter linear layer.

What fixes it without any implementation to compare against:
  * a worked example computed by hand (tests/golden/hand_example.txt);
  * the merged identity W0 x + s B (A x) == (W0 + s B A) x for one adapter;
  * base-only cases: id -1, inactive rows, B = 0 give exactly W0 x;
  * a closed form with selector adapters (unit-vector rows of A and B);
  * invariance under row permutation;
  * agreement of three formulations (grouped, per-row, gathered);
  * brute force with scalar Python loops on tiny shapes;
  * padding rows of the pool (j >= rank) filled with NaN change nothing.
A final test plants plausible mistakes in a copy of the oracle and checks
that these pins catch every one of them.
"""
import numpy as np
import pytest

import oracle
from oracle import layer as L
from golden_io import load


def _hand():
    g = load("hand_example.txt")
    A = np.full((2, 2, 3), np.nan)
    B = np.full((2, 2, 2), np.nan)       # [slot, d_out, R_cap]
    A[0, :1] = g["A0"]
    A[1, :2] = g["A1"]
    B[0, :, :1] = np.asarray(g["B0"]).reshape(2, 1)
    B[1, :, :2] = np.asarray(g["B1"])
    return g, A, B


def test_hand_example():
    g, A, Bt = _hand()
    ids = g["ids"].astype(int)
    act = g["active"].astype(int)
    rank = g["rank"].astype(int)
    y = L.linear(g["x"], g["W0"], ids, act, A, Bt, rank, g["scale"])
    assert np.array_equal(y, g["y"])
    v = L.shrink_rows(g["x"], ids, act, A, rank)
    assert np.array_equal(v[0], g["v_row0"]) and v[1, 0] == g["v_row1"] and v[1, 1] == 0
    assert np.all(v[2:] == 0)
    seg = oracle.build_segments(ids, act)
    assert list(seg["perm"]) == list(g["perm"].astype(int))
    assert list(seg["seg_start"]) == list(g["seg_start"].astype(int))
    assert list(seg["seg_adapter"]) == list(g["seg_adapter"].astype(int))


def _case(T=37, d_in=24, d_out=20, N=5, R_cap=6, seed=0, pad=np.nan):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, d_in))
    W0 = g.standard_normal((d_out, d_in))
    rank = g.integers(1, R_cap + 1, N)
    scale = g.uniform(0.25, 3, N)
    A = np.full((N, R_cap, d_in), pad)
    Bt = np.full((N, d_out, R_cap), pad)
    for a in range(N):
        A[a, :rank[a]] = g.standard_normal((rank[a], d_in))
        Bt[a, :, :rank[a]] = g.standard_normal((d_out, rank[a]))
    ids = g.integers(-1, N, T)
    act = (g.uniform(size=T) > 0.2).astype(np.uint8)
    return x, W0, ids, act, A, Bt, rank, scale


def test_merged_identity_single_adapter():
    x, W0, _, _, A, Bt, rank, scale = _case(pad=0.0)
    for a in range(A.shape[0]):
        ids = np.full(x.shape[0], a)
        y = L.linear(x, W0, ids, None, A, Bt, rank, scale)
        m = L.merged_linear(x, W0, A[a], Bt[a], int(rank[a]), float(scale[a]))
        assert np.abs(y - m).max() <= 1e-12 * np.abs(m).max()


def test_base_only_cases_are_exact():
    x, W0, ids, act, A, Bt, rank, scale = _case()
    base = x @ W0.T
    assert np.array_equal(L.linear(x, W0, np.full_like(ids, -1), act, A, Bt, rank, scale), base)
    assert np.array_equal(L.linear(x, W0, ids, np.zeros_like(act), A, Bt, rank, scale), base)
    Bz = np.where(np.isnan(Bt), np.nan, 0.0)
    y = L.linear(x, W0, ids, act, A, Bz, rank, scale)
    assert np.all(y == base)
    # rows that are not live are bit-identical to the base output
    y = L.linear(x, W0, ids, act, A, Bt, rank, scale)
    dead = ~L.live_rows(ids, act)
    assert np.array_equal(y[dead], base[dead])


def test_selector_closed_form():
    # A_a[j] = e_{k_j}, B_a[:, j] = e_{n_j}: delta[i, n_j] = s_a * x[i, k_j] exactly
    T, d_in, d_out, N, R = 8, 10, 9, 3, 4
    g = np.random.default_rng(5)
    x = g.integers(-8, 8, (T, d_in)).astype(np.float64)
    W0 = np.zeros((d_out, d_in))
    A = np.full((N, R, d_in), np.nan)
    Bt = np.full((N, d_out, R), np.nan)
    rank = np.array([1, 3, 4])
    scale = np.array([2.0, -0.5, 3.0])
    picks = {}
    for a in range(N):
        ks = g.choice(d_in, rank[a], replace=False)
        ns = g.choice(d_out, rank[a], replace=False)
        A[a, :rank[a]] = np.eye(d_in)[ks]
        Bt[a, :, :rank[a]] = np.eye(d_out)[ns].T
        picks[a] = (ks, ns)
    ids = np.array([0, 1, 2, -1, 2, 1, 0, 2])
    y = L.linear(x, W0, ids, None, A, Bt, rank, scale)
    want = np.zeros((T, d_out))
    for i, a in enumerate(ids):
        if a < 0:
            continue
        ks, ns = picks[a]
        for k, n in zip(ks, ns):
            want[i, n] = scale[a] * x[i, k]
    assert np.array_equal(y, want)


def test_row_permutation_invariance():
    x, W0, ids, act, A, Bt, rank, scale = _case(T=53, seed=2)
    y = L.linear(x, W0, ids, act, A, Bt, rank, scale)
    p = np.random.default_rng(9).permutation(len(ids))
    yp = L.linear(x[p], W0, ids[p], act[p], A, Bt, rank, scale)
    assert np.abs(yp - y[p]).max() <= 1e-12 * np.abs(y).max()


def test_three_formulations_agree():
    x, W0, ids, act, A, Bt, rank, scale = _case(T=41, seed=3)
    d1 = L.lora_delta(x, ids, act, A, Bt, rank, scale)
    d2 = L.lora_delta_per_row(x, ids, act, A, Bt, rank, scale)
    d3 = L.lora_delta_gathered(x, ids, act, A, Bt, rank, scale)
    ref = np.abs(d1).max()
    assert np.abs(d1 - d2).max() <= 1e-12 * ref
    assert np.abs(d1 - d3).max() <= 1e-12 * ref
    # v used by an expand-only check reproduces the same delta
    v = L.shrink_rows(x, ids, act, A, rank)
    d4 = L.lora_delta(x, ids, act, A, Bt, rank, scale, v_rows=v)
    assert np.abs(d1 - d4).max() <= 1e-12 * ref


def _brute(x, W0, ids, act, A, Bt, rank, scale):
    T, d_in = len(x), len(x[0])
    d_out = len(W0)
    y = [[0.0] * d_out for _ in range(T)]
    for i in range(T):
        for n in range(d_out):
            acc = 0.0
            for k in range(d_in):
                acc += float(W0[n][k]) * float(x[i][k])
            if ids[i] >= 0 and act[i]:
                a = int(ids[i])
                for j in range(int(rank[a])):
                    vj = 0.0
                    for k in range(d_in):
                        vj += float(A[a][j][k]) * float(x[i][k])
                    acc += float(scale[a]) * float(Bt[a][n][j]) * vj
            y[i][n] = acc
    return np.array(y)


def test_brute_force_tiny():
    args = _case(T=9, d_in=7, d_out=5, N=3, R_cap=3, seed=4)
    y = L.linear(*args[:2], *args[2:])
    b = _brute(*args)
    assert np.abs(y - b).max() <= 1e-12 * np.abs(b).max()


def test_padding_rows_never_read():
    x, W0, ids, act, A, Bt, rank, scale = _case(seed=6, pad=0.0)
    y0 = L.linear(x, W0, ids, act, A, Bt, rank, scale)
    A2, B2 = A.copy(), Bt.copy()
    for a in range(A.shape[0]):
        A2[a, rank[a]:] = np.nan
        B2[a, :, rank[a]:] = np.nan
    y1 = L.linear(x, W0, ids, act, A2, B2, rank, scale)
    assert np.array_equal(y0, y1)


def test_fp8_base_uses_dequantised_weights():
    from lora_inputs import e4m3_quantise_rows
    g = np.random.default_rng(8)
    w = (g.standard_normal((6, 32)) * 0.02).astype(np.float32)
    codes, s = e4m3_quantise_rows(w)
    x = g.standard_normal((3, 32))
    deq = oracle.decode_e4m3(codes) * s.astype(np.float64)[:, None]
    assert np.array_equal(L.base_output(x, (codes, s)), x @ deq.T)
    # dequantised weights are within half an e4m3 ulp of the fp32 draw
    assert np.all(np.abs(deq - w) <= 2.0 ** -4 * np.abs(w) + 2.0 ** -10 * s[:, None])


# --- planted mistakes -----------------------------------------------------

def _mutants():
    good = L.linear

    def no_scale(x, W0, ids, act, A, Bt, rank, scale):
        return good(x, W0, ids, act, A, Bt, rank, np.ones_like(scale))

    def wrong_sign(x, W0, ids, act, A, Bt, rank, scale):
        return good(x, W0, ids, act, A, Bt, rank, -np.asarray(scale))

    def transposed_base(x, W0, ids, act, A, Bt, rank, scale):
        y = good(x, W0, ids, act, A, Bt, rank, scale)
        return y - x @ np.asarray(W0).T + x @ np.asarray(W0)

    def rank_minus_one(x, W0, ids, act, A, Bt, rank, scale):
        return good(x, W0, ids, act, A, Bt, np.maximum(np.asarray(rank) - 1, 0), scale)

    def rank_plus_one(x, W0, ids, act, A, Bt, rank, scale):
        r = np.minimum(np.asarray(rank) + 1, np.asarray(A).shape[1])
        return good(x, W0, ids, act, A, Bt, r, scale)

    def adapter_off_by_one(x, W0, ids, act, A, Bt, rank, scale):
        ids2 = np.where(np.asarray(ids) >= 0, (np.asarray(ids) + 1) % np.asarray(A).shape[0], -1)
        return good(x, W0, ids2, act, A, Bt, rank, scale)

    def ignore_active(x, W0, ids, act, A, Bt, rank, scale):
        return good(x, W0, ids, None, A, Bt, rank, scale)

    def swapped_pools(x, W0, ids, act, A, Bt, rank, scale):
        # uses B^T's first d_in columns as the down-projection (square-ish mix-up)
        # B's rank columns read as if they were A's rank rows (square shapes)
        A2 = np.swapaxes(np.asarray(Bt), 1, 2) if np.asarray(Bt).shape[1] == np.asarray(x).shape[1] else A
        return good(x, W0, ids, act, A2, Bt, rank, scale)

    return [no_scale, wrong_sign, transposed_base, rank_minus_one, rank_plus_one,
            adapter_off_by_one, ignore_active, swapped_pools]


def _pins_pass(fn):
    """Re-run the value pins against ``fn``; return False on the first failure."""
    g, A, Bt = _hand()
    try:
        y = fn(g["x"], g["W0"], g["ids"].astype(int), g["active"].astype(int), A, Bt,
               g["rank"].astype(int), g["scale"])
        if not np.array_equal(y, g["y"]):
            return False
    except Exception:
        return False
    args = _case(T=9, d_in=7, d_out=7, N=3, R_cap=3, seed=4, pad=0.0)
    try:
        y = fn(*args)
    except Exception:
        return False
    b = _brute(*args)
    return bool(np.abs(y - b).max() <= 1e-12 * np.abs(b).max())


def test_pins_accept_the_oracle():
    assert _pins_pass(L.linear)


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_pins_catch_planted_mistakes(mutant):
    assert not _pins_pass(mutant)


# --- W8A8: per-token activation quantisation in the base product ------------
#
# EpiLoRA 2 and Fig. 4(a): y = (x_q W_q^T) s_x s_w for the base; 3 (K1, K2):
# the adapter's down-projection uses the unquantised activations.  Pinned by
# a hand-worked example (tests/golden/w8a8_hand_example.txt), by a closed
# form (rows that quantise exactly give the W8A16 result bit for bit), by the
# e4m3 rounding bound, and by planted mistakes that these pins must reject.

def _w8a8_hand():
    g = load("w8a8_hand_example.txt")
    codes = g["w_codes"].astype(np.uint8)
    s_w = g["w_scale"].astype(np.float32)
    A = np.asarray(g["A0"], np.float64).reshape(1, 1, 2)
    Bt = np.asarray(g["B0"], np.float64).reshape(1, 2, 1)
    ids = np.array([0, 0])
    act = np.array([1, 1], np.uint8)
    return g, codes, s_w, ids, act, A, Bt, np.array([1]), np.array([g["scale"]])


def test_w8a8_hand_example():
    g, codes, s_w, ids, act, A, Bt, rank, scale = _w8a8_hand()
    q, s_x = L.act_quant_e4m3(g["x"])
    assert np.array_equal(q, g["x_q_codes"].astype(np.uint8))
    assert np.array_equal(s_x.astype(np.float64), g["s_x"])
    y = L.linear_w8a8(g["x"], codes, s_w, ids, act, A, Bt, rank, scale)
    assert np.array_equal(y, g["y"])
    # without adapters the same call is the base product alone
    y0 = L.linear_w8a8(g["x"], codes, s_w, np.full(2, -1), act, A, Bt, rank, scale)
    assert np.array_equal(y0, g["base"])


def _exact_rows_case(seed=11, T=6, d_in=32, d_out=12):
    """Rows whose values are e4m3 values times 2^k with amax 448 * 2^k: each
    quantises exactly (s_x = 2^k, x / s_x on the e4m3 grid)."""
    from lora_inputs import e4m3_quantise_rows
    g = np.random.default_rng(seed)
    grid = oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))          # 0 .. 448
    x = np.empty((T, d_in))
    for i in range(T):
        v = g.choice(grid, d_in) * np.where(g.uniform(size=d_in) < 0.5, -1.0, 1.0)
        v[g.integers(d_in)] = 448.0 * (1 if i % 2 else -1)
        x[i] = v * 2.0 ** int(g.integers(-12, 3))
    codes, s_w = e4m3_quantise_rows((g.standard_normal((d_out, d_in)) * 0.02).astype(np.float32))
    N, R = 3, 4
    rank = np.array([4, 2, 3])
    A = np.full((N, R, d_in), np.nan)
    Bt = np.full((N, d_out, R), np.nan)
    for a in range(N):
        A[a, :rank[a]] = g.standard_normal((rank[a], d_in))
        Bt[a, :, :rank[a]] = g.standard_normal((d_out, rank[a]))
    ids = np.array([0, 2, -1, 1, 0, 2])[:T]
    act = np.array([1, 1, 1, 0, 1, 1], np.uint8)[:T]
    return x, codes, s_w, ids, act, A, Bt, rank, np.array([0.5, 2.0, -1.0])


def test_w8a8_exact_rows_equal_w8a16():
    x, codes, s_w, ids, act, A, Bt, rank, scale = _exact_rows_case()
    y8 = L.linear_w8a8(x, codes, s_w, ids, act, A, Bt, rank, scale)
    y16 = L.linear(x, (codes, s_w), ids, act, A, Bt, rank, scale)
    assert np.array_equal(y8, y16)


def test_w8a8_within_the_e4m3_rounding_bound():
    # |x - x_q| <= 2^-4 |x| (3 mantissa bits, round to nearest) + 2^-10 s_x
    # (half the subnormal spacing 2^-9), so the base moves by at most
    # sum_k |x_k - x_q,k| |W_nk|; the adapter term is unchanged.
    from lora_inputs import e4m3_quantise_rows
    g = np.random.default_rng(12)
    T, d_in, d_out = 9, 48, 10
    x = g.standard_normal((T, d_in)) * np.exp(g.uniform(-6, 6, (T, 1)))
    x = x.astype(np.float32).astype(np.float64)
    codes, s_w = e4m3_quantise_rows((g.standard_normal((d_out, d_in)) * 0.02).astype(np.float32))
    W = oracle.decode_e4m3(codes) * s_w.astype(np.float64)[:, None]
    N, R = 2, 2
    A = g.standard_normal((N, R, d_in))
    Bt = g.standard_normal((N, d_out, R))
    rank, scale = np.array([2, 1]), np.array([1.5, -0.5])
    ids = g.integers(-1, N, T)
    y8 = L.linear_w8a8(x, codes, s_w, ids, None, A, Bt, rank, scale)
    y16 = L.linear(x, (codes, s_w), ids, None, A, Bt, rank, scale)
    s_x = np.abs(x).max(axis=1) / 448.0
    bound = (2.0 ** -4 * np.abs(x) + 2.0 ** -10 * s_x[:, None]) @ np.abs(W).T
    assert np.all(np.abs(y8 - y16) <= bound * (1 + 1e-6))
    # the bound is not vacuous: the two differ somewhere
    assert np.abs(y8 - y16).max() > 0


def _w8a8_mutants():
    decode = oracle.decode_e4m3

    def lora_from_xq(x, codes, s_w, ids, act, A, Bt, rank, scale):
        q, s_x = L.act_quant_e4m3(x)
        xq = decode(q) * s_x.astype(np.float64)[:, None]
        return xq @ L.dequant_e4m3_rows(codes, s_w).T + L.lora_delta(xq, ids, act, A, Bt, rank, scale)

    def s_x_wrong_axis(x, codes, s_w, ids, act, A, Bt, rank, scale):
        q, s_x = L.act_quant_e4m3(x)
        xq = decode(q) * s_x.astype(np.float64)[None, :]
        return xq @ L.dequant_e4m3_rows(codes, s_w).T + L.lora_delta(x, ids, act, A, Bt, rank, scale)

    def no_s_w(x, codes, s_w, ids, act, A, Bt, rank, scale):
        q, s_x = L.act_quant_e4m3(x)
        xq = decode(q) * s_x.astype(np.float64)[:, None]
        return xq @ decode(codes).T + L.lora_delta(x, ids, act, A, Bt, rank, scale)

    def no_s_x(x, codes, s_w, ids, act, A, Bt, rank, scale):
        q, _ = L.act_quant_e4m3(x)
        return decode(q) @ L.dequant_e4m3_rows(codes, s_w).T + L.lora_delta(x, ids, act, A, Bt, rank, scale)

    def unquantised(x, codes, s_w, ids, act, A, Bt, rank, scale):
        return L.linear(x, (codes, s_w), ids, act, A, Bt, rank, scale)

    def no_adapter(x, codes, s_w, ids, act, A, Bt, rank, scale):
        q, s_x = L.act_quant_e4m3(x)
        xq = decode(q) * s_x.astype(np.float64)[:, None]
        return xq @ L.dequant_e4m3_rows(codes, s_w).T

    return [lora_from_xq, s_x_wrong_axis, no_s_w, no_s_x, unquantised, no_adapter]


def _w8a8_pins_pass(fn):
    g, codes, s_w, ids, act, A, Bt, rank, scale = _w8a8_hand()
    try:
        if not np.array_equal(fn(g["x"], codes, s_w, ids, act, A, Bt, rank, scale), g["y"]):
            return False
        x, codes, s_w, ids, act, A, Bt, rank, scale = _exact_rows_case()
        y = fn(x, codes, s_w, ids, act, A, Bt, rank, scale)
        return bool(np.array_equal(y, L.linear(x, (codes, s_w), ids, act, A, Bt, rank, scale)))
    except Exception:
        return False


def test_w8a8_pins_accept_the_oracle():
    assert _w8a8_pins_pass(L.linear_w8a8)


@pytest.mark.parametrize("mutant", _w8a8_mutants(), ids=lambda f: f.__name__)
def test_w8a8_pins_catch_planted_mistakes(mutant):
    assert not _w8a8_pins_pass(mutant)
