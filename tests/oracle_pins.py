"""Pins for the fp64 oracle: checks against what mathematics fixes, each
independent of the oracle's own code path.

Every ``check_*`` takes a loaded oracle library (``oracle.load(path)``) and
raises AssertionError on a mismatch. ``tests/test_oracle.py`` runs them on the
real oracle; ``tests/test_oracle_mutants.py`` runs them on deliberately broken
copies of the oracle source and requires that at least one fails, so that a
plausible mistake anywhere in the oracle is caught.

Nothing here comes from the HIP path. The pages ("[CUTLASS] Conv2d dgrad",
apache/tvm #10110, and the other pages) print no worked numerical example, so
the fixed values below are derived by hand from the definition of dgrad as the
adjoint of a strided, padded cross-correlation; each derivation is written out.
"""
from __future__ import annotations

import itertools

import numpy as np

import oracle

# ----------------------------------------------------------------- helpers


def f16(a):
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def forward_conv(x, w, stride, pad_h, pad_w=None):
    """Forward cross-correlation by slicing a zero-padded input (fp64):
    y[n,p,q,k] = sum_{r,t,c} xpad[n, p*s + r, q*s + t, c] * w[k,r,t,c]."""
    if pad_w is None:
        pad_w = pad_h
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N, H, W, C = x.shape
    K, R, S, C2 = w.shape
    assert C == C2
    P = (H + 2 * pad_h - R) // stride + 1
    Q = (W + 2 * pad_w - S) // stride + 1
    xp = np.zeros((N, H + 2 * pad_h, W + 2 * pad_w, C))
    xp[:, pad_h:pad_h + H, pad_w:pad_w + W, :] = x
    y = np.zeros((N, P, Q, K))
    for r in range(R):
        for t in range(S):
            patch = xp[:, r:r + stride * (P - 1) + 1:stride, t:t + stride * (Q - 1) + 1:stride, :]
            y += patch @ w[:, r, t, :].T
    return y


def scatter_dgrad(dy, w, H, W, stride, pad):
    """Brute force in the scatter direction: every dy element pushes
    dy[n,p,q,k] * w[k,r,t,:] to dx[n, p*s - pad + r, q*s - pad + t, :]
    when that position exists. No division or modulo anywhere."""
    dy = np.asarray(dy, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    N, P, Q, K = dy.shape
    _, R, S, C = w.shape
    dx = np.zeros((N, H, W, C))
    for n in range(N):
        for p in range(P):
            for q in range(Q):
                for r in range(R):
                    h = p * stride - pad + r
                    if h < 0 or h >= H:
                        continue
                    for t in range(S):
                        x = q * stride - pad + t
                        if x < 0 or x >= W:
                            continue
                        dx[n, h, x, :] += dy[n, p, q, :] @ w[:, r, t, :]
    return dx


def hardswish(z):
    """hardswish(z) = z * min(max(z + 3, 0), 6) / 6 (textbook form)."""
    return z * min(max(z + 3.0, 0.0), 6.0) / 6.0


def _ext(n, f, s, p):
    return (n + 2 * p - f) // s + 1


# ----------------------------------------------------------------- pins

W9 = np.arange(1, 10, dtype=np.float64).reshape(3, 3)   # [[1,2,3],[4,5,6],[7,8,9]]


def check_fp16_decode(lib):
    """Every one of the 65536 binary16 patterns decodes to numpy's value."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([lib.oracle_half_to_double(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def check_fp16_rne_encode(lib):
    """fp64 -> fp16 rounding equals numpy's correctly rounded (RNE) cast,
    on random values across the range, exact ties, subnormals, overflow."""
    rng = np.random.Generator(np.random.PCG64(3))
    vals = [rng.standard_normal(4000) * s for s in (1e-6, 1e-3, 1.0, 100.0, 3e4)]
    # exact ties: midpoints between neighbouring fp16 values
    h = np.arange(0, 0x7bff, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    hn = (np.arange(0, 0x7bff, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    mids = (h + hn) / 2
    specials = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 70000.0, -65520.0,
                         2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 2049.0, 2051.0, -2051.0])
    x = np.concatenate(vals + [mids, -mids, specials])
    got = oracle.round_to_half(x, lib=lib)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def check_out_extent(lib):
    """P = floor((H + 2 pad - R)/s) + 1, spot values worked by hand."""
    cases = {(56, 3, 2, 1): 28, (55, 3, 2, 1): 28, (56, 1, 2, 0): 28, (14, 3, 1, 1): 14,
             (7, 3, 1, 1): 7, (4, 3, 2, 1): 2, (3, 3, 2, 1): 2, (2, 3, 1, 0): 0, (1, 1, 3, 0): 1}
    for (n, f, s, p), want in cases.items():
        assert lib.oracle_out_extent(n, f, s, p) == want, (n, f, s, p)


def check_hand_examples(lib):
    """E1-E4: one channel, hand-worked from the definition.

    E1: 3x3 filter w = [[1,2,3],[4,5,6],[7,8,9]], stride 1, pad 1, H=W=3,
        dy = all ones (P=Q=3). dx[h,x] sums w[r,t] over r with 0 <= h+1-r < 3
        and t with 0 <= x+1-t < 3:
          corner (0,0): r,t in {0,1} -> 1+2+4+5 = 12
          edge   (0,1): r in {0,1}, t in {0,1,2} -> 1+2+3+4+5+6 = 21
          corner (0,2): r in {0,1}, t in {1,2} -> 2+3+5+6 = 16
          centre (1,1): all nine -> 45 ... and so on by symmetry.
        A filter-flip mistake gives 28 at (0,0) instead.
    E2: same w, one-hot dy at (1,1): dx[h,x] = w[h+1-1, x+1-1] = w[h,x], so dx = w.
        One-hot at (0,0): dx[h,x] = w[h+1, x+1] where defined -> [[5,6,0],[8,9,0],[0,0,0]].
    E3: stride 2, pad 1, H=W=4 (P=Q=2), dy = [[1,2],[3,4]].
        Row h takes taps r = h + 1 - 2p: h=0 -> (p=0,r=1); h=1 -> (p=0,r=2),(p=1,r=0);
        h=2 -> (p=1,r=1); h=3 -> (p=1,r=2). Columns likewise. E.g.
        dx[1,1] = sum over p,q in {0,1}: dy[p,q] * w[2-2p, 2-2q]
                = 1*9 + 2*7 + 3*3 + 4*1 = 36.
        With H=W=3 (still P=Q=2) dx is the top-left 3x3 block.
    E4: 1x1 filter w = 2, stride 2, pad 0, H=W=4, dy = [[1,2],[3,4]]:
        only even (h,x) are reached: dx[2p,2q] = 2*dy[p,q], zeros elsewhere.
    """
    w = f16(W9.reshape(1, 3, 3, 1))
    e1 = oracle.dgrad(f16(np.ones((1, 3, 3, 1))), w, 3, 3, 1, 1, lib=lib)[0, :, :, 0]
    assert np.array_equal(e1, [[12, 21, 16], [27, 45, 33], [24, 39, 28]])

    dy = np.zeros((1, 3, 3, 1))
    dy[0, 1, 1, 0] = 1
    assert np.array_equal(oracle.dgrad(f16(dy), w, 3, 3, 1, 1, lib=lib)[0, :, :, 0], W9)
    dy = np.zeros((1, 3, 3, 1))
    dy[0, 0, 0, 0] = 1
    assert np.array_equal(oracle.dgrad(f16(dy), w, 3, 3, 1, 1, lib=lib)[0, :, :, 0],
                          [[5, 6, 0], [8, 9, 0], [0, 0, 0]])

    dy = f16(np.array([[1, 2], [3, 4]]).reshape(1, 2, 2, 1))
    e3 = [[5, 14, 10, 12], [14, 36, 24, 30], [15, 34, 20, 24], [24, 55, 32, 36]]
    assert np.array_equal(oracle.dgrad(dy, w, 4, 4, 2, 1, lib=lib)[0, :, :, 0], e3)
    assert np.array_equal(oracle.dgrad(dy, w, 3, 3, 2, 1, lib=lib)[0, :, :, 0],
                          np.array(e3)[:3, :3])

    e4 = oracle.dgrad(dy, f16(np.full((1, 1, 1, 1), 2.0)), 4, 4, 2, 0, lib=lib)[0, :, :, 0]
    assert np.array_equal(e4, [[2, 0, 4, 0], [0, 0, 0, 0], [6, 0, 8, 0], [0, 0, 0, 0]])


def _scatter_cases():
    """A structured sweep over (R, stride, pad, H) plus random shapes
    covering N, W != H, S != R, C, K."""
    rng = np.random.Generator(np.random.PCG64(5))
    cases = []
    for R, s, pad, H in itertools.product((1, 2, 3), (1, 2, 3), (0, 1, 2), range(1, 7)):
        S = int(rng.integers(1, 4))
        W = int(rng.integers(1, 8))
        N = int(rng.integers(1, 3))
        C = int(rng.integers(1, 4))
        K = int(rng.integers(1, 4))
        cases.append((N, H, W, C, K, R, S, s, pad))
    for _ in range(120):
        R, S = (int(v) for v in rng.integers(1, 6, size=2))
        s = int(rng.integers(1, 5))
        pad = int(rng.integers(0, 3))
        H, W = (int(v) for v in rng.integers(1, 10, size=2))
        cases.append((int(rng.integers(1, 3)), H, W, int(rng.integers(1, 5)),
                      int(rng.integers(1, 5)), R, S, s, pad))
    return [c for c in cases if _ext(c[1], c[5], c[7], c[8]) >= 1 and _ext(c[2], c[6], c[7], c[8]) >= 1]


def check_scatter_bruteforce(lib, cases=None):
    """Integer-valued inputs: gather oracle == scatter brute force exactly."""
    rng = np.random.Generator(np.random.PCG64(6))
    for (N, H, W, C, K, R, S, s, pad) in (cases or _scatter_cases()):
        P, Q = _ext(H, R, s, pad), _ext(W, S, s, pad)
        dy = f16(rng.integers(-3, 4, size=(N, P, Q, K)))
        w = f16(rng.integers(-3, 4, size=(K, R, S, C)))
        got = oracle.dgrad(dy, w, H, W, s, pad, lib=lib)
        ref = scatter_dgrad(dy, w, H, W, s, pad)
        assert np.array_equal(got, ref), (N, H, W, C, K, R, S, s, pad)


def check_adjoint_identity(lib):
    """<fwd(x, w), dy> == <x, dgrad(dy, w)> to 1e-9 relative (fp64),
    the forward computed by slicing a padded input."""
    rng = np.random.Generator(np.random.PCG64(8))
    shapes = [(2, 9, 7, 5, 6, 3, 3, 2, 1), (1, 8, 8, 8, 8, 3, 3, 1, 1), (2, 11, 10, 3, 4, 5, 3, 3, 2),
              (1, 6, 9, 4, 4, 1, 1, 2, 0), (1, 7, 5, 2, 3, 2, 4, 2, 0), (3, 5, 5, 4, 2, 3, 3, 1, 0),
              (1, 13, 13, 3, 3, 7, 7, 4, 3)]
    for (N, H, W, C, K, R, S, s, pad) in shapes:
        P, Q = _ext(H, R, s, pad), _ext(W, S, s, pad)
        x = rng.standard_normal((N, H, W, C))
        dy = f16(rng.standard_normal((N, P, Q, K)))
        w = f16(rng.standard_normal((K, R, S, C)))
        lhs = np.sum(forward_conv(x, w, s, pad) * dy.astype(np.float64))
        rhs = np.sum(x * oracle.dgrad(dy, w, H, W, s, pad, lib=lib))
        assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(lhs)), (lhs, rhs)


def check_adjoint_unit_vectors(lib):
    """Build the forward operator column by column from unit inputs e_i and
    check dgrad(dy) == A^T dy entry by entry (the full transpose)."""
    rng = np.random.Generator(np.random.PCG64(9))
    for (N, H, W, C, K, R, S, s, pad) in [(1, 5, 4, 2, 3, 3, 2, 2, 1), (2, 4, 5, 2, 2, 3, 3, 1, 1),
                                          (1, 6, 6, 1, 2, 2, 2, 3, 1)]:
        P, Q = _ext(H, R, s, pad), _ext(W, S, s, pad)
        w = f16(rng.standard_normal((K, R, S, C)))
        dy = f16(rng.standard_normal((N, P, Q, K)))
        nx = N * H * W * C
        A = np.zeros((N * P * Q * K, nx))
        for i in range(nx):
            e = np.zeros(nx)
            e[i] = 1.0
            A[:, i] = forward_conv(e.reshape(N, H, W, C), w, s, pad).ravel()
        ref = A.T @ dy.astype(np.float64).ravel()
        got = oracle.dgrad(dy, w, H, W, s, pad, lib=lib).ravel()
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def check_matmul_special_cases(lib):
    """1x1 filters: stride 1 is a plain matmul dy[M,K] @ w[K,C]; stride s
    puts that product on the (s*p, s*q) lattice and zeros elsewhere."""
    rng = np.random.Generator(np.random.PCG64(10))
    N, H, W, C, K = 2, 5, 6, 7, 9
    dy = f16(rng.standard_normal((N, H, W, K)))
    w = f16(rng.standard_normal((K, 1, 1, C)))
    got = oracle.dgrad(dy, w, H, W, 1, 0, lib=lib)
    ref = (dy.astype(np.float64).reshape(-1, K) @ w.astype(np.float64).reshape(K, C)).reshape(N, H, W, C)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    for s, H, W in [(2, 7, 8), (3, 7, 9), (2, 6, 6)]:
        P, Q = _ext(H, 1, s, 0), _ext(W, 1, s, 0)
        dy = f16(rng.standard_normal((N, P, Q, K)))
        got = oracle.dgrad(dy, w, H, W, s, 0, lib=lib)
        ref = np.zeros((N, H, W, C))
        ref[:, ::s, ::s, :][:, :P, :Q, :] = (dy.astype(np.float64).reshape(-1, K)
                                             @ w.astype(np.float64).reshape(K, C)).reshape(N, P, Q, C)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
        mask = np.ones((H, W), bool)
        mask[::s, ::s] = False
        assert np.all(got[:, mask, :] == 0.0)


def check_stride1_flipped_forward(lib):
    """Stride 1: dgrad(dy, w, pad) is the forward correlation of dy with the
    filter rotated 180 degrees and in/out channels swapped,
    w'[c, r, t, k] = w[k, R-1-r, S-1-t, c], padded by R-1-pad and S-1-pad."""
    rng = np.random.Generator(np.random.PCG64(12))
    for (N, H, W, C, K, R, S, pad) in [(2, 6, 7, 3, 4, 3, 3, 1), (1, 8, 5, 2, 5, 3, 2, 0),
                                       (1, 9, 9, 4, 3, 5, 5, 2), (2, 5, 6, 3, 3, 4, 3, 1)]:
        P, Q = _ext(H, R, 1, pad), _ext(W, S, 1, pad)
        dy = f16(rng.standard_normal((N, P, Q, K)))
        w = f16(rng.standard_normal((K, R, S, C)))
        wflip = np.transpose(w.astype(np.float64)[:, ::-1, ::-1, :], (3, 1, 2, 0))
        ref = forward_conv(dy, wflip, 1, R - 1 - pad, S - 1 - pad)
        got = oracle.dgrad(dy, w, H, W, 1, pad, lib=lib)
        assert got.shape == ref.shape
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def check_torch_conv2d_input(lib):
    """Cross-check with PyTorch's CPU fp64 conv2d input gradient (NCHW)."""
    import torch
    rng = np.random.Generator(np.random.PCG64(13))
    for (N, H, W, C, K, R, S, s, pad) in [(2, 9, 8, 5, 6, 3, 3, 2, 1), (1, 14, 14, 8, 8, 3, 3, 1, 1),
                                          (2, 8, 8, 6, 4, 1, 1, 2, 0), (1, 11, 7, 3, 5, 5, 3, 3, 2),
                                          (1, 10, 10, 4, 4, 3, 3, 2, 0)]:
        P, Q = _ext(H, R, s, pad), _ext(W, S, s, pad)
        dy = f16(rng.standard_normal((N, P, Q, K)))
        w = f16(rng.standard_normal((K, R, S, C)))
        ref = torch.nn.grad.conv2d_input(
            (N, C, H, W),
            torch.from_numpy(w.astype(np.float64)).permute(0, 3, 1, 2).contiguous(),
            torch.from_numpy(dy.astype(np.float64)).permute(0, 3, 1, 2).contiguous(),
            stride=s, padding=pad).permute(0, 2, 3, 1).numpy()
        got = oracle.dgrad(dy, w, H, W, s, pad, lib=lib)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def check_epilogue_factors(lib):
    """relu'(z) = [z > 0] (0 at z = 0); hardswish'(z) from the textbook
    hardswish: 0 below -3, z/3 + 1/2 on [-3, 3] (closed, the reading at the
    kinks), 1 above 3. Away from the kinks it must match central finite
    differences of hardswish itself."""
    for zv, g in [(-4, 0), (-3, -0.5), (-1.5, 0), (0, 0.5), (1.5, 1), (3, 1.5), (4, 1), (-3.5, 0), (10, 1)]:
        assert lib.oracle_hardswish_grad(float(zv)) == g, zv
    for zv, g in [(-1, 0), (0, 0), (-0.0, 0), (1e-8, 1), (2, 1)]:
        assert lib.oracle_relu_grad(float(zv)) == g, zv
    rng = np.random.Generator(np.random.PCG64(14))
    hstep = 1e-5
    for zv in rng.uniform(-6, 6, 400):
        if min(abs(zv - 3), abs(zv + 3)) < 1e-3:
            continue
        fd = (hardswish(zv + hstep) - hardswish(zv - hstep)) / (2 * hstep)
        assert abs(fd - lib.oracle_hardswish_grad(float(zv))) < 1e-6, zv


def check_epilogue_applied(lib):
    """dgrad with an epilogue equals plain dgrad times g(z) elementwise, with
    g from the finite-difference-pinned closed forms above."""
    rng = np.random.Generator(np.random.PCG64(15))
    N, H, W, C, K, R, S, s, pad = 2, 6, 5, 4, 3, 3, 3, 2, 1
    P, Q = _ext(H, R, s, pad), _ext(W, S, s, pad)
    dy = f16(rng.standard_normal((N, P, Q, K)))
    w = f16(rng.standard_normal((K, R, S, C)))
    z = f16(rng.choice([-4, -3, -1.5, -0.25, 0, 0.75, 1.5, 3, 4], size=(N, H, W, C)))
    base = scatter_dgrad(dy, w, H, W, s, pad)
    zz = z.astype(np.float64)
    g_hs = np.where(zz < -3, 0.0, np.where(zz > 3, 1.0, zz / 3 + 0.5))
    g_relu = (zz > 0).astype(np.float64)
    assert np.allclose(oracle.dgrad(dy, w, H, W, s, pad, 2, z, lib=lib), base * g_hs, rtol=1e-12, atol=1e-12)
    assert np.allclose(oracle.dgrad(dy, w, H, W, s, pad, 1, z, lib=lib), base * g_relu, rtol=1e-12, atol=1e-12)


def check_rows_api(lib):
    """Sampled-row evaluation equals the matching rows of the full tensor."""
    rng = np.random.Generator(np.random.PCG64(16))
    N, H, W, C, K, R, S, s, pad = 2, 7, 6, 5, 4, 3, 3, 2, 1
    P, Q = _ext(H, R, s, pad), _ext(W, S, s, pad)
    dy = f16(rng.standard_normal((N, P, Q, K)))
    w = f16(rng.standard_normal((K, R, S, C)))
    z = f16(rng.standard_normal((N, H, W, C)))
    full = oracle.dgrad(dy, w, H, W, s, pad, 2, z, lib=lib).reshape(-1, C)
    rows = rng.choice(N * H * W, size=20, replace=False)
    part = oracle.dgrad(dy, w, H, W, s, pad, 2, z, rows=rows, lib=lib)
    assert np.array_equal(part, full[rows])


# ----------------------------------------------------------------- wgrad pins


def check_wgrad_hand_examples(lib):
    """Single channel, x = W9 = [[1,2,3],[4,5,6],[7,8,9]], worked by hand.

    (a) 3x3 filter, stride 1, no padding: P = Q = 1, so dw[r,t] = dy * x[r,t];
        with dy = 1 that is W9 itself.
    (b) 3x3 filter, stride 1, padding 1, dy = all ones (3x3): dw[r,t] sums x
        over the rows h = p - 1 + r and columns w = q - 1 + t that stay inside.
        r = 0 keeps rows 0-1, r = 1 all rows, r = 2 rows 1-2 (columns alike):
        [[1+2+4+5, 1+2+3+4+5+6, 2+3+5+6],
         [1+2+4+5+7+8, 45, 2+3+5+6+8+9],
         [4+5+7+8, 4+5+6+7+8+9, 5+6+8+9]] = [[12,21,16],[27,45,33],[24,39,28]].
    (c) 1x1 filter, stride 2, no padding: P = Q = 2 at x[0,0], x[0,2], x[2,0],
        x[2,2] = 1, 3, 7, 9; with dy = [[1,2],[3,4]], dw = 1 + 6 + 21 + 36 = 64.
    """
    x = f16(W9.reshape(1, 3, 3, 1))
    got = oracle.wgrad(f16(np.ones((1, 1, 1, 1))), x, 3, 3, 1, 0, lib=lib)
    assert np.array_equal(got.reshape(3, 3), W9)
    got = oracle.wgrad(f16(np.ones((1, 3, 3, 1))), x, 3, 3, 1, 1, lib=lib)
    assert np.array_equal(got.reshape(3, 3), np.array([[12, 21, 16], [27, 45, 33], [24, 39, 28]], float))
    got = oracle.wgrad(f16(np.array([[1, 2], [3, 4]]).reshape(1, 2, 2, 1)), x, 1, 1, 2, 0, lib=lib)
    assert got.reshape(()) == 64.0


WGRAD_CASES = [(2, 7, 6, 3, 4, 3, 3, 2, 1), (1, 8, 8, 2, 3, 3, 3, 1, 1), (2, 6, 7, 4, 2, 1, 1, 2, 0),
               (1, 9, 8, 3, 2, 5, 3, 3, 2), (1, 5, 5, 2, 2, 2, 4, 1, 0), (2, 10, 9, 2, 3, 3, 3, 2, 0)]


def _wgrad_inputs(rng, N, H, W, C, K, R, S, s, pad):
    P, Q = _ext(H, R, s, pad), _ext(W, S, s, pad)
    return f16(rng.standard_normal((N, P, Q, K))), f16(rng.standard_normal((N, H, W, C)))


def check_wgrad_adjoint_forward(lib):
    """<wgrad(dy, x), w> = <dy, forward(x, w)> for any w: wgrad is the
    adjoint of the map w -> forward(x, w); the forward here slices a padded x."""
    rng = np.random.Generator(np.random.PCG64(30))
    for (N, H, W, C, K, R, S, s, pad) in WGRAD_CASES:
        dy, x = _wgrad_inputs(rng, N, H, W, C, K, R, S, s, pad)
        w = rng.standard_normal((K, R, S, C))
        lhs = np.sum(oracle.wgrad(dy, x, R, S, s, pad, lib=lib) * w)
        rhs = np.sum(forward_conv(x, w, s, pad) * dy.astype(np.float64))
        assert np.isclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def check_wgrad_adjoint_dgrad(lib):
    """<wgrad(dy, x), w> = <dy, forward(x, w)> = <dgrad(dy, w), x>: the two
    gradients of one layer are tied through its forward."""
    rng = np.random.Generator(np.random.PCG64(31))
    for (N, H, W, C, K, R, S, s, pad) in WGRAD_CASES:
        dy, x = _wgrad_inputs(rng, N, H, W, C, K, R, S, s, pad)
        w = f16(rng.standard_normal((K, R, S, C)))
        lhs = np.sum(oracle.wgrad(dy, x, R, S, s, pad, lib=lib) * w.astype(np.float64))
        rhs = np.sum(oracle.dgrad(dy, w, H, W, s, pad, lib=lib) * x.astype(np.float64))
        assert np.isclose(lhs, rhs, rtol=1e-11, atol=1e-11)


def check_wgrad_unit_vectors(lib):
    """Build the map w -> forward(x, w) column by column from unit filters;
    wgrad(dy, x) must be its transpose applied to dy."""
    rng = np.random.Generator(np.random.PCG64(32))
    for (N, H, W, C, K, R, S, s, pad) in [(1, 5, 4, 2, 2, 3, 3, 2, 1), (2, 4, 5, 1, 3, 2, 3, 1, 0)]:
        dy, x = _wgrad_inputs(rng, N, H, W, C, K, R, S, s, pad)
        nw = K * R * S * C
        A = np.zeros((dy.size, nw))
        for i in range(nw):
            e = np.zeros(nw)
            e[i] = 1.0
            A[:, i] = forward_conv(x, e.reshape(K, R, S, C), s, pad).ravel()
        ref = (A.T @ dy.astype(np.float64).ravel()).reshape(K, R, S, C)
        assert np.allclose(oracle.wgrad(dy, x, R, S, s, pad, lib=lib), ref, rtol=1e-12, atol=1e-12)


def check_wgrad_matmul_special_cases(lib):
    """1x1 filters: stride 1 is dy[M,K]^T @ x[M,C]; stride s reads x on the
    (s*p, s*q) lattice only."""
    rng = np.random.Generator(np.random.PCG64(33))
    N, H, W, C, K = 2, 5, 6, 7, 9
    dy = f16(rng.standard_normal((N, H, W, K)))
    x = f16(rng.standard_normal((N, H, W, C)))
    got = oracle.wgrad(dy, x, 1, 1, 1, 0, lib=lib).reshape(K, C)
    ref = dy.astype(np.float64).reshape(-1, K).T @ x.astype(np.float64).reshape(-1, C)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)
    for s, H, W in [(2, 7, 8), (3, 7, 9)]:
        P, Q = _ext(H, 1, s, 0), _ext(W, 1, s, 0)
        dy = f16(rng.standard_normal((N, P, Q, K)))
        x = f16(rng.standard_normal((N, H, W, C)))
        got = oracle.wgrad(dy, x, 1, 1, s, 0, lib=lib).reshape(K, C)
        ref = dy.astype(np.float64).reshape(-1, K).T @ x.astype(np.float64)[:, ::s, ::s, :][:, :P, :Q, :].reshape(-1, C)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def check_wgrad_torch_conv2d_weight(lib):
    """Cross-check with PyTorch's CPU fp64 conv2d weight gradient (NCHW)."""
    import torch
    rng = np.random.Generator(np.random.PCG64(34))
    for (N, H, W, C, K, R, S, s, pad) in WGRAD_CASES:
        dy, x = _wgrad_inputs(rng, N, H, W, C, K, R, S, s, pad)
        ref = torch.nn.grad.conv2d_weight(
            torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2).contiguous(), (K, C, R, S),
            torch.from_numpy(dy.astype(np.float64)).permute(0, 3, 1, 2).contiguous(),
            stride=s, padding=pad).permute(0, 2, 3, 1).numpy()
        got = oracle.wgrad(dy, x, R, S, s, pad, lib=lib)
        assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def check_wgrad_rows_and_abs(lib):
    """Sampled filter rows equal the full result's rows, and the magnitude
    sums equal wgrad of |dy| and |x| (|d * v| = |d| * |v|)."""
    rng = np.random.Generator(np.random.PCG64(35))
    N, H, W, C, K, R, S, s, pad = 2, 7, 6, 5, 4, 3, 3, 2, 1
    dy, x = _wgrad_inputs(rng, N, H, W, C, K, R, S, s, pad)
    full, mag = oracle.wgrad(dy, x, R, S, s, pad, with_abs=True, lib=lib)
    rows = rng.choice(K * R * S, size=12, replace=False)
    part = oracle.wgrad(dy, x, R, S, s, pad, rows=rows, lib=lib)
    assert np.array_equal(part, full.reshape(-1, C)[rows])
    ref = oracle.wgrad(np.abs(dy), np.abs(x), R, S, s, pad, lib=lib)
    assert np.allclose(mag, ref, rtol=1e-12, atol=1e-12)
    assert np.all(mag >= np.abs(full) - 1e-12)


# ----------------------------------------------------------------- forward pins


def check_forward_hand_examples(lib):
    """x = W9 (one channel), 3x3 filter of ones, one output channel.

    No padding: z = bias + 45 (the sum of 1..9). With bias -40, z = 5 and
    hardswish(5) = 5 * min(8, 6) / 6 = 5; with bias -44, z = 1 and
    hardswish(1) = 1 * 4 / 6 = 2/3; with bias -50, z = -5 and hardswish = 0.
    Padding 1, bias 0: the 3x3 output is the window sums
    [[12, 21, 16], [27, 45, 33], [24, 39, 28]] (rows 0-1 / all / 1-2 and
    columns alike), and act = 0 returns z itself.
    """
    x = f16(W9.reshape(1, 3, 3, 1))
    w = f16(np.ones((1, 3, 3, 1)))
    for b, zz, yy in [(-40.0, 5.0, 5.0), (-44.0, 1.0, 2.0 / 3.0), (-50.0, -5.0, 0.0)]:
        z, y = oracle.forward(x, w, f16([b]), 1, 0, act=1, lib=lib)
        assert z.reshape(()) == zz and np.isclose(y.reshape(()), yy, rtol=0, atol=1e-15)
    z, y = oracle.forward(x, w, f16([0.0]), 1, 1, act=0, lib=lib)
    want = np.array([[12, 21, 16], [27, 45, 33], [24, 39, 28]], float)
    assert np.array_equal(z.reshape(3, 3), want) and np.array_equal(y.reshape(3, 3), want)


FWD_CASES = [(2, 7, 6, 3, 4, 3, 3, 2, 1), (1, 8, 8, 2, 3, 3, 3, 1, 1), (2, 6, 7, 4, 2, 1, 1, 2, 0),
             (1, 9, 8, 3, 2, 5, 3, 3, 2), (1, 5, 5, 2, 2, 2, 4, 1, 0)]


def _fwd_inputs(rng, N, H, W, C, K, R, S):
    return (f16(rng.standard_normal((N, H, W, C))), f16(rng.standard_normal((K, R, S, C))),
            f16(rng.standard_normal(K)))


def check_forward_vs_slicing(lib):
    """z equals the slicing forward plus bias, and y the textbook hardswish of z."""
    rng = np.random.Generator(np.random.PCG64(40))
    for (N, H, W, C, K, R, S, s, pad) in FWD_CASES:
        x, w, b = _fwd_inputs(rng, N, H, W, C, K, R, S)
        z, y = oracle.forward(x, w, b, s, pad, act=1, lib=lib)
        ref = forward_conv(x, w, s, pad) + b.astype(np.float64)
        assert np.allclose(z, ref, rtol=1e-12, atol=1e-12)
        assert np.allclose(y, np.vectorize(hardswish)(z), rtol=1e-15, atol=1e-15)


def check_forward_torch(lib):
    """Cross-check with PyTorch's CPU fp64 conv2d (NCHW) and hardswish."""
    import torch
    rng = np.random.Generator(np.random.PCG64(41))
    for (N, H, W, C, K, R, S, s, pad) in FWD_CASES:
        x, w, b = _fwd_inputs(rng, N, H, W, C, K, R, S)
        zt = torch.nn.functional.conv2d(
            torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2),
            torch.from_numpy(w.astype(np.float64)).permute(0, 3, 1, 2),
            torch.from_numpy(b.astype(np.float64)), stride=s, padding=pad)
        yt = torch.nn.functional.hardswish(zt)
        z, y = oracle.forward(x, w, b, s, pad, act=1, lib=lib)
        assert np.allclose(z, zt.permute(0, 2, 3, 1).numpy(), rtol=1e-12, atol=1e-12)
        assert np.allclose(y, yt.permute(0, 2, 3, 1).numpy(), rtol=1e-12, atol=1e-12)


def check_forward_adjoint_dgrad(lib):
    """<z - bias, dy> = <x, dgrad(dy, w)>: the forward's adjoint is the
    (separately pinned) dgrad."""
    rng = np.random.Generator(np.random.PCG64(42))
    for (N, H, W, C, K, R, S, s, pad) in FWD_CASES:
        x, w, b = _fwd_inputs(rng, N, H, W, C, K, R, S)
        z, _ = oracle.forward(x, w, b, s, pad, act=0, lib=lib)
        dy = f16(rng.standard_normal(z.shape))
        lhs = np.sum((z - b.astype(np.float64)) * dy.astype(np.float64))
        rhs = np.sum(x.astype(np.float64) * oracle.dgrad(dy, w, H, W, s, pad, lib=lib))
        assert np.isclose(lhs, rhs, rtol=1e-11, atol=1e-11)


# ------------------------------------------------- chain of two dgrad steps


def _grad_factor(epi, z):
    """relu'(z) = [z > 0]; hardswish'(z) = 0 below -3, z/3 + 1/2 on [-3, 3],
    1 above 3 (the textbook derivative of z * min(max(z + 3, 0), 6) / 6)."""
    z = np.asarray(z, dtype=np.float64)
    if epi == oracle.EPI_NONE:
        return np.ones_like(z)
    if epi == oracle.EPI_DRELU:
        return (z > 0).astype(np.float64)
    return np.where(z < -3, 0.0, np.where(z > 3, 1.0, z / 3 + 0.5))


def check_chain_hand_examples(lib):
    """One pixel, 1x1 filters, worked by hand.

    dy = 2, w1 = 3, w2 = [0.5, -1]: the first step gives 6; relu'(1) = 1
    keeps it, so dx = 6 * [0.5, -1] = [3, -6]. With hardswish' at z = 0 the
    factor is 1/2: t = 3 and dx = [1.5, -3], and sum |t||w2| = [1.5, 3].
    Rounding of t: K = 2, dy = [1, 1], w1 = [1, 2^-11] gives 1 + 2^-11, the
    midpoint between the fp16 neighbours 1 and 1 + 2^-10; ties to even give
    t = 1, so with w2 = 1 the chain yields exactly 1 (not 1 + 2^-11).
    """
    one = lambda v, shape: f16(np.asarray(v, dtype=np.float64).reshape(shape))
    dy, w1 = one([2.0], (1, 1, 1, 1)), one([3.0], (1, 1, 1, 1))
    w2 = one([0.5, -1.0], (1, 1, 1, 2))
    got = oracle.chain(dy, w1, one([1.0], (1, 1, 1, 1)), w2, 1, 1, 0, oracle.EPI_DRELU, lib=lib)
    assert np.array_equal(got.reshape(-1), [3.0, -6.0])
    got, mag = oracle.chain(dy, w1, one([0.0], (1, 1, 1, 1)), w2, 1, 1, 0, oracle.EPI_DHARDSWISH,
                            with_abs=True, lib=lib)
    assert np.array_equal(got.reshape(-1), [1.5, -3.0]) and np.array_equal(mag.reshape(-1), [1.5, 3.0])
    got = oracle.chain(one([1.0, 1.0], (1, 1, 1, 2)), one([1.0, 2.0 ** -11], (2, 1, 1, 1)), None,
                       one([1.0], (1, 1, 1, 1)), 1, 1, 0, lib=lib)
    assert got.reshape(-1)[0] == 1.0


CHAIN_CASES = [(2, 7, 6, 16, 8, 24, 3, 3, 1), (1, 5, 9, 8, 16, 8, 3, 3, 1), (1, 6, 6, 8, 8, 16, 1, 1, 0),
               (2, 4, 5, 24, 8, 16, 3, 3, 0), (1, 8, 7, 8, 24, 32, 5, 3, 2)]


def _chain_inputs(rng, N, H, W, Cm, K, C, R, S, pad):
    P, Q = _ext(H, R, 1, pad), _ext(W, S, 1, pad)
    dy = f16(rng.standard_normal((N, P, Q, K)))
    w1 = f16(rng.standard_normal((K, R, S, Cm)) / np.sqrt(K * R * S))
    z = f16(rng.standard_normal((N, H, W, Cm)) * 2.5)
    w2 = f16(rng.standard_normal((Cm, 1, 1, C)) / np.sqrt(Cm))
    return dy, w1, z, w2


def check_chain_torch(lib):
    """Cross-check with PyTorch's CPU fp64 input gradients: the RxS step,
    the textbook derivative factor, numpy's RNE cast of t to fp16, then the
    1x1 step, for every epilogue kind."""
    import torch
    rng = np.random.Generator(np.random.PCG64(61))
    for (N, H, W, Cm, K, C, R, S, pad) in CHAIN_CASES:
        dy, w1, z, w2 = _chain_inputs(rng, N, H, W, Cm, K, C, R, S, pad)
        a = torch.nn.grad.conv2d_input(
            (N, Cm, H, W), torch.from_numpy(w1.astype(np.float64)).permute(0, 3, 1, 2).contiguous(),
            torch.from_numpy(dy.astype(np.float64)).permute(0, 3, 1, 2).contiguous(),
            stride=1, padding=pad).permute(0, 2, 3, 1).numpy()
        for epi in (oracle.EPI_NONE, oracle.EPI_DRELU, oracle.EPI_DHARDSWISH):
            t = (a * _grad_factor(epi, z)).astype(np.float16).astype(np.float64)
            ref = torch.nn.grad.conv2d_input(
                (N, C, H, W), torch.from_numpy(w2.astype(np.float64)).permute(0, 3, 1, 2).contiguous(),
                torch.from_numpy(t).permute(0, 3, 1, 2).contiguous(), stride=1, padding=0).permute(0, 2, 3, 1).numpy()
            got = oracle.chain(dy, w1, z, w2, H, W, pad, epi, lib=lib)
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-12)


def check_chain_identity_second_step(lib):
    """With w2 the identity (C = Cm) the chain is the first step rounded to
    fp16, i.e. the separately pinned dgrad with its epilogue."""
    rng = np.random.Generator(np.random.PCG64(62))
    for (N, H, W, Cm, K, _, R, S, pad) in CHAIN_CASES[:3]:
        dy, w1, z, _ = _chain_inputs(rng, N, H, W, Cm, K, 8, R, S, pad)
        eye = f16(np.eye(Cm).reshape(Cm, 1, 1, Cm))
        for epi in (oracle.EPI_DRELU, oracle.EPI_DHARDSWISH):
            got = oracle.chain(dy, w1, z, eye, H, W, pad, epi, lib=lib)
            ref = oracle.dgrad(dy, w1, H, W, 1, pad, epi, z, lib=lib).astype(np.float16).astype(np.float64)
            assert np.array_equal(got, ref)


def check_chain_rows_and_abs(lib):
    """Sampled pixels equal the full result's rows; the magnitude sum bounds
    |dx| and equals it when every t and w2 is non-negative."""
    rng = np.random.Generator(np.random.PCG64(63))
    N, H, W, Cm, K, C, R, S, pad = CHAIN_CASES[0]
    dy, w1, z, w2 = _chain_inputs(rng, N, H, W, Cm, K, C, R, S, pad)
    full, mag = oracle.chain(dy, w1, z, w2, H, W, pad, oracle.EPI_DHARDSWISH, with_abs=True, lib=lib)
    rows = np.array([0, 5, N * H * W - 1, 17], dtype=np.int64)
    part, pmag = oracle.chain(dy, w1, z, w2, H, W, pad, oracle.EPI_DHARDSWISH, rows=rows, with_abs=True, lib=lib)
    assert np.array_equal(part, full.reshape(-1, C)[rows]) and np.array_equal(pmag, mag.reshape(-1, C)[rows])
    assert np.all(mag >= np.abs(full))
    got, mag = oracle.chain(f16(np.abs(dy)), f16(np.abs(w1)), None, f16(np.abs(w2)), H, W, pad,
                            with_abs=True, lib=lib)
    assert np.array_equal(got, mag)


ALL_CHECKS = [
    check_fp16_decode, check_fp16_rne_encode, check_out_extent, check_hand_examples,
    check_scatter_bruteforce, check_adjoint_identity, check_adjoint_unit_vectors,
    check_matmul_special_cases, check_stride1_flipped_forward, check_torch_conv2d_input,
    check_epilogue_factors, check_epilogue_applied, check_rows_api,
    check_wgrad_hand_examples, check_wgrad_adjoint_forward, check_wgrad_adjoint_dgrad,
    check_wgrad_unit_vectors, check_wgrad_matmul_special_cases, check_wgrad_torch_conv2d_weight,
    check_wgrad_rows_and_abs,
    check_forward_hand_examples, check_forward_vs_slicing, check_forward_torch, check_forward_adjoint_dgrad,
    check_chain_hand_examples, check_chain_torch, check_chain_identity_second_step, check_chain_rows_and_abs,
]


def run_all(lib) -> list:
    """Run every pin; return the names of those that failed (or raised)."""
    failed = []
    for chk in ALL_CHECKS:
        try:
            chk(lib)
        except Exception as e:  # noqa: BLE001 - a mutant may fail in any way
            failed.append(f"{chk.__name__}: {type(e).__name__}")
    return failed
