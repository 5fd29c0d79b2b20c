"""Pins for the oracle's fused Adam step with 16-bit packed moments.

"Training 10M Gaussians in 8 GB: Spirula Studio's VRAM efficiency" (mhpq.cn), quantised
training section: 16-bit moment codes with (min, max) bounds per 256 units.  The code format
is checked at its endpoints; the update against Adam's closed form for the first step and
against torch.optim.Adam (float64, CPU) over several steps, within the quantisation bound.
"""
import numpy as np
import torch

import oracle.adam as A

H = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8)


def test_codes_at_the_bounds():
    x = np.linspace(-3.0, 5.0, 300)  # two blocks: 256 + 44
    codes, lo, hi = A.encode_blocks(x)
    assert lo[0] == np.float32(-3.0) and hi[0] == np.float32(x[255])
    assert codes[0] == 0 and codes[255] == 65535 and codes[256] == 0 and codes[299] == 65535
    # a block of two values and their midpoint: rint(32767.5) = 32768 (ties to even)
    c, l, h = A.encode_blocks(np.array([0.0, 1.0, 0.5]))
    assert list(c) == [0, 65535, 32768]
    # constant block: code 0, bounds equal, decodes exactly
    c, l, h = A.encode_blocks(np.full(10, 0.25))
    assert np.all(c == 0) and l[0] == h[0] == np.float32(0.25)
    assert np.all(A.decode(c, l[0], h[0]) == 0.25)


def test_first_step_closed_form():
    rng = np.random.default_rng(1)
    U = 1000
    p = rng.normal(size=U).astype(np.float32)
    g = (rng.uniform(0.5, 2.0, U) * rng.choice([-1, 1], U)).astype(np.float32)
    nb = (U + 255) // 256
    p1, w1, b1 = A.adam_q16(p, g, np.zeros(U, np.uint32), np.zeros((nb, 4), np.float32), step=1, **H)
    # from zero moments: m_hat = g, v_hat = g^2, so the step is lr g / (|g| + eps)
    g64 = g.astype(np.float64)
    want = (p.astype(np.float64) - np.float32(H["lr"]) * g64 / (np.abs(g64) + np.float32(H["eps"]))).astype(np.float32)
    assert np.max(np.abs(p1.astype(np.float64) - want)) <= 2.0 ** -23 * 4


def test_steps_follow_torch_adam():
    rng = np.random.default_rng(2)
    U = 2048
    p0 = rng.normal(size=U)
    theta = torch.tensor(p0.astype(np.float32).astype(np.float64), requires_grad=True)
    opt = torch.optim.Adam([theta], lr=np.float32(H["lr"]).item(), betas=(np.float32(0.9).item(),
                           np.float32(0.999).item()), eps=np.float32(H["eps"]).item())
    p = p0.astype(np.float32)
    w = np.zeros(U, np.uint32)
    b = np.zeros((U // 256, 4), np.float32)
    err_m = err_v = np.zeros(U)  # bound on the decoded moments' distance from unquantised Adam
    for t in range(1, 6):
        g = (rng.uniform(0.5, 2.0, U) * rng.choice([-1, 1], U)).astype(np.float32)
        theta.grad = torch.tensor(g.astype(np.float64))
        opt.step()
        p, w, b = A.adam_q16(p, g, w, b, step=t, **H)
        # decoded moments against torch's: each step adds at most half a code step (plus the
        # float32 rounding of the bounds) to the previous error, which decays by beta
        st = opt.state[theta]
        blk = np.arange(U) // 256
        m = A.decode(w & 0xFFFF, b[blk, 0], b[blk, 1])
        v = A.decode(w >> 16, b[blk, 2], b[blk, 3])
        step_m = (b[blk, 1].astype(np.float64) - b[blk, 0]) / 65535.0
        step_v = (b[blk, 3].astype(np.float64) - b[blk, 2]) / 65535.0
        err_m = 0.9 * err_m + 0.5 * step_m + 2e-7 * np.abs(m) + 1e-12
        err_v = 0.999 * err_v + 0.5 * step_v + 2e-7 * np.abs(v) + 1e-12
        assert np.all(np.abs(m - st["exp_avg"].numpy()) <= err_m), t
        assert np.all(np.abs(v - st["exp_avg_sq"].numpy()) <= err_v), t
    # parameters: every moment error above is < 2e-5 relative here, so the trajectories agree
    # to a small fraction of one step (lr = 1e-2)
    assert np.max(np.abs(p.astype(np.float64) - theta.detach().numpy())) < 1e-4


def test_empty():
    p, w, b = A.adam_q16(np.zeros(0, np.float32), np.zeros(0, np.float32), np.zeros(0, np.uint32),
                         np.zeros((0, 4), np.float32), step=1, **H)
    assert p.shape == (0,) and w.shape == (0,) and b.shape == (0, 4)


# --- parameters packed too (adam_fpbo) ---------------------------------------------------------


def test_fpbo_pack_layout_and_round_trip():
    rng = np.random.default_rng(3)
    U = 600  # blocks of 256, 256 and 88
    p = rng.normal(size=U).astype(np.float32)
    st, bd = A.fpbo_pack(p)
    assert st.shape == (3, 3, 256) and st.dtype == np.uint16 and bd.shape == (3, 6)
    # moments start at zero; the padding past the last unit is zero
    assert not st[:, 1:, :].any() and not bd[:, 2:].any() and not st[2, 0, 88:].any()
    for b in range(3):
        seg = p[256 * b:256 * b + 256]
        assert bd[b, 0] == seg.min() and bd[b, 1] == seg.max()
        assert st[b, 0, np.argmin(seg)] == 0 and st[b, 0, np.argmax(seg)] == 65535
    # every parameter decodes within half a code step of its float32 value
    blk = np.arange(U) // 256
    half = (bd[blk, 1].astype(np.float64) - bd[blk, 0]) / 65535.0 / 2
    dec = A.fpbo_decode_params(st, bd, U)
    assert np.all(np.abs(dec.astype(np.float64) - p) <= half * (1 + 1e-9) + np.spacing(np.abs(p)))
    # a constant block keeps its value exactly
    st, bd = A.fpbo_pack(np.full(5, -1.5, np.float32))
    assert np.all(st[0, 0] == 0) and bd[0, 0] == bd[0, 1] == np.float32(-1.5)
    assert np.all(A.fpbo_decode_params(st, bd, 5) == np.float32(-1.5))


def test_fpbo_first_step_closed_form():
    rng = np.random.default_rng(4)
    U = 1000
    p = rng.normal(size=U).astype(np.float32)
    g = (rng.uniform(0.5, 2.0, U) * rng.choice([-1, 1], U)).astype(np.float32)
    st, bd = A.fpbo_pack(p)
    theta0 = A.fpbo_decode_params(st, bd, U).astype(np.float64)
    st1, bd1, p1 = A.adam_fpbo(st, bd, g, step=1, **H)
    # from zero moments: m_hat = g, v_hat = g^2, so the parameter moves by lr g / (|g| + eps);
    # the stored result is that value to within half a code step of its new block
    g64 = g.astype(np.float64)
    want = theta0 - np.float32(H["lr"]) * g64 / (np.abs(g64) + np.float32(H["eps"]))
    blk = np.arange(U) // 256
    half = (bd1[blk, 1].astype(np.float64) - bd1[blk, 0]) / 65535.0 / 2
    assert np.all(np.abs(p1.astype(np.float64) - want) <= half * (1 + 1e-6) + np.spacing(np.abs(want)))
    # the new bounds are the extremes of the new parameters (rounded to float32)
    for b in range(bd1.shape[0]):
        seg = want[256 * b:256 * b + 256]
        assert abs(bd1[b, 0] - seg.min()) <= abs(np.spacing(np.float32(seg.min()))) + 1e-12
        assert abs(bd1[b, 1] - seg.max()) <= abs(np.spacing(np.float32(seg.max()))) + 1e-12
    # first moment after one step is (1 - b1) g: its codes sit at the block's two ends when
    # the gradients of a block take just two values
    st2, bd2, _ = A.adam_fpbo(st, bd, np.where(np.arange(U) % 2, 1.0, -1.0).astype(np.float32), step=1, **H)
    assert set(np.unique(st2[:3, 1, :])) == {0, 65535}
    assert bd2[0, 2] == np.float32(-0.1 * 1.0) or abs(bd2[0, 2] + 0.1) < 1e-7


def test_fpbo_steps_follow_torch_adam():
    rng = np.random.default_rng(5)
    U = 2048
    p0 = rng.normal(size=U).astype(np.float32)
    st, bd = A.fpbo_pack(p0)
    p = A.fpbo_decode_params(st, bd, U)
    theta = torch.tensor(p.astype(np.float64), requires_grad=True)
    opt = torch.optim.Adam([theta], lr=np.float32(H["lr"]).item(), betas=(np.float32(0.9).item(),
                           np.float32(0.999).item()), eps=np.float32(H["eps"]).item())
    drift = 0.0
    for t in range(1, 6):
        g = (rng.uniform(0.5, 2.0, U) * rng.choice([-1, 1], U)).astype(np.float32)
        theta.grad = torch.tensor(g.astype(np.float64))
        opt.step()
        st, bd, p = A.adam_fpbo(st, bd, g, step=t, **H)
        # each step stores the parameter to within half a code step (~5.5 / 65535 / 2 for these
        # N(0, 1) blocks), and the quantised moments move the update by far less than that here
        blk = np.arange(U) // 256
        drift += np.max((bd[blk, 1].astype(np.float64) - bd[blk, 0]) / 65535.0 / 2) + 2e-6
        assert np.max(np.abs(p.astype(np.float64) - theta.detach().numpy())) <= drift, t
    # the moments against torch's, as in the moments-only form
    mm = st[:, 1, :].reshape(-1)[:U]
    m = A.decode(mm, bd[blk, 2], bd[blk, 3])
    step_m = (bd[blk, 3].astype(np.float64) - bd[blk, 2]) / 65535.0
    assert np.max(np.abs(m - opt.state[theta]["exp_avg"].numpy()) / step_m) < 4.0


def test_fpbo_empty():
    st, bd = A.fpbo_pack(np.zeros(0, np.float32))
    assert st.shape == (0, 3, 256) and bd.shape == (0, 6)
    st, bd, p = A.adam_fpbo(st, bd, np.zeros(0, np.float32), step=1, **H)
    assert st.shape == (0, 3, 256) and p.shape == (0,)
