"""GPU parity: the HIP library through its C ABI against the fp64 oracle.

Protocol (per matrix, relative Frobenius error ||Y - Y*|| / ||Y*|| in fp64 on
the host, absolute when ||Y*|| = 0):
  * both sides run free from the same seeded inputs: the oracle keeps its own
    fp64 momentum and never sees a value computed on the GPU;
  * momentum M_t            <= 1e-5
  * direction U_t, read as -W_t / lr from a weight that is zero before the
    step:  RowNorm <= 1e-5, fp32-MFMA NS5 <= 1e-3, bf16-MFMA NS5 <= 2e-2;
  * branch indexing bit-exact (muon_branch, and the observed U: long-axis
    slice norms equal gamma exactly on RowNorm steps only).
"""

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

TOL_MOMENTUM = 1e-5
TOL_ROWNORM = 1e-5
TOL_NS5 = {0: 2e-2, 1: 1e-3, 2: 2e-2}     # ns_precision: bf16, f32, bf16 with X's remainder


def _lib():
    import matrix_aware_optimizer_periodic_amd as m
    m.lib()                        # raises if the HIP library is missing
    return m


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    d = np.linalg.norm(a - b)
    return d / nb if nb > 0 else d


def oracle_cfg(m, cfg):
    return oracle.OracleConfig(
        lr=float(np.float32(cfg.lr)), beta=float(np.float32(cfg.beta)),
        gamma=float(np.float32(cfg.gamma)), eps_row=float(np.float32(cfg.eps_row)), K=cfg.K,
        ns_iters=cfg.ns_iters, ns_a=float(np.float32(cfg.ns_a)),
        ns_b=float(np.float32(cfg.ns_b)), ns_c=float(np.float32(cfg.ns_c)),
        ns_eps=float(np.float32(cfg.ns_eps)), rownorm_axis=cfg.rownorm_axis,
        bp_blocks=cfg.bp_blocks, bp_period=cfg.bp_period,
        bp_lr_ratio=float(np.float32(cfg.bp_lr_ratio)), muon_wd=float(np.float32(cfg.muon_wd)),
        adam_lr=float(np.float32(cfg.adam_lr)), adam_b1=float(np.float32(cfg.adam_b1)),
        adam_b2=float(np.float32(cfg.adam_b2)), adam_eps=float(np.float32(cfg.adam_eps)),
        adam_wd=float(np.float32(cfg.adam_wd)))


def dir_tol(br, prec):
    return TOL_ROWNORM if br == oracle.BRANCH_ROWNORM else TOL_NS5[prec]


def run_direction_parity(shapes, steps, grad_dtype="bf16", grad_std=1e-3, seed=0,
                         shape_grads=None, **over):
    """Run `steps` steps with W zeroed before each; check M_t and U_t."""
    m = _lib()
    tdt = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    G = [torch.zeros(s, dtype=tdt, device="cuda") for s in shapes]
    sess = m.MuonSession(W, G, kinds=[m.MUON_KIND_MATRIX] * len(shapes), **over)
    try:
        return _direction_loop(sess, shapes, steps, W, G, tdt, grad_dtype, grad_std, seed,
                               shape_grads)
    finally:
        sess.close()


def _direction_loop(sess, shapes, steps, W, G, tdt, grad_dtype, grad_std, seed, shape_grads):
    m = _lib()
    ocfg = oracle_cfg(m, sess.cfg)
    Mo = [np.zeros(s) for s in shapes]
    worst = {}
    for t in range(steps):
        gh = []
        for i, s in enumerate(shapes):
            g = workloads.host_grad(seed, t, i, s, grad_std, grad_dtype)
            if shape_grads is not None:
                g = shape_grads(i, t, g)
            gh.append(g)
            G[i].copy_(torch.from_numpy(g).to(tdt))
            W[i].zero_()
        sess.step(t)
        torch.cuda.synchronize()
        br = sess.branch(t)
        assert br == oracle.branch(t, ocfg)
        for i, s in enumerate(shapes):
            Mo[i] = oracle.momentum_update(Mo[i], gh[i], ocfg.beta)
            Uo, lr = oracle.direction(Mo[i], t, ocfg)
            Ug = -W[i].double().cpu().numpy() / lr
            Mg = sess.state_view(i).double().cpu().numpy()
            em = rel(Mg, Mo[i])
            eu = rel(Ug, Uo)
            tol = dir_tol(br, sess.cfg.ns_precision)
            worst[(br, s)] = max(worst.get((br, s), 0.0), eu)
            print(f"t={t} shape={s} branch={br} momentum {em:.2e} direction {eu:.2e} "
                  f"(tol {tol:g})", flush=True)
            assert em <= TOL_MOMENTUM, f"t={t} shape={s} momentum err {em:.3e}"
            assert eu <= tol, f"t={t} shape={s} branch={br} direction err {eu:.3e} > {tol}"
            if br == oracle.BRANCH_ROWNORM:
                axis = 0 if (s[0] > s[1] and sess.cfg.rownorm_axis == 0) else 1
                norms = np.linalg.norm(Ug, axis=axis)
                live = np.linalg.norm(Mo[i], axis=axis) > ocfg.eps_row
                np.testing.assert_allclose(norms[live], ocfg.gamma, rtol=1e-5)
    return worst


# ------------------------------------------------------------------ single matrix
@pytest.mark.parametrize("prec", [0, 1])
def test_single_256x512_fp32_grads(prec):
    """256 x 512 fp32 weight, N(0,1) fp32 grads, 6 steps: 2 refreshes, 4 RowNorm."""
    wl = workloads.WORKLOADS["single-256x512"]
    shapes = [(m_, n_) for _, m_, n_ in wl.shapes]
    worst = run_direction_parity(shapes, wl.steps, grad_dtype="f32", grad_std=wl.grad_std,
                                 ns_precision=prec)
    print({k: f"{v:.2e}" for k, v in worst.items()})


def test_single_256x512_ns5_against_svd_polar_band():
    """The refresh direction shares its singular vectors with the SVD polar
    factor and its singular values follow the quintic's band."""
    m = _lib()
    W = torch.zeros(256, 512, device="cuda")
    g = workloads.host_grad(0, 0, 0, (256, 512), 1.0, "f32")
    G = torch.from_numpy(g).cuda()
    sess = m.MuonSession([W], [G], ns_precision=1)
    sess.step(0)
    torch.cuda.synchronize()
    U = -W.double().cpu().numpy() / np.float32(sess.cfg.lr)
    u, s, vt = np.linalg.svd(g.astype(np.float64), full_matrices=False)
    D = u.T @ U @ vt.T
    off = D - np.diag(np.diag(D))
    assert np.linalg.norm(off) / np.linalg.norm(D) < 1e-3
    x = s / (np.linalg.norm(g) + 1e-7)
    assert np.all((np.diag(D)[x > 5.2e-3] > 0.68) & (np.diag(D)[x > 5.2e-3] < 1.14))
    sess.close()


# wide r = 384 (whole-triangle Gram, 128 x 256 products), tall r = 700 (128-tiles), wide and tall
# r = 1100 (256-tiles, the tall last product through the mirror pass), tall r = 384
SPECTRUM_SHAPES = [(384, 1536), (1536, 700), (1100, 2600), (3000, 1100), (2000, 384)]


def test_refresh_on_spread_spectra():
    """Momenta whose singular values spread over decades (geometric to 1e-4
    and 1e-2, rank r/8 plus noise, one value 100x the rest), one refresh
    against the fp64 oracle.  bf16 storage of X loses the small singular
    directions that the a X term keeps growing; carrying X's bf16 remainder
    (MUON_NS_BF16_COMP) restores them to the bf16 bar, and fp32 holds its
    own.  Plain bf16 is printed: it exceeds 2e-2 on the spread spectra."""
    m = _lib()
    for kind in workloads.SPECTRA:
        for idx, s in enumerate(SPECTRUM_SHAPES):
            M = workloads.host_spectrum_matrix(5, idx, s, kind)
            ref = oracle.newton_schulz(M.astype(np.float64))
            errs = {}
            for prec in (0, 2, 1):
                W = torch.zeros(*s, device="cuda")
                G = torch.from_numpy(M).cuda()
                sess = m.MuonSession([W], [G], ns_precision=prec)
                sess.step(0)
                torch.cuda.synchronize()
                U = -W.double().cpu().numpy() / np.float32(sess.cfg.lr)
                sess.close()
                errs[prec] = rel(U, ref)
            print(f"{kind} {s}: bf16 {errs[0]:.2e}  bf16 + remainder {errs[2]:.2e}  fp32 {errs[1]:.2e}",
                  flush=True)
            assert errs[2] <= TOL_NS5[2] and errs[1] <= TOL_NS5[1], (kind, s, errs)
            assert errs[2] < errs[0] or errs[0] < 1e-2, (kind, s, errs)


@pytest.mark.parametrize("std", [1e-6, 1.0, 1e3])
def test_refresh_gradient_scale_sweep(std):
    """The polar factor of M equals that of kappa * M: a refresh step must
    match the oracle whatever the gradient's magnitude (the Frobenius
    pre-scale must reach every entry of X X^T and of X_1)."""
    shapes = [(256, 512), (512, 256), (300, 700), (1200, 1030)]
    for prec in (0, 1):
        run_direction_parity(shapes, 1, grad_dtype="f32", grad_std=std, seed=3, ns_precision=prec)


# ------------------------------------------------------------------ ragged sets
RAGGED = [(300, 700), (700, 300), (128, 128), (1, 64), (64, 1), (260, 260), (33, 2050),
          (2050, 33), (1200, 1030)]


@pytest.mark.parametrize("prec", [0, 1, 2])
def test_ragged_mixed_set(prec):
    """Tall, wide, square, single-row/column and non-tile-multiple shapes in
    one grouped launch set, bf16 grads, several tiles and ragged tails."""
    run_direction_parity(RAGGED, 6, ns_precision=prec)


TALL = [(1000, 300), (129, 4), (4096, 1024), (520, 516), (32768, 256), (2050, 512), (2200, 2048)]


@pytest.mark.parametrize("single", [1, 0])
@pytest.mark.parametrize("grad_dtype", ["bf16", "f32"])
def test_tall_rownorm_single_and_two_pass(single, grad_dtype):
    """Long-axis RowNorm of tall matrices in one pass (column statistics
    formed across workgroups) and in two passes, against the oracle: ragged
    last row chunk (1000, 129, 520, 2050, 2200 rows), a part-filled last
    column strip (300, 516 columns), a 4-column matrix, the largest strip the
    single pass takes (32768 rows = 128 chunks), and each column layout of a
    strip (contiguous for n % 128 != 0, runs a quarter row apart for 256, 512
    and 1024 columns, runs 512 columns apart for 2048).  No workgroup may give
    up waiting (muon_sync), and the single pass must be the kernel that ran."""
    m = _lib()
    shapes = TALL
    tdt = torch.bfloat16 if grad_dtype == "bf16" else torch.float32
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    G = [torch.zeros(s, dtype=tdt, device="cuda") for s in shapes]
    sess = m.MuonSession(W, G, kinds=[m.MUON_KIND_MATRIX] * len(shapes), tall_single_pass=single)
    try:
        m.muon_timing_enable(sess.ctx, True)
        _direction_loop(sess, shapes, 3, W, G, tdt, grad_dtype, 1e-3, 11, None)
        sess.sync()
        rec = m.muon_timing_read(sess.ctx)
        assert (rec["rownorm_tall"][1] > 0) == bool(single)
        assert (rec["rownorm_cols1"][1] > 0) == (not single)
        assert sess.tall_giveups() == 0
    finally:
        sess.close()


def test_tall_single_pass_forced_giveups_are_repaired():
    """With a poll limit of 0, every workgroup of the single-pass tall
    RowNorm that does not itself complete its strip stops waiting at once:
    it must leave its tile of W alone and list it, and the repair launch
    must write it.  W then matches the oracle on the same ragged and DiT
    shapes as above, and equals a run at the default limit bit for bit
    (same arithmetic, whichever launch writes a tile).  The limit is set from
    the host, so every kernel still exits normally."""
    m = _lib()
    shapes = [(1000, 300), (129, 4), (4096, 1024), (32768, 256), (2200, 2048), (6144, 2048)]
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    G = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    sess = m.MuonSession(W, G, kinds=[m.MUON_KIND_MATRIX] * len(shapes))
    try:
        m.muon_tall_poll_limit(sess.ctx, 0)
        m.muon_timing_enable(sess.ctx, True)
        _direction_loop(sess, shapes, 3, W, G, torch.bfloat16, "bf16", 1e-3, 12, None)
        rec = m.muon_timing_read(sess.ctx)
        gave = sess.tall_giveups()
        print(f"waits that gave up and were repaired: {gave}", flush=True)
        assert rec["rownorm_tall"][1] == 2 and rec["rownorm_repair"][1] == 2
        assert gave > 0
    finally:
        sess.close()
    out = {}
    for limit in (0, None):
        Wb = [torch.from_numpy(workloads.host_weight0(5, i, s)).cuda() for i, s in enumerate(shapes)]
        Gb = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
        sb = m.MuonSession(Wb, Gb, kinds=[m.MUON_KIND_MATRIX] * len(shapes), K=1000)
        try:
            if limit is not None:
                m.muon_tall_poll_limit(sb.ctx, limit)
            for t in range(1, 6):
                for i, s in enumerate(shapes):
                    Gb[i].copy_(torch.from_numpy(workloads.host_grad(5, t, i, s, 1e-3, "bf16")).to(
                        torch.bfloat16))
                sb.step(t)
            gave = sb.tall_giveups()
            assert (gave > 0) == (limit == 0), gave
            out[limit] = [w.clone() for w in Wb] + [sb.state_view(i).clone() for i in range(len(shapes))]
        finally:
            sb.close()
    for a, b in zip(out[0], out[None]):
        assert torch.equal(a, b)


def test_tall_single_pass_with_two_pass_fallback():
    """One context holding tall matrices the single pass takes (1000 x 300)
    and ones it leaves to the two-pass kernels: more than 32768 rows
    (33000 x 40) and an odd column count (700 x 301).  Both kernel families
    run in the same RowNorm step, and every matrix matches the oracle."""
    m = _lib()
    shapes = [(33000, 40), (700, 301), (1000, 300)]
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    G = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    sess = m.MuonSession(W, G, kinds=[m.MUON_KIND_MATRIX] * len(shapes))
    try:
        m.muon_timing_enable(sess.ctx, True)
        _direction_loop(sess, shapes, 3, W, G, torch.bfloat16, "bf16", 1e-3, 5, None)
        sess.sync()
        rec = m.muon_timing_read(sess.ctx)
        assert rec["rownorm_tall"][1] == 2 and rec["rownorm_cols1"][1] == 2
    finally:
        sess.close()


def test_tall_single_pass_repeated_launches():
    """Twenty RowNorm steps in a row on a set of tall matrices (DiT-1.3B
    qkv, adaLN and fc1 shapes among them, and 4200 x 4096, whose strips take
    runs from two 2048-column groups): the strip counters return to zero
    after every launch, so each step matches the two-pass kernels to fp32
    rounding of the column sums, and no wait gives up."""
    m = _lib()
    shapes = [(6144, 2048), (12288, 2048), (8192, 2048), (1536, 512), (700, 300), (4200, 4096)]
    out = {}
    for single in (1, 0):
        W = [torch.from_numpy(workloads.host_weight0(3, i, s)).cuda() for i, s in enumerate(shapes)]
        G = [torch.from_numpy(workloads.host_grad(3, 0, i, s, 1e-3, "bf16")).to(torch.bfloat16).cuda()
             for i, s in enumerate(shapes)]
        sess = m.MuonSession(W, G, kinds=[m.MUON_KIND_MATRIX] * len(shapes), K=1000,
                             tall_single_pass=single)
        try:
            for t in range(1, 21):
                sess.step(t)
            assert sess.tall_giveups() == 0
            out[single] = [w.double().cpu().numpy() for w in W]
        finally:
            sess.close()
    W0 = [workloads.host_weight0(3, i, s).astype(np.float64) for i, s in enumerate(shapes)]
    for a, b, w0 in zip(out[1], out[0], W0):
        assert rel(a - w0, b - w0) <= 1e-5


def test_long_ragged_rows():
    """Rows longer than 8 K values that end inside a 1024-value chunk: the
    wide RowNorm kernel's 16- and 32-chunk register variants (W loaded in
    batches after the row reduction, chunks past the row end re-read and
    dropped), next to a tall matrix with a ragged last row tile."""
    run_direction_parity([(3, 9000), (2, 20000), (5, 16388), (1030, 260)], 3, ns_precision=1)


def test_edge_values_zero_and_subthreshold_slices():
    """A zero gradient matrix, zero rows, and rows whose norm stays below eps."""
    shapes = [(64, 256), (256, 64), (40, 96)]

    def edit(i, t, g):
        g = g.copy()
        if i == 2:
            g[:] = 0.0
        else:
            if shapes[i][0] <= shapes[i][1]:
                g[3] = 0.0
                g[7] = workloads.round_to_bf16(g[7] * np.float32(1e-9))
            else:
                g[:, 3] = 0.0
                g[:, 7] = workloads.round_to_bf16(g[:, 7] * np.float32(1e-9))
        return g
    run_direction_parity(shapes, 6, shape_grads=edit, ns_precision=1)


def test_rownorm_stored_rows_mode():
    run_direction_parity([(512, 96), (96, 512), (257, 31)], 3, rownorm_axis=1)


@pytest.mark.parametrize("prec", [0, 1])
def test_other_ns_coefficients_and_iterations(prec):
    """A recorded variant: the convergent quintic (15/8, -5/4, 3/8) with 8
    iterations instead of the default coefficients and 5; also 3 iterations
    of the defaults.  The library takes them from the config like the oracle."""
    shapes = [(256, 640), (640, 256), (300, 700)]
    run_direction_parity(shapes, 2, ns_a=1.875, ns_b=-1.25, ns_c=0.375, ns_iters=8,
                         ns_precision=prec)
    run_direction_parity(shapes, 1, ns_iters=3, ns_precision=prec)


def test_vanilla_muon_K1():
    run_direction_parity([(256, 640), (640, 256)], 3, K=1, ns_precision=1)


def test_muonbp_blocks():
    """MuonBP: full NS5 every 3rd step, 8 column blocks orthogonalised on
    their own with half the step size otherwise."""
    run_direction_parity([(512, 1024), (1024, 512), (384, 384)], 6, bp_blocks=8, bp_period=3,
                         ns_precision=1)
    # bf16: also blocks with r = 384 (384 x 384 and, tall, 768 x 384), whose
    # Gram runs in one workgroup per block
    run_direction_parity([(512, 1024), (1024, 512), (384, 3072), (768, 3072)], 3, bp_blocks=8,
                         bp_period=3, ns_precision=0)
    # bf16 with X's remainder, on the same kinds of blocks
    run_direction_parity([(1024, 512), (384, 3072), (768, 3072)], 3, bp_blocks=8, bp_period=3,
                         ns_precision=2)


def test_workspace_cap_splits_the_refresh_into_chunks():
    """A workspace cap of 4 MiB splits the refresh into several chunks, each
    run through every Newton-Schulz round before the next starts; a problem
    larger than the cap (1200 x 1030) runs alone.  Under MuonBP, a 2 MiB cap
    splits the block steps too, with r = 384 blocks in them.  Every step
    matches the oracle as without the cap."""
    shapes = [(300, 700), (700, 300), (1200, 1030), (384, 3072), (260, 260), (512, 256)]
    run_direction_parity(shapes, 4, ns_workspace_max=4 << 20)
    run_direction_parity([(384, 3072), (768, 3072), (512, 1024)], 3, bp_blocks=8, bp_period=3,
                         ns_precision=0, ns_workspace_max=2 << 20)


def test_whole_triangle_gram_shapes():
    """bf16 problems whose short side pads to 384 (r from 257 to 384) take the
    Gram that computes all of A = X X^T in one workgroup: wide, tall and
    square, ragged r and c, c up to 18432 (576 k-steps), over two refreshes
    and the RowNorm steps between them, against the oracle."""
    shapes = [(384, 3072), (3072, 384), (384, 384), (257, 1000), (1000, 300), (384, 18432)]
    run_direction_parity(shapes, 4, ns_precision=0)


def test_long_rows_streaming_path():
    """Rows longer than the register-resident limit take the two-pass path."""
    run_direction_parity([(4, 40000), (3, 33001)], 3)


# ------------------------------------------------------------------ whole step
def test_weight_accumulation_and_decay_free_running():
    m = _lib()
    shapes = [(200, 520), (520, 200)]
    W0 = [workloads.host_weight0(0, i, s) for i, s in enumerate(shapes)]
    W = [torch.from_numpy(w).cuda() for w in W0]
    G = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    sess = m.MuonSession(W, G, muon_wd=0.01, ns_precision=1)
    ocfg = oracle_cfg(m, sess.cfg)
    Wo = [w.astype(np.float64) for w in W0]
    Mo = [np.zeros(s) for s in shapes]
    for t in range(6):
        for i, s in enumerate(shapes):
            g = workloads.host_grad(3, t, i, s, 1e-3, "bf16")
            G[i].copy_(torch.from_numpy(g).to(torch.bfloat16))
            Wo[i], Mo[i], _ = oracle.muon_matrix_step(Wo[i], Mo[i], g, t, ocfg)
        sess.step(t)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        Wg = W[i].double().cpu().numpy()
        assert rel(Wg - W0[i], Wo[i] - W0[i]) <= 1e-3
        assert rel(Wg, Wo[i]) <= 1e-5
    sess.close()


def test_adamw_tensors():
    m = _lib()
    sizes = [(1, 3), (1, 4096), (1, 5000), (1, 12289)]
    P0 = [workloads.host_weight0(1, i, s) for i, s in enumerate(sizes)]
    P = [torch.from_numpy(p).cuda().view(-1) for p in P0]
    G = [torch.zeros(s[1], dtype=torch.bfloat16 if i % 2 else torch.float32, device="cuda")
         for i, s in enumerate(sizes)]
    sess = m.MuonSession(P, G, adam_wd=0.01, adam_lr=3e-3)
    ocfg = oracle_cfg(m, sess.cfg)
    st = [(np.zeros(s[1]), np.zeros(s[1])) for s in sizes]
    po = [p.astype(np.float64).reshape(-1) for p in P0]
    for t in range(5):
        for i, s in enumerate(sizes):
            dt = "bf16" if i % 2 else "f32"
            g = workloads.host_grad(5, t, i, (s[1],), 1e-2, dt)
            G[i].copy_(torch.from_numpy(g).to(G[i].dtype))
            po[i], mo, vo = oracle.adamw_step(po[i], g, st[i][0], st[i][1], t, ocfg)
            st[i] = (mo, vo)
        sess.step(t)
    torch.cuda.synchronize()
    for i in range(len(sizes)):
        pg = P[i].double().cpu().numpy()
        assert rel(pg - P0[i].reshape(-1), po[i] - P0[i].reshape(-1)) <= 1e-5
        assert rel(sess.state_view(i, 0).double().cpu().numpy().reshape(-1), st[i][0]) <= 1e-5
        assert rel(sess.state_view(i, 1).double().cpu().numpy().reshape(-1), st[i][1]) <= 1e-5
    sess.close()


def _run_steps(m, shapes, steps, t0=0, state=None, **over):
    W = [torch.from_numpy(workloads.host_weight0(7, i, s)).cuda() for i, s in enumerate(shapes)]
    G = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    sess = m.MuonSession(W, G, **over)
    if state is not None:
        for i in range(len(shapes)):
            sess.state_view(i).copy_(state[1][i])
            W[i].copy_(state[0][i])
    for t in range(t0, t0 + steps):
        for i, s in enumerate(shapes):
            G[i].copy_(torch.from_numpy(workloads.host_grad(8, t, i, s, 1e-3, "bf16")).to(torch.bfloat16))
        sess.step(t)
    torch.cuda.synchronize()
    out = ([w.clone() for w in W], [sess.state_view(i).clone() for i in range(len(shapes))])
    sess.close()
    return out


def test_determinism_and_resume_bitwise():
    """Two runs are bitwise identical (no unordered reductions); 3 steps,
    checkpoint through muon_state views, fresh context, 3 more steps equals 6
    straight steps bitwise."""
    m = _lib()
    shapes = [(512, 1536), (1536, 512), (300, 700)]
    a = _run_steps(m, shapes, 6)
    b = _run_steps(m, shapes, 6)
    for x, y in zip(a[0] + a[1], b[0] + b[1]):
        assert torch.equal(x, y)
    half = _run_steps(m, shapes, 3)
    ckpt = ([w.cpu() for w in half[0]], [s.cpu() for s in half[1]])
    resumed = _run_steps(m, shapes, 3, t0=3, state=ckpt)
    for x, y in zip(a[0] + a[1], resumed[0] + resumed[1]):
        assert torch.equal(x, y)


def test_pointer_change_between_steps():
    """Passing other W / G buffers on a step patches the launch tables."""
    m = _lib()
    shapes = [(256, 512), (512, 256)]
    W1 = [torch.zeros(s, device="cuda") for s in shapes]
    G1 = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    sess = m.MuonSession(W1, G1, ns_precision=1)
    W2 = [torch.zeros(s, device="cuda") for s in shapes]
    G2 = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
    ocfg = oracle_cfg(m, sess.cfg)
    Mo = [np.zeros(s) for s in shapes]
    for t in range(4):
        Wt, Gt = (W1, G1) if t % 2 == 0 else (W2, G2)
        for i, s in enumerate(shapes):
            g = workloads.host_grad(9, t, i, s, 1e-3, "bf16")
            Gt[i].copy_(torch.from_numpy(g).to(torch.bfloat16))
            Wt[i].zero_()
            Mo[i] = oracle.momentum_update(Mo[i], g, ocfg.beta)
        sess.step(t, params=Wt, grads=Gt)
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            Uo, lr = oracle.direction(Mo[i], t, ocfg)
            assert rel(-Wt[i].double().cpu().numpy() / lr, Uo) <= dir_tol(sess.branch(t), 1)
    sess.close()


def test_step_validation_on_device_context():
    m = _lib()
    W = [torch.zeros(64, 128, device="cuda")]
    G = [torch.zeros(64, 128, dtype=torch.bfloat16, device="cuda")]
    sess = m.MuonSession(W, G)
    with pytest.raises(m.MuonError) as e:
        sess.step(-1)
    assert e.value.status == m.binding.MUON_E_ARG
    with pytest.raises(m.MuonError) as e:
        sess.step(0, grads=[torch.zeros(64, 128, device="cuda")])
    assert e.value.status == m.binding.MUON_E_DTYPE
    bad = m.tensor_desc(torch.zeros(64, 130, device="cuda"))
    with pytest.raises(m.MuonError) as e:
        m.muon_step(sess.ctx, [bad], sess.gdesc, 0)
    assert e.value.status == m.binding.MUON_E_SHAPE
    sess.close()


def test_empty_parameter_list():
    m = _lib()
    cfg = m.muon_config_default()
    assert m.muon_state_bytes(cfg, [], []) == 0
    ctx = m.muon_init(cfg, [], [], [], 0, 0, 0)
    m.muon_step(ctx, [], [], 0)
    m.muon_free(ctx)


# ------------------------------------------------------------------ full size
def _dit_full_set(m, wl, seed=0):
    dev = torch.device("cuda")
    shapes = [(a, b) for _, a, b in wl.shapes]
    params = [torch.zeros(s, device=dev) for s in shapes]
    grads = [torch.empty(s, dtype=torch.bfloat16, device=dev) for s in shapes]
    kinds = [m.MUON_KIND_MATRIX] * len(shapes)
    for b in range(wl.blocks):
        for j, L in enumerate(workloads.dit_bias_sizes(wl.d)):
            params.append(torch.zeros(L, device=dev))
            grads.append(torch.zeros(L, dtype=torch.bfloat16, device=dev))
            kinds.append(m.MUON_KIND_ADAMW)
    return shapes, params, grads, kinds


def _spectral_norm(X, iters=30):
    """Largest singular value of X by power iteration on X X^T (an estimate
    from below, which only tightens a bound that uses it)."""
    g = torch.Generator(device=X.device).manual_seed(1)
    v = torch.randn(X.shape[0], device=X.device, generator=g)
    for _ in range(iters):
        v = X @ (X.t() @ v)
        v = v / v.norm()
    return float((X.t() @ v).norm())


# workload -> (steps, compare every matrix with the oracle on RowNorm steps).
# Every set compares one matrix of each of the five shapes with the oracle on
# every step (full NS5, MuonBP block NS5 and RowNorm); DiT-1.3B also compares
# all of its 90 matrices, element by element, on its RowNorm steps.
FULL_SETS = {
    "dit-1.3b": (3, True),
    "dit-4b": (2, False),
    "dit-4b-muonbp": (3, False),
    "dit-15b": (2, False),
}


@pytest.mark.parametrize("name", list(FULL_SETS))
def test_dit_full_set_sampled(name):
    """The whole DiT-shaped set in one context, as the benchmark runs it
    (every W zeroed before each step, so U = -W / lr).

    * One matrix of each shape, from different blocks, is compared with the
      oracle (momentum and direction) on every step.
    * Every matrix, on a RowNorm step: each long-axis slice of U has norm
      gamma; on DiT-1.3B every matrix's momentum and direction are also
      compared with the oracle element by element (relative Frobenius 1e-5,
      one matrix at a time on the host).
    * Every matrix, on a full NS5 step: U = q(X X^T) X for the quintic's
      composed polynomial q, so X U^T (wide) / M^T U (tall) is symmetric; a
      misplaced tile, mirror or transposition breaks that.
    """
    m = _lib()
    wl = workloads.WORKLOADS[name]
    steps, rownorm_all = FULL_SETS[name]
    shapes, params, grads, kinds = _dit_full_set(m, wl)
    per = len(workloads.dit_block_shapes(wl.d))
    L = wl.blocks
    sample = {b * per + k: k for b, k in [(3 % L, 0), (L - 1, 1), (9 % L, 2), (0, 3), (11 % L, 4)]}
    tracked = range(len(shapes)) if rownorm_all else sorted(sample)
    sess = m.MuonSession(params, grads, kinds=kinds)
    try:
        ocfg = oracle_cfg(m, sess.cfg)
        tol_ns = TOL_NS5[sess.cfg.ns_precision]
        Mo = {i: np.zeros(shapes[i]) for i in tracked}
        for t in range(steps):
            for i, s in enumerate(shapes):
                workloads.device_normal_(grads[i], wl.grad_std, workloads.seed_for(0, t, i, 1))
                params[i].zero_()
            sess.step(t)
            sess.sync()
            br = sess.branch(t)
            assert br == oracle.branch(t, ocfg)
            lr = ocfg.lr * (ocfg.bp_lr_ratio if br == oracle.BRANCH_BLOCK_NS5 else 1.0)
            compared = 0
            for i in tracked:
                g = grads[i].float().cpu().double().numpy()
                Mo[i] = oracle.momentum_update(Mo[i], g, ocfg.beta)
                em = rel(sess.state_view(i).double().cpu().numpy(), Mo[i])
                assert em <= TOL_MOMENTUM, f"{name} t={t} matrix {i} momentum {em:.3e}"
                if i not in sample and br != oracle.BRANCH_ROWNORM:
                    continue
                compared += 1
                Uo, lr_o = oracle.direction(Mo[i], t, ocfg)
                assert abs(lr_o - lr) <= 1e-12
                Ug = -params[i].double().cpu().numpy() / lr
                eu = rel(Ug, Uo)
                if i in sample:
                    print(f"{name} t={t} matrix {i} {shapes[i]} branch {br}: momentum {em:.2e} "
                          f"direction {eu:.2e}", flush=True)
                assert eu <= dir_tol(br, sess.cfg.ns_precision), \
                    f"{name} t={t} matrix {i} direction {eu:.3e}"
                del Uo, Ug
            print(f"{name} t={t} branch {br}: {compared} matrices compared with the oracle, "
                  f"momentum of {len(tracked)}", flush=True)
            if br == oracle.BRANCH_ROWNORM:
                worst, where = 0.0, None
                for i, s in enumerate(shapes):
                    U = params[i].double() / -lr
                    norms = U.norm(dim=0 if s[0] > s[1] else 1)
                    dev = (norms - ocfg.gamma).abs() / ocfg.gamma
                    if float(dev.max()) > worst:
                        bad = torch.where(dev > 1e-5)[0]
                        worst, where = float(dev.max()), (i, s, len(bad), bad[:8].tolist())
                print(f"{name} t={t} RowNorm: worst slice-norm deviation {worst:.2e} "
                      f"(matrix, shape, slices over 1e-5, first ones: {where})", flush=True)
                assert worst <= 1e-5
            elif br == oracle.BRANCH_NS5:
                worst = 0.0
                for i, s in enumerate(shapes):
                    U = params[i] / -lr
                    M = sess.state_view(i)
                    if s[0] > s[1]:                      # wide orientation X = M^T
                        X, Uw = M.t().contiguous(), U.t().contiguous()
                    else:
                        X, Uw = M, U
                    S = X @ Uw.t().contiguous()
                    asym = float((S - S.t()).norm() / S.norm())
                    assert torch.isfinite(U).all()
                    # ||dU||_F <= eps ||U||_F gives ||X dU^T - dU X^T||_F <= 2 eps ||X||_2 ||U||_F
                    bound = 2 * tol_ns * _spectral_norm(X) * float(Uw.norm()) / float(S.norm())
                    assert asym <= bound, f"{name} matrix {i} {s}: asymmetry {asym:.3e} > {bound:.3e}"
                    worst = max(worst, asym / bound)
                    del S, X, Uw
                print(f"{name} t={t} NS5: worst asymmetry of X U^T / its bound {worst:.2e}",
                      flush=True)
        # the residency bound holds on an otherwise idle device: no wait gave up
        assert sess.tall_giveups() == 0
    finally:
        sess.close()
        del params, grads
        torch.cuda.empty_cache()


# ------------------------------------------------------------------ graph capture
def test_step_replays_from_hip_graphs():
    """muon_step only enqueues kernels (no allocation, no synchronisation), so
    each branch of a K-cycle can be captured once in a HIP graph and replayed.
    Replays, with eager gradient copies and synchronisations between them,
    must give bitwise the same weights and momentum as eager steps.  Only
    matrices here: an AdamW tensor's bias correction depends on t, which a
    captured launch would freeze."""
    m = _lib()
    shapes = [(256, 640), (640, 256), (300, 700)]
    K = 3
    W0 = [torch.from_numpy(workloads.host_weight0(4, i, s)).cuda() for i, s in enumerate(shapes)]

    def make():
        W = [w.clone() for w in W0]
        G = [torch.zeros(s, dtype=torch.bfloat16, device="cuda") for s in shapes]
        return W, G

    stream = torch.cuda.Stream()
    We, Ge = make()
    Wg, Gg = make()
    with torch.cuda.stream(stream):
        eager = m.MuonSession(We, Ge, stream=stream, K=K)
        graphed = m.MuonSession(Wg, Gg, stream=stream, K=K)
    graphs = []
    try:
        grads = lambda t: [torch.from_numpy(workloads.host_grad(6, t, i, s, 1e-3, "bf16")).to(
            torch.bfloat16).cuda() for i, s in enumerate(shapes)]
        # capture one step per branch position of the cycle, t = 0 .. K-1
        torch.cuda.synchronize()
        for t in range(K):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                graphed.step(t)
            graphs.append(g)
        torch.cuda.synchronize()
        for t in range(3 * K):
            gt = grads(t)
            for dst_e, dst_g, src in zip(Ge, Gg, gt):
                dst_e.copy_(src)
                dst_g.copy_(src)
            torch.cuda.synchronize()
            with torch.cuda.stream(stream):
                eager.step(t)
            graphs[t % K].replay()
            torch.cuda.synchronize()
            for i in range(len(shapes)):
                assert torch.equal(We[i], Wg[i]), f"t={t} matrix {i}: W differs"
                assert torch.equal(eager.state_view(i), graphed.state_view(i)), f"t={t} matrix {i}"
        print(f"{3 * K} graph replays match eager steps bitwise", flush=True)
    finally:
        del graphs
        eager.close()
        graphed.close()
