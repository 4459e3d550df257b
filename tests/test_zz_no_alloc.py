"""muon_step_noalloc (no context, scratch in a static device array) against
muon_step (the context's state buffer) on the same inputs, through the C ABI.

Calls in a row alternate a larger and a smaller set of matrices and both
branches (a refresh step and a RowNorm step each, one refresh of matrices
whose short side is 384, which the whole-triangle Gram kernel takes, and one
MuonBP block step), so every call finds the array holding the previous
call's different layout; the outputs must
match muon_step's to the tolerances of the optimizer's parity bar (momentum
and RowNorm 1e-5, bf16-MFMA NS5 2e-2, relative Frobenius of the update).
The same kernels run on the same values, so they are expected to match bit
for bit.  A matrix whose workspace does not fit is refused with
MUON_E_WORKSPACE and nothing enqueued.
"""

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

BIG = [(1000, 300), (512, 1536), (2200, 2048), (6144, 2048)]
SMALL = [(256, 512), (700, 300)]
TRI = [(384, 3072), (3072, 384), (384, 384)]    # short side 384: the whole-triangle Gram kernel


def _lib():
    import matrix_aware_optimizer_periodic_amd as m
    m.lib()
    return m


def rel(a, b):
    a = a.double().cpu().numpy()
    b = b.double().cpu().numpy()
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / nb if nb > 0 else np.linalg.norm(a - b)


def _inputs(shapes, seed):
    W0 = [torch.from_numpy(workloads.host_weight0(seed, i, s)).cuda() for i, s in enumerate(shapes)]
    M0 = [torch.from_numpy(workloads.host_grad(seed, 50, i, s, 1e-2, "f32")).cuda()
          for i, s in enumerate(shapes)]
    G = [torch.from_numpy(workloads.host_grad(seed, 51, i, s, 1e-3, "bf16")).to(torch.bfloat16).cuda()
         for i, s in enumerate(shapes)]
    return W0, M0, G


def _call_pair(m, shapes, t, seed, **over):
    W0, M0, G = _inputs(shapes, seed)
    cfg = m.muon_config_default(**over)
    # existing entry point
    Wr = [w.clone() for w in W0]
    sess = m.MuonSession(Wr, G, kinds=[m.MUON_KIND_MATRIX] * len(shapes), cfg=cfg)
    for i in range(len(shapes)):
        sess.state_view(i).copy_(M0[i])
    sess.step(t)
    torch.cuda.synchronize()
    Mr = [sess.state_view(i).clone() for i in range(len(shapes))]
    sess.close()
    # no-alloc entry point
    Wn = [w.clone() for w in W0]
    Mn = [x.clone() for x in M0]
    stream = torch.cuda.current_stream()
    m.muon_step_noalloc(cfg, [m.tensor_desc(w) for w in Wn],
                        [m.tensor_desc(g) for g in G], [m.tensor_desc(x) for x in Mn], t,
                        stream.cuda_stream)
    torch.cuda.synchronize()
    br = m.muon_branch(cfg, t)
    tol = 1e-5 if br == m.MUON_BRANCH_ROWNORM else 2e-2
    bitwise = True
    for i, s in enumerate(shapes):
        em = rel(Mn[i], Mr[i])
        ew = rel(Wn[i] - W0[i], Wr[i] - W0[i])
        same = torch.equal(Wn[i], Wr[i]) and torch.equal(Mn[i], Mr[i])
        bitwise &= same
        print(f"t={t} branch={br} {s}: momentum {em:.2e} update {ew:.2e} bitwise {same}", flush=True)
        assert em <= 1e-5 and ew <= tol, (s, em, ew)
    return bitwise


def test_noalloc_matches_muon_step_on_consecutive_calls():
    m = _lib()
    calls = [(BIG, 0, {}), (SMALL, 1, {}), (TRI, 3, {}), (BIG, 1, {}), (SMALL, 3, {}),
             ([(512, 1024), (1024, 512)], 2, dict(bp_blocks=8, bp_period=3))]
    same = [_call_pair(m, shapes, t, 20 + k, **over) for k, (shapes, t, over) in enumerate(calls)]
    print(f"bitwise equal per call: {same}", flush=True)


def test_noalloc_refuses_a_matrix_beyond_the_scratch():
    m = _lib()
    W = torch.zeros(3072, 18432, device="cuda")
    G = torch.zeros(3072, 18432, dtype=torch.bfloat16, device="cuda")
    M = torch.ones(3072, 18432, device="cuda")
    cfg = m.muon_config_default()
    with pytest.raises(m.MuonError) as e:
        m.muon_step_noalloc(cfg, [m.tensor_desc(W)], [m.tensor_desc(G)], [m.tensor_desc(M)], 0,
                            torch.cuda.current_stream().cuda_stream)
    assert e.value.status == m.binding.MUON_E_WORKSPACE
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert not torch.any(W) and torch.all(M == 1)
    # the array is still usable afterwards
    assert _call_pair(m, SMALL, 0, 40) is not None
