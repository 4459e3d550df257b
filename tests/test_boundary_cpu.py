"""The C-ABI library on the CPU: it loads, exports what include/muon.h
declares, and its host-side logic (defaults, branch schedule, sizing and
argument validation) behaves as documented.  Nothing here launches a kernel;
every muon_init call below fails validation before touching a device.
"""

import os
import re

import pytest

import oracle
import workloads

m = pytest.importorskip("matrix_aware_optimizer_periodic_amd")
HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "muon.h")

# Skip only when the library was never built; a built library that does not
# load is an error.
HAVE_LIB = os.path.exists(os.path.join(os.path.dirname(m.__file__), "libmuon_hip.so"))
if HAVE_LIB:
    m.lib()
pytestmark = pytest.mark.skipif(not HAVE_LIB, reason="libmuon_hip.so not built")

FAKE = 0x10000  # aligned stand-in address, never dereferenced by validation


def desc(rows, cols, dtype=m.MUON_F32, ptr=FAKE):
    return m.MuonTensor(ptr, rows, cols, cols, dtype, 0)


def test_exports_every_declared_function():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const char\*|muon_status|int32_t|void)\s+(muon_\w+)\s*\(",
                              text, re.M))
    assert declared == set(m.EXPORTED)
    lib = m.lib()
    for name in declared:
        assert hasattr(lib, name), name


def test_kernel_classes_follow_the_header_enum():
    text = open(HEADER).read()
    pairs = re.findall(r"^\s*MUON_K_(\w+)\s*=\s*(\d+)", text, re.M)
    enum = {name.lower(): int(v) for name, v in pairs}
    count = enum.pop("count")
    assert count == len(m.KERNEL_CLASSES)
    assert [n for n, _ in sorted(enum.items(), key=lambda kv: kv[1])] == list(m.KERNEL_CLASSES)


def test_defaults_match_the_pages_and_the_oracle():
    c = m.muon_config_default()
    o = oracle.OracleConfig()
    assert c.K == o.K == 3
    assert abs(c.gamma - o.gamma) < 1e-7
    for f in ("lr", "beta", "eps_row", "ns_a", "ns_b", "ns_c", "ns_eps", "adam_lr", "adam_b1",
              "adam_b2", "adam_eps", "bp_lr_ratio"):
        assert abs(getattr(c, f) - getattr(o, f)) <= 1e-6 * max(1.0, abs(getattr(o, f))), f
    assert c.ns_iters == o.ns_iters and c.bp_period == o.bp_period
    assert c.tall_single_pass == 1 and c.reserved0 == 0


def test_state_bytes_do_not_depend_on_the_tall_rownorm_form():
    """The state buffer holds the tables and partial sums of both tall
    RowNorm forms (the device decides at init which matrices take the single
    pass), so its size is a host-only function of the shapes: the same with
    the single pass on or off, and larger than the two-pass form alone would
    need for tall matrices whose single-pass partials take more room."""
    wl = workloads.WORKLOADS["dit-1.3b"]
    ps = [desc(a, b) for _, a, b in wl.shapes]
    on = m.muon_state_bytes(m.muon_config_default(), ps, [0] * len(ps))
    off = m.muon_state_bytes(m.muon_config_default(tall_single_pass=0), ps, [0] * len(ps))
    assert on >= off
    # wide matrices and tall ones the single pass cannot take size the same either way
    for shape in [(2048, 8192), (700, 301), (33000, 40)]:
        a = m.muon_state_bytes(m.muon_config_default(), [desc(*shape)], [0])
        b = m.muon_state_bytes(m.muon_config_default(tall_single_pass=0), [desc(*shape)], [0])
        assert a == b, shape


@pytest.mark.parametrize("K", [1, 2, 3, 4, 7])
def test_branch_indexing_is_bit_exact_with_the_oracle(K):
    c = m.muon_config_default(K=K)
    o = oracle.OracleConfig(K=K)
    for t in list(range(50)) + [2 ** 31 + 5, 2 ** 40 + 3]:
        assert m.muon_branch(c, t) == oracle.branch(t, o)


def test_branch_muonbp_and_invalid():
    c = m.muon_config_default(bp_blocks=8, bp_period=3)
    o = oracle.OracleConfig(bp_blocks=8, bp_period=3)
    assert [m.muon_branch(c, t) for t in range(30)] == [oracle.branch(t, o) for t in range(30)]
    assert m.muon_branch(c, -1) == -1
    assert m.muon_branch(m.muon_config_default(K=0), 0) == -1


def test_status_strings():
    for s in range(8):
        assert m.muon_status_str(s)
    assert m.muon_status_str(99) == "unknown status"


def test_state_bytes_counts_state_and_workspace():
    c = m.muon_config_default()
    assert m.muon_state_bytes(c, [], []) == 0
    wl = workloads.WORKLOADS["dit-1.3b"]
    ps = [desc(a, b) for _, a, b in wl.shapes]
    nbytes = m.muon_state_bytes(c, ps, [m.MUON_KIND_MATRIX] * len(ps))
    assert nbytes >= 4 * wl.elements + 4 * wl.elements   # momentum + two bf16 X buffers
    c32 = m.muon_config_default(ns_precision=m.MUON_NS_F32)
    assert m.muon_state_bytes(c32, ps, [0] * len(ps)) > nbytes
    # bf16 with X's remainder: one more bf16 copy of every X (no cap: one chunk,
    # and every DiT X is a whole number of 256-byte blocks)
    comp = m.muon_config_default(ns_precision=m.MUON_NS_BF16_COMP)
    assert m.muon_state_bytes(comp, ps, [0] * len(ps)) == nbytes + 2 * wl.elements
    adam = m.muon_state_bytes(c, [desc(1, 1000)], [m.MUON_KIND_ADAMW])
    assert 8000 <= adam < 8000 + 4096
    # a workspace cap splits the NS5 work and shrinks the buffer
    capped = m.muon_config_default(ns_workspace_max=1 << 30)
    assert m.muon_state_bytes(capped, ps, [0] * len(ps)) < nbytes


@pytest.mark.parametrize("bad,status", [
    (dict(rows=0), m.binding.MUON_E_SHAPE),
    (dict(cols=-3), m.binding.MUON_E_SHAPE),
    (dict(ld=7), m.binding.MUON_E_ALIGN),
    (dict(dtype=m.MUON_BF16), m.binding.MUON_E_DTYPE),
    (dict(dtype=5), m.binding.MUON_E_DTYPE),
    (dict(reserved=1), m.binding.MUON_E_SHAPE),
])
def test_state_bytes_rejects_bad_params(bad, status):
    d = desc(8, 16)
    for k, v in bad.items():
        setattr(d, k, v)
    with pytest.raises(m.MuonError) as e:
        m.muon_state_bytes(m.muon_config_default(), [d], [0])
    assert e.value.status == status


@pytest.mark.parametrize("field,value", [("K", 0), ("ns_iters", 0), ("ns_precision", 3),
                                         ("rownorm_axis", 2), ("bp_blocks", -1),
                                         ("adam_b1", 1.0), ("eps_row", -1.0),
                                         ("lr", float("nan")), ("tall_single_pass", 2),
                                         ("reserved0", 1)])
def test_config_validation(field, value):
    c = m.muon_config_default(**{field: value})
    with pytest.raises(m.MuonError) as e:
        m.muon_state_bytes(c, [desc(4, 4)], [0])
    assert e.value.status == m.binding.MUON_E_ARG


def test_muonbp_split_must_be_even():
    c = m.muon_config_default(bp_blocks=8)
    with pytest.raises(m.MuonError) as e:
        m.muon_state_bytes(c, [desc(64, 36)], [0])
    assert e.value.status == m.binding.MUON_E_SHAPE
    assert m.muon_state_bytes(c, [desc(64, 48)], [0]) > 0


def test_workspace_matrix_over_4gib_is_rejected():
    """X (r x c, padded) is addressed with 32-bit buffer offsets: a matrix
    whose workspace copy reaches 4 GiB must fail planning, not run wrong."""
    with pytest.raises(m.MuonError) as e:
        m.muon_state_bytes(m.muon_config_default(), [desc(40000, 60000)], [0])
    assert e.value.status == m.binding.MUON_E_SHAPE
    assert "4 GiB" in m.muon_last_error()
    # just under the limit in bf16, over it in fp32
    assert m.muon_state_bytes(m.muon_config_default(), [desc(32768, 65000)], [0]) > 0
    with pytest.raises(m.MuonError):
        m.muon_state_bytes(m.muon_config_default(ns_precision=m.MUON_NS_F32),
                           [desc(32768, 65000)], [0])


def test_unknown_kind():
    with pytest.raises(m.MuonError) as e:
        m.muon_state_bytes(m.muon_config_default(), [desc(4, 4)], [9])
    assert e.value.status == m.binding.MUON_E_ARG


def _init(params, grads, kinds, state=FAKE, nbytes=None):
    c = m.muon_config_default()
    if nbytes is None:
        nbytes = m.muon_state_bytes(c, params, kinds)
    return m.muon_init(c, params, grads, kinds, state, nbytes, 0)


@pytest.mark.parametrize("case,status", [
    ("null_param", m.binding.MUON_E_ARG),
    ("misaligned_grad", m.binding.MUON_E_ALIGN),
    ("grad_shape", m.binding.MUON_E_SHAPE),
    ("small_state", m.binding.MUON_E_WORKSPACE),
    ("null_state", m.binding.MUON_E_WORKSPACE),
    ("misaligned_state", m.binding.MUON_E_ALIGN),
])
def test_init_validation_happens_before_any_device_call(case, status):
    p, g = desc(32, 64), desc(32, 64, m.MUON_BF16)
    kw = {}
    if case == "null_param":
        p.ptr = None
    elif case == "misaligned_grad":
        g.ptr = FAKE + 2
    elif case == "grad_shape":
        g = desc(32, 65, m.MUON_BF16)
    elif case == "small_state":
        kw["nbytes"] = 1024
    elif case == "null_state":
        kw["state"] = 0
    elif case == "misaligned_state":
        kw["state"] = FAKE + 64
    with pytest.raises(m.MuonError) as e:
        _init([p], [g], [0], **kw)
    assert e.value.status == status
    assert m.muon_last_error()


def test_step_on_null_context():
    st = m.lib().muon_step(None, None, None, 0)
    assert st == m.binding.MUON_E_ARG
