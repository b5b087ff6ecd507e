"""GPU parity of the top-k / top-p truncated step against the oracle.

With truncation P, Q and the proposal law are the truncated laws of their rows
("Introspective Diffusion Language Models | Summary", section 4.1 samples with
top-k 50 and top-p 0.95; section 3.3: verify with the law of the proposal
mechanism actually used).  Proposals x are drawn by the oracle from the
truncated Q rows with their own uniforms, as a truncated proposer would.
"""

import numpy as np
import pytest

from isd_inputs import CONFIGS, gen_step
from oracle import isd_oracle as O
from tests.isd_testlib import compare, log, oracle_step, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def isd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import speculative_verification_amd as isd_mod
    isd_mod.lib()
    return isd_mod


def _truncated_proposals(d, dtype, T, top_k, top_p, seed):
    """x drawn from the truncated law of each q row (oracle, fp64)."""
    rng = np.random.default_rng(seed)
    q = O.decode_logits(d["q"], dtype)
    u = rng.random(d["x"].shape)
    tok, _, _, _ = O.propose_sample(q, u, T, top_k=top_k, top_p=top_p)
    return tok.astype(np.int32)


def _case(isd, cfg, seed, top_k, top_p, label, *, x_from_q=True, mutate=None, **variant):
    import torch
    d = gen_step(2, seed, cfg=cfg)
    if mutate is not None:
        mutate(d)
    if variant.get("q_onehot"):
        d["x"] = O.argmax_first(O.decode_logits(d["q"], cfg["dtype"])).astype(np.int32)
    elif x_from_q:
        d["x"] = _truncated_proposals(d, cfg["dtype"], cfg["T"], top_k, top_p, seed)
    dd = to_device(d, cfg["dtype"])
    q = None if variant.get("q_onehot") else dd["q"]
    o = isd.step(dd["p"], q, dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"],
                 temperature=cfg["T"], top_k=top_k, top_p=top_p, **variant)
    torch.cuda.synchronize()
    g = to_host(o)
    ref = _oracle(d, cfg, top_k, top_p, **variant)
    st = compare(g, ref, label=label)
    return g, ref, st


def _oracle(d, cfg, top_k, top_p, chunk=8, **variant):
    """oracle_step with truncation (verify and propose both truncated)."""
    return oracle_step(d, cfg["dtype"], "sample", cfg["T"], chunk=chunk,
                       relax=variant.get("relax", 0.0), q_onehot=variant.get("q_onehot", False),
                       sampler=variant.get("sampler", "cdf"), top_k=top_k, top_p=top_p)


@pytest.mark.parametrize("top_k,top_p", [(50, 0.95), (8, 1.0), (64, 0.5), (1, 1.0), (20, 0.8)])
def test_truncated_step_midsize(isd, top_k, top_p):
    cfg = dict(CONFIGS[2], C=8, L=8, V=10000)
    acc = 0
    for step in range(3):
        g, ref, st = _case(isd, cfg, 900 + step, top_k, top_p, f"k={top_k} p={top_p} step {step}")
        acc += int(ref["accept_len"].sum())
        assert np.all(g["next_tokens"] >= 0)
    log(f"top-k {top_k} top-p {top_p}: accepted positions {acc}")


@pytest.mark.parametrize("top_k,top_p", [(50, 0.95), (64, 1.0), (3, 0.5)])
def test_truncated_one_segment_per_row(isd, top_k, top_p):
    """C=64, L=8 makes 1536 rows, so every row is one workgroup (the item
    finishes its row from registers); 3 tiles per row."""
    cfg = dict(CONFIGS[2], C=64, L=8, V=5000)
    _case(isd, cfg, 960, top_k, top_p, f"one segment k={top_k} p={top_p}")


@pytest.mark.parametrize("V", [1, 7, 64, 65])
def test_truncated_tiny_vocabularies(isd, V):
    """Rows shorter than k (k is cut to V) and a single entry: every entry
    survives top-k, and with one entry every law is a point mass."""
    cfg = dict(CONFIGS[2], C=3, L=4, V=V)
    _case(isd, cfg, 980, 50, 0.95, f"tiny V={V}")


@pytest.mark.parametrize("V,dtype", [(5003, "bf16"), (4099, "f32"), (40, "bf16"), (2048, "bf16")])
def test_truncated_ragged_and_small(isd, V, dtype):
    """Unaligned rows (scalar loads), fp32, a row shorter than k, one exact tile."""
    cfg = dict(CONFIGS[2], C=6, L=4, V=V, dtype=dtype)
    for step in range(2):
        _case(isd, cfg, 950 + step, 50, 0.9, f"V={V} {dtype} step {step}")


def _coarse(d):
    """Logits rounded to a grid of 0.5 (frequent ties), with one constant row."""
    from isd_inputs import f32_to_bf16_bits
    for key in ("p", "q", "qn"):
        v = O.decode_logits(d[key], "bf16")
        v = np.round(v * 2) / 2
        v[0, 1] = 1.0
        d[key] = f32_to_bf16_bits(v.astype(np.float32))


def test_truncated_ties_rank_lower_index_first(isd):
    """Logits rounded to a coarse grid tie often: ranks go to the lower index;
    constant rows keep their first k entries."""
    cfg = dict(CONFIGS[2], C=6, L=4, V=6000)
    for step in range(2):
        _case(isd, cfg, 970 + step, 16, 0.9, f"ties step {step}", mutate=_coarse)


@pytest.mark.parametrize("segments,V", [(1, 200000), (1, 200003), (2, 200000)])
def test_truncated_long_rows(isd, segments, V):
    """Rows of 98 tiles.  In one segment the selection records its group
    maxima in two LDS chunks (80 + 18 tiles) and carries the best group keys
    across them; two segments take one chunk each.  V = 200003 takes the
    scalar-load path.  Random and tie-heavy logits."""
    cfg = dict(CONFIGS[2], C=2, L=3, V=V)
    isd.set_trunc_tuning(segments)
    try:
        for step in range(2):
            _case(isd, cfg, 1010 + step, 50, 0.95, f"V={V} St={segments} step {step}")
        _case(isd, cfg, 1020, 64, 1.0, f"V={V} St={segments} ties", mutate=_coarse)
    finally:
        isd.set_trunc_tuning(0)


@pytest.mark.parametrize("variant", [dict(q_onehot=True), dict(relax=0.5),
                                     dict(sampler="gumbel"),
                                     dict(sampler="gumbel", q_onehot=True, relax=0.25)])
def test_truncated_variants(isd, variant):
    cfg = dict(CONFIGS[2], C=8, L=8, V=10000)
    for step in range(2):
        _case(isd, cfg, 990 + step, 50, 0.95, f"{variant} step {step}", **variant)


def test_truncated_full_size(isd):
    """The serving shape C=64, L=8, V=151936 at the pages' top-k 50, top-p 0.95."""
    cfg = CONFIGS[2]
    seqs = np.arange(cfg["C"])
    d = gen_step(2, 11, seqs=seqs, workers=8)
    import torch
    d["x"] = _truncated_proposals(d, cfg["dtype"], cfg["T"], 50, 0.95, 11)
    dd = to_device(d, cfg["dtype"])
    o = isd.step(dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"],
                 temperature=cfg["T"], top_k=50, top_p=0.95)
    torch.cuda.synchronize()
    ref = _oracle(d, cfg, 50, 0.95)
    st = compare(to_host(o), ref, label="full truncated")
    log(f"full-size top-k 50 top-p 0.95: {st}, mean accept_len {ref['accept_len'].mean():.3f}")


def test_truncated_entry_points_masks_and_workspace(isd):
    """verify_step, propose, alpha (with its batch mean) and the masked step on
    the truncated path agree with the oracle and with each other, and the
    workspace is zero after every call."""
    import torch
    cfg = dict(CONFIGS[2], C=8, L=8, V=10000)
    d = gen_step(2, 1001, cfg=cfg)
    d["x"] = _truncated_proposals(d, cfg["dtype"], cfg["T"], 32, 0.9, 1001)
    dd = to_device(d, cfg["dtype"])
    ref = _oracle(d, cfg, 32, 0.9)
    kw = dict(temperature=cfg["T"], top_k=32, top_p=0.9)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")

    def clean(what):
        torch.cuda.synchronize()
        nz = torch.nonzero(ws).flatten()[:8].tolist()
        assert not nz, f"workspace not zero after {what}: bytes {nz}"

    v = to_host(isd.verify_step(dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], ws=ws, **kw))
    clean("verify_step")
    compare(v, ref, propose=False, label="verify_step")
    pr = to_host(isd.propose(dd["qn"], dd["up"], ws=ws, **kw))
    clean("propose")
    compare(pr, ref, verify=False, label="propose")
    a = to_host(isd.alpha(dd["p"], dd["q"], dd["x"], ws=ws, **kw))
    clean("alpha")
    np.testing.assert_allclose(a["alpha"], ref["alpha"], rtol=1e-5)
    np.testing.assert_allclose(a["alpha_mean"][0], ref["alpha"].mean(), rtol=1e-5)

    full = to_host(isd.step(dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"],
                            ws=ws, **kw))
    clean("step")
    vmask = np.array([1, 0, 1, 1, 0, 0, 1, 0], dtype=np.int32)
    pmask = np.array([0, 1, 1, 0, 1, 0, 1, 1], dtype=np.int32)
    h = to_host(isd.step_masked(dd["p"], dd["q"], dd["x"], dd["ua"], dd["ur"], dd["qn"], dd["up"],
                                torch.from_numpy(vmask).cuda(), torch.from_numpy(pmask).cuda(),
                                ws=ws, **kw))
    clean("step_masked")
    on, off = vmask == 1, vmask == 0
    for key in ("accept_len", "n_emitted", "out_tokens", "p_x", "q_x", "alpha"):
        np.testing.assert_array_equal(h[key][on], full[key][on], err_msg=key)
    assert np.all(h["accept_len"][off] == -1) and np.all(h["out_tokens"][off] == -1)
    np.testing.assert_array_equal(h["next_tokens"][pmask == 1], full["next_tokens"][pmask == 1])
    assert np.all(h["next_tokens"][pmask == 0] == -1)
    isd.check_device_error(ws)
