"""S3R_DEBUG: the host-side checks of the device data the kernels trust.

With S3R_DEBUG set, every call first checks on the host the sequence lengths,
page-table entries and draft token ids it would read. A bad value makes it fail
with INVALID_ARGUMENT before anything is launched, which the tests see as
outputs left exactly as they were. Valid inputs give bit-identical results with
and without the checks.

The corrupted inputs never reach a kernel unchecked: the tests set S3R_DEBUG
before any call on them. Even so, every buffer an unchecked launch could index
with a bad value (pools, bounds, page-table rows, logits) has a spare page or
row on each side inside its own allocation, so no such access leaves it.
"""
import math

import pytest
import torch

import self_sparse_speculative_paged_amd as s3r
from s3r_inputs import make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda"
CFG = dict(B=4, Hq=8, Hkv=2, D=128, L=None, P=16, budget=64, gamma=4, V=1000, kv_dtype="bf16",
           draft_sd=2.0, noise_sd=0.7, temperature=1.0, heavy_pages=0)
CTX = [150, 300, 37, 64]
BUDGET, GAMMA = 64, 4
SCALE = 1.0 / math.sqrt(128)


def _padded(t):
    """A contiguous view of t inside an allocation with one spare row (first
    index) before it and one after it."""
    big = torch.zeros((t.shape[0] + 2,) + tuple(t.shape[1:]), dtype=t.dtype, device=DEV)
    big[1:-1] = t.to(DEV)
    return big[1:-1]


class Setup:
    def __init__(self, seed=0):
        wl = make_workload(CFG, device="cpu", seed=seed, ctx=CTX, with_logits=True)
        self.wl = wl
        self.k, self.v = _padded(wl.k_pool), _padded(wl.v_pool)
        self.pt = _padded(wl.page_table)
        self.seq = [s.to(DEV) for s in wl.seq_lens]
        self.n_phys = wl.k_pool.shape[0]
        self.bounds = _padded(torch.zeros((self.n_phys, 2, 2, 128), dtype=torch.bfloat16))
        self.q = wl.q_verify.to(DEV)
        self.q0 = wl.draft_q(0).to(DEV)
        self.dl, self.tl = _padded(wl.draft_logits), _padded(wl.target_logits)
        self.tok = _padded(wl.draft_tokens)
        self.first = (self.seq[0] - 1).contiguous()
        g = torch.Generator().manual_seed(seed + 1)
        self.k_new = torch.randn((4, GAMMA + 1, 2, 128), generator=g).to(torch.bfloat16).to(DEV)
        self.v_new = torch.randn((4, GAMMA + 1, 2, 128), generator=g).to(torch.bfloat16).to(DEV)

    def kv(self, step):
        return s3r.PagedKVCache(self.k, self.v, self.pt, self.seq[step], CFG["Hq"])


def _sentinel(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    if dtype.is_floating_point:
        t.fill_(7.0)
    else:
        t.fill_(-7)
    return t


# Every call that reads the paged KV, each writing into fresh outputs; returns
# the outputs, in order. Bounds are computed first, as a caller would.
def _kv_calls(st):
    B, Hq, Hkv, k = 4, CFG["Hq"], 2, BUDGET // 16
    sel = torch.zeros((B, Hkv, k), dtype=torch.int32, device=DEV)  # page 0 only, a valid list
    sel[:, :, 1:] = -1
    return [
        ("s3r_page_bounds_update",
         lambda kv, o: s3r.page_bounds_update(kv, o[0]), 0, [st.bounds]),
        ("s3r_page_select",
         lambda kv, o: s3r.page_select(kv, st.bounds, st.q0, BUDGET, SCALE, o[0], o[1]),
         0, [_sentinel((B, Hkv, k), torch.int32), _sentinel((B,), torch.int32)]),
        ("s3r_sparse_draft_attn",
         lambda kv, o: s3r.sparse_draft_attn(kv, st.q0, sel, SCALE, out=o[0]),
         0, [_sentinel((B, Hq, 128), torch.float32)]),
        ("s3r_sparse_draft_step",
         lambda kv, o: s3r.sparse_draft_step(kv, st.bounds, st.q0, BUDGET, SCALE, st.first,
                                             o[1], o[2], o[0]),
         0, [_sentinel((B, Hq, 128), torch.float32), _sentinel((B, Hkv, k), torch.int32),
             _sentinel((B,), torch.int32)]),
        ("s3r_sparse_draft_round",
         lambda kv, o: s3r.sparse_draft_round(kv, st.bounds, st.q0, BUDGET, GAMMA, SCALE, st.first,
                                              o[1], o[2], o[0]),
         0, [_sentinel((B, Hq, 128), torch.float32), _sentinel((B, Hkv, k), torch.int32),
             _sentinel((B,), torch.int32)]),
        ("s3r_dense_verify_attn",
         lambda kv, o: s3r.dense_verify_attn(kv, st.q, SCALE, out=o[0]),
         GAMMA, [_sentinel((B, GAMMA + 1, Hq, 128), torch.float32)]),
    ]


def _run_everything(debug, monkeypatch):
    """Every entry point once, on fresh buffers; returns all outputs and the
    pools and bounds after a KV commit."""
    if debug:
        monkeypatch.setenv("S3R_DEBUG", "1")
    else:
        monkeypatch.delenv("S3R_DEBUG", raising=False)
    st = Setup()
    outs = []
    for _, call, step, o in _kv_calls(st):
        call(st.kv(step), o)
        outs += [t.clone() for t in o]
    kv = st.kv(0)
    kv.set_seq_lens((st.seq[0] + 2).contiguous())
    s3r.kv_commit(kv, st.k_new, st.v_new, st.first, st.bounds)
    tokens, nacc = s3r.spec_sample(st.dl, st.tl, st.tok, 1.0, 5, 0)
    torch.cuda.synchronize()
    return outs + [st.k.clone(), st.v.clone(), st.bounds.clone(), tokens, nacc]


def test_valid_inputs_give_identical_results_with_checks(monkeypatch):
    print("S3R_DEBUG: valid inputs, B=4 bf16 D=128, every entry point", flush=True)
    plain = _run_everything(False, monkeypatch)
    checked = _run_everything(True, monkeypatch)
    for i, (a, b) in enumerate(zip(plain, checked)):
        assert torch.equal(a, b), i


def _expect_rejected(fn, where):
    with pytest.raises(s3r.S3RError) as e:
        fn()
    assert e.value.status == 1 and where in str(e.value), str(e.value)


def _assert_untouched(outs, before):
    torch.cuda.synchronize()
    for a, b in zip(outs, before):
        assert torch.equal(a, b)


@pytest.mark.parametrize("entry", ["past_pool", "negative"])
def test_bad_page_entry_rejected_before_launch(entry, monkeypatch, capfd):
    monkeypatch.setenv("S3R_DEBUG", "1")
    print(f"S3R_DEBUG: page_table[1][2] {entry}", flush=True)
    st = Setup()
    s3r.page_bounds_update(st.kv(0), st.bounds)  # on the valid table
    torch.cuda.synchronize()
    bad = st.n_phys if entry == "past_pool" else -1
    st.pt[1, 2] = bad                             # page 2 of sequence 1 (300 tokens)
    for where, call, step, outs in _kv_calls(st):
        before = [t.clone() for t in outs]
        _expect_rejected(lambda: call(st.kv(step), outs), where)
        _assert_untouched(outs, before)
    err = capfd.readouterr().err
    assert f"page_table[1][2] = {bad}" in err, err
    # The KV commit reads page 2 too (it lies below the committed tail), where a
    # negative entry is an unallocated page, not an error.
    k0, v0 = st.k.clone(), st.v.clone()
    if entry == "past_pool":
        _expect_rejected(lambda: s3r.kv_commit(st.kv(0), st.k_new, st.v_new, st.first, st.bounds),
                         "s3r_kv_commit")
        _assert_untouched([st.k, st.v], [k0, v0])
    else:
        s3r.kv_commit(st.kv(0), st.k_new, st.v_new, st.first, st.bounds)
        torch.cuda.synchronize()
        assert not torch.equal(st.k, k0)


def test_commit_into_a_page_past_the_pool_rejected(monkeypatch):
    monkeypatch.setenv("S3R_DEBUG", "1")
    print("S3R_DEBUG: kv_commit into page_table[3][4] past the pool", flush=True)
    st = Setup()
    # sequence 3 has 64 tokens: its commit of 5 rows from position 63 writes page 4
    st.pt[3, 4] = st.n_phys
    k0, v0, b0 = st.k.clone(), st.v.clone(), st.bounds.clone()
    _expect_rejected(lambda: s3r.kv_commit(st.kv(0), st.k_new, st.v_new, st.first, st.bounds),
                     "s3r_kv_commit")
    _assert_untouched([st.k, st.v, st.bounds], [k0, v0, b0])


def test_sequence_longer_than_its_table_row_rejected(monkeypatch, capfd):
    monkeypatch.setenv("S3R_DEBUG", "1")
    print("S3R_DEBUG: seq_lens[0] one past its page-table row", flush=True)
    st = Setup()
    maxp = st.pt.shape[1]
    lens = st.seq[GAMMA].clone()
    lens[0] = maxp * 16 + 1        # row 0: one page more than the row holds
    kv = s3r.PagedKVCache(st.k, st.v, st.pt, lens, CFG["Hq"])
    b0 = st.bounds.clone()
    _expect_rejected(lambda: s3r.page_bounds_update(kv, st.bounds), "s3r_page_bounds_update")
    out = _sentinel((4, GAMMA + 1, CFG["Hq"], 128), torch.float32)
    o0 = out.clone()
    _expect_rejected(lambda: s3r.dense_verify_attn(kv, st.q, SCALE, out=out), "s3r_dense_verify_attn")
    _assert_untouched([st.bounds, out], [b0, o0])
    assert f"seq_lens[0] = {maxp * 16 + 1}" in capfd.readouterr().err


@pytest.mark.parametrize("where,value", [((1, 1), "vocab"), ((2, 0), -1)])
def test_draft_token_outside_vocab_rejected(where, value, monkeypatch):
    monkeypatch.setenv("S3R_DEBUG", "1")
    print(f"S3R_DEBUG: draft token {value} at {where}", flush=True)
    st = Setup()
    st.tok[where] = CFG["V"] if value == "vocab" else value
    out = _sentinel((4, GAMMA + 1), torch.int32)
    nacc = _sentinel((4,), torch.int32)
    _expect_rejected(lambda: s3r.spec_sample(st.dl, st.tl, st.tok, 1.0, 5, 0, out, nacc),
                     "s3r_spec_sample")
    _assert_untouched([out, nacc], [_sentinel((4, GAMMA + 1), torch.int32),
                                    _sentinel((4,), torch.int32)])


def test_checks_refuse_graph_capture(monkeypatch):
    monkeypatch.setenv("S3R_DEBUG", "1")
    print("S3R_DEBUG: verify under graph capture", flush=True)
    st = Setup()
    kv = st.kv(GAMMA)
    out = torch.empty((4, GAMMA + 1, CFG["Hq"], 128), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(s3r.attn_workspace(kv, GAMMA + 1, st.pt.shape[1]), 1), dtype=torch.uint8,
                     device=DEV)
    x = torch.ones(16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(g, stream=s):
        x.mul_(2.0)
        try:
            s3r.dense_verify_attn(kv, st.q, SCALE, out=out, workspace=ws)
        except s3r.S3RError as e:
            status = e.status
    assert status == 2
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(x, torch.full((16,), 2.0, device=DEV))  # captured, not run, then one replay
