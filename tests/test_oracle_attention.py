"""Pins of the oracle's attention against things other than itself.

* torch scaled_dot_product_attention on the CPU with an explicit causal mask
  over the gathered tokens (a library routine);
* a second decode path that streams one token at a time (running max/sum);
* special cases with closed forms: all-equal logits give the mean of V; one
  visible token gives that token's V; a budget covering every page makes the
  sparse draft equal the dense decode.
"""
import numpy as np
import pytest
import torch

import oracle
from s3r_inputs import make_workload
from tests.oracle_io import f64, i32


def _small(seed=0, kv="f32", D=64, ctx=(40, 23), G=2, Hkv=2, gamma=3):
    return make_workload(dict(B=len(ctx), Hq=G * Hkv, Hkv=Hkv, D=D, L=None, P=16, budget=32,
                              gamma=gamma, V=16, kv_dtype=kv, draft_sd=1.0, noise_sd=0.5,
                              temperature=1.0, heavy_pages=0), seed=seed, ctx=list(ctx))


def _np(wl, j):
    return (f64(wl.k_pool), f64(wl.v_pool), i32(wl.page_table), i32(wl.seq_lens[j]))


def _sdpa_reference(q, K, V, pt, L, nq, Hkv, scale):
    """Gather tokens by the page table, then torch SDPA with a causal mask."""
    B, _, Hq, D = q.shape
    G = Hq // Hkv
    P = K.shape[2]
    out = np.zeros((B, nq, Hq, D))
    for b in range(B):
        pos = np.arange(L[b])
        phys = pt[b, pos // P]
        for g in range(Hq):
            h = g // G
            Kt = torch.from_numpy(K[phys, h, pos % P, :])
            Vt = torch.from_numpy(V[phys, h, :, pos % P])
            qq = torch.from_numpy(q[b, :, g, :])
            qpos = L[b] - nq + np.arange(nq)
            mask = torch.from_numpy(pos[None, :] <= qpos[:, None])
            o = torch.nn.functional.scaled_dot_product_attention(
                qq[None, None], Kt[None, None], Vt[None, None], attn_mask=mask[None, None],
                scale=scale)
            out[b, :, g] = o[0, 0].numpy()
    return out


@pytest.mark.parametrize("kv", ["f32", "bf16"])
def test_dense_verify_matches_torch_sdpa(kv):
    wl = _small(seed=1, kv=kv)
    gamma = wl.cfg["gamma"]
    K, V, pt, L = _np(wl, gamma)
    q = f64(wl.q_verify)
    scale = 1 / np.sqrt(wl.cfg["D"])
    got = oracle.dense_verify_attn(q, K, V, pt, L, scale)
    ref = _sdpa_reference(q, K, V, pt, L, gamma + 1, wl.cfg["Hkv"], scale)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-12)


def test_dense_verify_equals_sequential_streaming_decodes():
    wl = _small(seed=2, ctx=(37, 64, 17), gamma=4)
    gamma = wl.cfg["gamma"]
    K, V, pt, L = _np(wl, gamma)
    q = f64(wl.q_verify)
    scale = 0.125
    got = oracle.dense_verify_attn(q, K, V, pt, L, scale)
    G = wl.cfg["Hq"] // wl.cfg["Hkv"]
    for b in range(len(L)):
        for i in range(gamma + 1):
            for g in range(wl.cfg["Hq"]):
                ref = oracle.decode_streaming(q[b, i, g], K, V, pt, b, g // G, L[b] - gamma + i, scale)
                np.testing.assert_allclose(got[b, i, g], ref, rtol=1e-11, atol=1e-13)


def test_sparse_with_all_pages_equals_dense_decode():
    wl = _small(seed=3, ctx=(50, 33))
    for j in range(wl.cfg["gamma"] + 1):
        K, V, pt, L = _np(wl, j)
        q = f64(wl.draft_q(j))
        n = [oracle.n_pages(x, 16) for x in L]
        k = 8
        sel = np.full((len(L), wl.cfg["Hkv"], k), -1, dtype=np.int32)
        for b in range(len(L)):
            sel[b, :, :n[b]] = np.arange(n[b])
        got = oracle.sparse_draft_attn(q, K, V, pt, L, sel, 0.125)
        ref = oracle.dense_verify_attn(q[:, None], K, V, pt, L, 0.125)[:, 0]
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_sparse_matches_sdpa_on_gathered_pages():
    wl = _small(seed=4, ctx=(100, 70))
    K, V, pt, L = _np(wl, 0)
    q = f64(wl.draft_q(0))
    sel = np.array([[[0, 3, 6, -1], [1, 2, 4, 6]], [[4, -1, -1, -1], [0, 1, 2, 3]]], dtype=np.int32)
    got = oracle.sparse_draft_attn(q, K, V, pt, L, sel, 0.2)
    G = 2
    for b in range(2):
        for g in range(4):
            h = g // G
            pages = [j for j in sel[b, h] if j >= 0]
            pos = np.array([t for j in sorted(pages) for t in range(16 * j, min(16 * j + 16, L[b]))])
            phys = pt[b, pos // 16]
            Kt = torch.from_numpy(K[phys, h, pos % 16])
            Vt = torch.from_numpy(V[phys, h, :, pos % 16])
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[b, g])[None, None, None], Kt[None, None], Vt[None, None], scale=0.2)
            np.testing.assert_allclose(got[b, g], o.reshape(-1).numpy(), rtol=1e-10, atol=1e-12)


def test_closed_forms():
    # equal logits (q = 0): output is the plain mean of the visible V rows
    rng = np.random.default_rng(0)
    K = rng.standard_normal((4, 1, 16, 8))
    V = rng.standard_normal((4, 1, 8, 16))
    pt = np.array([[2, 0, 3]])
    L = np.array([37])
    q = np.zeros((1, 2, 1, 8))
    out = oracle.dense_verify_attn(q, K, V, pt, L, 1.0)
    vis = [V[pt[0, t // 16], 0, :, t % 16] for t in range(37)]
    np.testing.assert_allclose(out[0, 1, 0], np.mean(vis, axis=0), rtol=1e-13)
    np.testing.assert_allclose(out[0, 0, 0], np.mean(vis[:36], axis=0), rtol=1e-13)
    # a single visible token: output is exactly its V row
    out1 = oracle.dense_verify_attn(rng.standard_normal((1, 1, 1, 8)), K, V, pt, np.array([1]), 0.3)
    np.testing.assert_allclose(out1[0, 0, 0], V[2, 0, :, 0], rtol=0, atol=1e-15)
    # no visible token: zeros by definition
    out0 = oracle.dense_verify_attn(rng.standard_normal((1, 3, 1, 8)), K, V, pt, np.array([1]), 0.3)
    assert np.all(out0[0, :2] == 0) and np.all(out0[0, 2, 0] == V[2, 0, :, 0])


def test_value_layout_is_transposed_per_page():
    # v_pool[phys][h][d][slot]: the oracle must read d along axis 2
    V = np.arange(2 * 1 * 4 * 16, dtype=np.float64).reshape(2, 1, 4, 16)
    pt = np.array([[1, 0]])
    assert np.array_equal(oracle.value_row(V, pt, 0, 0, 3), V[1, 0, :, 3])
    assert np.array_equal(oracle.value_row(V, pt, 0, 0, 17), V[0, 0, :, 1])
