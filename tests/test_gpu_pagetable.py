"""Page-table entries outside [0, n_phys_pages) and prefill rows before
position 0, through the C ABI.

Every attention call gives the keys of a page whose table entry is out of
range no weight (the entry is never dereferenced): the decode skips the page,
the prefill kernels give its keys no score.  The expected values come from
the oracle over the same keys with that page's 64 keys taken out; the page
sits wholly below the prefill chunk, so every query of the chunk sees it and
its absolute positions shift by 64 in the shortened sequence.
"""
import numpy as np
import pytest
import torch

import attention_cross_layer_amd as K
import datagen
from oracle import attention as A
from tests._gpu_harness import Dense, Factorized, assert_close, note

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS
PAGE = 64


def _drop_page(x, b, page, T):
    """[B, T, ...] float64 copy with the 64 keys of `page` removed from
    sequence b (later keys move down; the freed tail is zero)."""
    y = np.array(A.f64(x), copy=True)
    keep = np.concatenate([y[b, :page * PAGE], y[b, (page + 1) * PAGE:]], axis=0)
    y[b] = 0.0
    y[b, :keep.shape[0]] = keep
    return y


@pytest.mark.parametrize("bad", ["neg", "past_end"])
def test_dense_out_of_range_page_is_skipped(bad):
    wl = W["cla2_64k"].with_(n_layers=2)
    B, ctx, lens, n = 2, 448, [448, 390], 100
    drop_b, drop_page = 0, 2                       # keys 128..191 of sequence 0
    note(f"[pagetable] dense {bad}: B={B} lens={lens} drop seq {drop_b} page {drop_page}")
    d = Dense(wl, B, ctx, lens)
    pt = d.cache.page_table.clone()
    pt[drop_b, drop_page] = -1 if bad == "neg" else d.cache.sizes.n_phys_pages
    d.cache.page_table.copy_(pt)
    torch.cuda.synchronize()
    lens2 = list(lens)
    lens2[drop_b] -= PAGE
    kk = {l: _drop_page(d.k[l], drop_b, drop_page, ctx) for l in d.owners}
    vv = {l: _drop_page(d.v[l], drop_b, drop_page, ctx) for l in d.owners}
    for l in range(wl.n_layers):
        ref = A.layer_decode(d.src.tolist(), d.w.tolist(), l, kk, vv, d.q(l), lens2)
        for s in (0, 1, 3):
            got = d.decode(l, n_splits=s)
            torch.cuda.synchronize()
            assert_close(got, ref, "bf16", f"decode layer {l} splits {s}")
        for causal in (True, False):
            q = datagen.prefill_q(wl, l, n, batch=B)
            got = K.kvs_attn_prefill_chunk(d.plan, d.cache, l, q.cuda(), d.seq_len, causal=causal)
            torch.cuda.synchronize()
            ref_p = A.layer_prefill(d.src.tolist(), d.w.tolist(), l, kk, vv, q, lens2, causal=causal)
            assert_close(got, ref_p, "bf16", f"prefill layer {l} causal {causal}")


def test_factorized_out_of_range_page_is_skipped():
    wl = W["factorized_64k"].with_(n_layers=2)
    B, ctx, lens, n = 2, 448, [448, 300], 90
    drop_b, drop_page = 1, 1
    note(f"[pagetable] factorized: B={B} lens={lens} drop seq {drop_b} page {drop_page}")
    f = Factorized(wl, B, ctx, lens)
    pt = f.cache.page_table.clone()
    pt[drop_b, drop_page] = -7
    f.cache.page_table.copy_(pt)
    torch.cuda.synchronize()
    lens2 = list(lens)
    lens2[drop_b] -= PAGE
    for l in range(wl.n_layers):
        k, v = f.kv(l)
        k2, v2 = _drop_page(k, drop_b, drop_page, ctx), _drop_page(v, drop_b, drop_page, ctx)
        ref = A.attend_decode(f.q(l), k2, v2, lens2)
        for s in (0, 1, 2):
            got = f.decode(l, n_splits=s)
            torch.cuda.synchronize()
            assert_close(got, ref, "bf16", f"factorized decode layer {l} splits {s}")
        q = datagen.prefill_q(wl, l, n, batch=B)
        for causal in (True, False):
            ref_p = A.attend_prefill(q, k2, v2, lens2, causal=causal)
            assert_close(f.prefill(l, q, causal=causal), ref_p, "bf16",
                         f"factorized prefill layer {l} causal {causal}")


def test_prefill_rows_before_position_zero_see_no_key():
    """seq_len[b] < n: causal rows at positions below 0 see no key (zeros);
    non-causal rows see every key of the sequence."""
    wl = W["tinyllama_cla2"].with_(n_layers=2)
    B, ctx, lens, n = 3, 200, [200, 40, 0], 70
    note(f"[pagetable] rows before 0: lens={lens} n={n}")
    d = Dense(wl, B, ctx, lens)
    f = Factorized(W["factorized_64k"].with_(n_layers=2), B, ctx, lens)
    for causal in (True, False):
        q = datagen.prefill_q(wl, 1, n, batch=B)
        got = K.kvs_attn_prefill_chunk(d.plan, d.cache, 1, q.cuda(), d.seq_len, causal=causal)
        torch.cuda.synchronize()
        ref = A.layer_prefill(d.src.tolist(), d.w.tolist(), 1, d.k, d.v, q, lens, causal=causal)
        assert_close(got, ref, "bf16", f"dense causal {causal}")
        if causal:
            # rows 0..n-lens[b]-1 of the short sequences are exactly zero
            assert torch.count_nonzero(got[1, :n - lens[1]]) == 0
        assert torch.count_nonzero(got[2]) == 0
        qf = datagen.prefill_q(f.wl, 1, n, batch=B)
        assert_close(f.prefill(1, qf, causal=causal), f.oracle_prefill(1, qf, causal=causal), "bf16",
                     f"factorized causal {causal}")
