"""kvs_attn_decode_noalloc against kvs_attn_decode, through the C ABI: the
same kernels with the partials in the library's device scratch instead of a
caller workspace, so equal n_splits give bit-identical outputs.  Each case
makes two calls in a row, the second on a smaller input (fewer sequences,
shorter contexts), so stale partials of the first call would show; both are
also held to the oracle's tolerance."""
import ctypes

import pytest
import torch

import attention_cross_layer_amd as K
import datagen
from tests._gpu_harness import Dense, Factorized, assert_close, note

pytestmark = pytest.mark.gpu

W = datagen.WORKLOADS


def _pair(rig, layer, B, lens, n_splits):
    """(noalloc output, workspace output) for the first B sequences at lens."""
    q = rig.q(layer)[:B].contiguous().cuda()
    seq_len = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    K.kvs_attn_decode_noalloc(rig.plan, rig.cache, layer, q, seq_len, max(lens), out,
                              n_splits=n_splits)
    ref = K.kvs_attn_decode(rig.plan, rig.cache, layer, q, seq_len, max(lens), n_splits=n_splits)
    torch.cuda.synchronize()
    return q, out, ref


@pytest.mark.parametrize("n_splits", [0, 3, 8])
def test_dense_noalloc_equals_workspace_call(n_splits):
    wl = W["cla2_64k"].with_(n_layers=2)
    lens = [1000, 640, 999, 513]
    note(f"[noalloc] dense splits={n_splits} lens={lens}")
    d = Dense(wl, 4, 1000, lens)
    for B, ls in ((4, lens), (2, [300, 129])):
        q, got, ref = _pair(d, 1, B, ls, n_splits)
        assert torch.equal(got, ref), f"B={B}: noalloc differs from the workspace call"
        from oracle import attention as A
        kk = {l: x[:B] for l, x in d.k.items()}
        vv = {l: x[:B] for l, x in d.v.items()}
        exp = A.layer_decode(d.src.tolist(), d.w.tolist(), 1, kk, vv, q.cpu(), ls)
        assert_close(got, exp, "bf16", f"dense noalloc B={B}")


@pytest.mark.parametrize("n_splits", [0, 5])
def test_factorized_noalloc_equals_workspace_call(n_splits):
    wl = W["factorized_64k"].with_(n_layers=2)
    lens = [900, 777]
    note(f"[noalloc] factorized splits={n_splits} lens={lens}")
    f = Factorized(wl, 2, 900, lens)
    from oracle import attention as A
    for B, ls in ((2, lens), (1, [200])):
        q, got, ref = _pair(f, 0, B, ls, n_splits)
        assert torch.equal(got, ref), f"B={B}: noalloc differs from the workspace call"
        k, v = f.kv(0, 0, B)
        assert_close(got, A.attend_decode(q.cpu(), k, v, ls), "bf16", f"factorized noalloc B={B}")


def test_noalloc_rejects_partials_beyond_the_scratch():
    """A split count whose partials exceed the 16 MiB scratch is refused on
    the host, before any launch."""
    wl = W["cla2_64k"]
    src, w = datagen.share_map(wl)
    plan = K.kvs_share_plan(K.make_config(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                                          "bf16", 256, 4096), src, w)
    need = K.kvs_decode_workspace_size(plan, 256, 64)
    assert need > 16 << 20
    cache = K.kvs_cache()          # never dereferenced: the call fails first
    st = K.lib().kvs_attn_decode_noalloc(plan.handle, ctypes.byref(cache), 1, 0x7e0000000000,
                                         0x7e0000000000, 256, 4096, 64, 0x7e0000000000, 0, None)
    assert st == K.KVS_ERR_RANGE
    msg = K.lib().kvs_last_error().decode()
    assert "scratch" in msg and str(need) in msg
