"""CPU tests of the C ABI: the library loads and exports every declared
symbol, the host planner agrees bit-exactly with the oracle's map semantics,
layout sizes follow the documented formulas, and the compute entry points
reject bad arguments before touching the GPU."""
import ctypes
import math
import os
import random
import re

import pytest
import torch

import attention_cross_layer_amd as K
import datagen
from oracle import plan as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "kvshare.h")).read()
    return sorted(set(re.findall(r"KVS_API\s+[\w\s\*]+?\b(kvs_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = K.lib()
    declared = _declared_symbols()
    assert len(declared) == len(K.EXPORTS) and set(declared) == set(K.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def _cfg(L, Hq=8, Hkv=2, hd=64, dtype="bf16", B=2, ctx=300, kind=K.KVS_DENSE, R=0, Rm=0):
    return K.make_config(L, Hq, Hkv, hd, dtype, B, ctx, kind=kind, basis_rank=R, resid_rank_max=Rm)


STATUS_OF = {P.OK: K.KVS_OK, P.ERR_MAP: K.KVS_ERR_MAP, P.ERR_NOT_SOURCE: K.KVS_ERR_NOT_SOURCE,
             P.ERR_UNSUPPORTED: K.KVS_ERR_UNSUPPORTED}


def _plan_status(src, w, cfg):
    try:
        plan = K.kvs_share_plan(cfg, src, w)
        return K.KVS_OK, plan
    except K.KvsError as e:
        return e.status, None


def _assert_plan_matches_oracle(plan, src, w):
    sl = P.slots(src, w)
    s = K.kvs_plan_summary(plan)
    assert s.n_slots == len(sl)
    assert s.last_owner_layer == P.last_owner_layer(src, w)
    for l in range(len(src)):
        li = K.kvs_plan_layer(plan, l)
        assert li.owns_kv == int(P.owns(src, w, l))
        want = P.layer_sources(src, w, l)
        assert li.n_src == len(want)
        for j, (s_l, s_slot, s_w) in enumerate(want):
            assert li.src_layer[j] == s_l and li.src_slot[j] == s_slot
            # weights stored bit-exactly as the fp32 input
            assert li.weight[j] == float(torch.tensor(s_w, dtype=torch.float32))
        for j in range(len(want), 2):
            assert li.src_layer[j] == -1 and li.src_slot[j] == -1
        assert li.masks_current == int(P.excludes_current(src, w, l))


@pytest.mark.parametrize("name", ["tiny_cla2", "tinyllama_cla2", "depthgraft", "cla2_64k"])
def test_plan_of_each_workload_matches_oracle(name):
    wl = datagen.WORKLOADS[name]
    src, w = datagen.share_map(wl)
    cfg = _cfg(wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.dtype, wl.batch, wl.ctx)
    st, plan = _plan_status(src, w, cfg)
    assert st == K.KVS_OK
    _assert_plan_matches_oracle(plan, src.tolist(), w.tolist())


def test_random_maps_classified_like_oracle():
    rng = random.Random(1234)
    for trial in range(400):
        L = rng.randint(1, 9)
        src, w = [], []
        for l in range(L):
            kind = rng.random()
            if kind < 0.35:
                src.append([l, -1]); w.append([1.0, 0.0])
            elif kind < 0.7:
                src.append([rng.randint(-1, L), -1]); w.append([rng.choice([1.0, 0.5]), 0.0])
            else:
                src.append([rng.randint(-1, L), rng.randint(-2, L)])
                w.append([rng.choice([0.25, 1.0, float("inf")]), rng.choice([0.75, float("nan"), 1.0])])
        want = P.check(src, w)
        st, plan = _plan_status(torch.tensor(src, dtype=torch.int32),
                                torch.tensor(w, dtype=torch.float32), _cfg(L))
        assert st == STATUS_OF[want], (src, w, want, st)
        if plan is not None:
            _assert_plan_matches_oracle(plan, src, w)


def test_config_rejections():
    src = torch.tensor([[0, -1]], dtype=torch.int32)
    with pytest.raises(K.KvsError) as e:
        K.kvs_share_plan(_cfg(1, hd=96), src)
    assert e.value.status == K.KVS_ERR_UNSUPPORTED
    with pytest.raises(K.KvsError) as e:
        K.kvs_share_plan(_cfg(1, Hq=6, Hkv=4), src)
    assert e.value.status == K.KVS_ERR_ARG
    with pytest.raises(K.KvsError) as e:
        K.kvs_share_plan(_cfg(1, B=0), src)
    assert e.value.status == K.KVS_ERR_ARG
    # factorized pools are addressed with 32-bit offsets per slot / layer:
    # 64 sequences x 64K tokens x 8 KV heads is the largest accepted size
    big = K.make_config(2, 32, 8, 128, "bf16", 64, 65536, kind=K.KVS_FACTORIZED, basis_rank=32,
                        resid_rank_max=16)
    K.kvs_share_plan(big, torch.tensor([[0, -1], [0, -1]], dtype=torch.int32))
    bigger = K.make_config(2, 32, 8, 128, "bf16", 65, 65536, kind=K.KVS_FACTORIZED, basis_rank=32,
                           resid_rank_max=16)
    with pytest.raises(K.KvsError) as e:
        K.kvs_share_plan(bigger, torch.tensor([[0, -1], [0, -1]], dtype=torch.int32))
    assert e.value.status == K.KVS_ERR_UNSUPPORTED


def test_cache_layout_sizes():
    wl = datagen.WORKLOADS["tinyllama_cla2"]
    src, w = datagen.share_map(wl)
    plan = K.kvs_share_plan(_cfg(22, 32, 4, 64, "bf16", 64, 2048), src, w)
    sz = K.kvs_cache_layout(plan)
    assert sz.page_tokens == 64 and sz.pages_per_seq == 32 and sz.n_phys_pages == 64 * 32
    assert sz.n_slots == 11
    # 11 owner layers x B64 x ctx2048 x Hkv4 x hd64 x 2 bytes: half of an unshared cache
    assert sz.k_pool_bytes == 11 * 64 * 2048 * 4 * 64 * 2 == sz.v_pool_bytes
    assert sz.page_table_bytes == 64 * 32 * 4
    plan = K.kvs_share_plan(_cfg(2, ctx=100, B=3), [[0, -1], [0, -1]])
    assert K.kvs_cache_layout(plan).pages_per_seq == 2


def test_decode_split_choice_and_workspace():
    wl = datagen.WORKLOADS["cla2_64k"]
    src, w = datagen.share_map(wl)
    plan = K.kvs_share_plan(_cfg(32, 32, 8, 128, "bf16", 4, 65536), src, w)
    s = K.kvs_decode_splits(plan, 4, 65536)
    # one 4-wave workgroup per (partition, KV head, sequence): about 192 of them
    assert 1 <= s <= 64 and 4 * 8 * s >= 192
    assert K.kvs_decode_splits(plan, 4, 64) == 1
    # partials [B][Hq][S][hd], maxima and sums [B][Hq][S]
    assert K.kvs_decode_workspace_size(plan, 4, s) == 4 * 32 * s * (128 + 2) * 4
    with pytest.raises(K.KvsError):
        K.kvs_decode_workspace_size(plan, 4, 65)
    with pytest.raises(K.KvsError):
        K.kvs_decode_splits(plan, 5, 100)


def test_decode_split_rule_by_kernel_and_call_size():
    # VALU kernel (hd 128): three workgroups per four CUs (192) for a call
    # streaming 1 GiB (4 x 8 x 6), and for a smaller one whose sequences and
    # KV heads reach 192 to 224 workgroups (8 x 8 x 3 at 256 MiB, 1 x 8 x 24)
    src, w = datagen.share_map(datagen.WORKLOADS["cla2_64k"])
    plan = K.kvs_share_plan(_cfg(32, 32, 8, 128, "bf16", 32, 65536), src, w)
    assert K.kvs_decode_splits(plan, 4, 65536) == 6
    assert K.kvs_decode_splits(plan, 2, 65536) == 12
    assert K.kvs_decode_splits(plan, 8, 65536) == 3
    assert K.kvs_decode_splits(plan, 8, 8192) == 3
    assert K.kvs_decode_splits(plan, 1, 65536) == 24
    assert K.kvs_decode_splits(plan, 7, 8192) == 4     # 7 x 8 x 4 = 224
    assert K.kvs_decode_splits(plan, 5, 8192) == 5     # 5 x 8 x 5 = 200
    # otherwise small calls take four per CU, at most 32 partitions
    assert K.kvs_decode_splits(plan, 16, 4096) == 8    # 16 x 8 x 2 = 256 > 224
    assert K.kvs_decode_splits(plan, 10, 8192) == 13   # 10 x 8 x 3 = 240 > 224
    # at least 4 pages per partition
    assert K.kvs_decode_splits(plan, 1, 4096) == 16
    assert K.kvs_decode_splits(plan, 8, 512) == 2
    assert K.kvs_decode_splits(plan, 32, 1024) == 4
    # a group of 8 at hd 128 runs one wave per SIMD: one workgroup per CU
    # for a small call too (4 x 8 x 8 = 256)
    plan8 = K.kvs_share_plan(_cfg(32, 64, 8, 128, "bf16", 8, 65536), src, w)
    assert K.kvs_decode_splits(plan8, 4, 16384) == 8
    # hd-64 bf16 MFMA kernel: one workgroup per CU
    src, w = datagen.share_map(datagen.WORKLOADS["tinyllama_cla2"])
    plan = K.kvs_share_plan(_cfg(22, 32, 4, 64, "bf16", 64, 2048), src, w)
    assert K.kvs_decode_splits(plan, 64, 2048) == 1
    assert K.kvs_decode_splits(plan, 16, 8192) == 4


class _FakeCache:
    """kvs_cache struct holding aligned non-null fake device addresses; only
    used on calls that must fail validation before any device access."""

    def __init__(self, misalign=False):
        self.struct = K.kvs_cache()
        base = 0x7f0000000000
        for i, n in enumerate(("k_pool", "v_pool", "page_table", "ck_pool", "cv_pool", "dk_pool",
                               "dv_pool", "sk_pool", "sv_pool", "rank_pool", "basis_k",
                               "basis_v", "ubasis_k", "ubasis_v")):
            setattr(self.struct, n, base + i * 0x100000 + (4 if misalign and n == "k_pool" else 0))


def _raw_append(plan, cache, layer, k, v, n, sp, B):
    return K.lib().kvs_append(plan.handle, ctypes.byref(cache.struct), layer, k, v, n, sp, B, None)


def _raw_decode(plan, cache, layer, q, sl, B, mx, S, out, odt, ws, wsb):
    return K.lib().kvs_attn_decode(plan.handle, ctypes.byref(cache.struct), layer, q, sl, B, mx, S,
                                   out, odt, ws, wsb, None)


def test_compute_calls_validate_before_launch():
    src, w = datagen.share_map(datagen.WORKLOADS["tiny_cla2"])
    plan = K.kvs_share_plan(_cfg(4, 4, 2, 64, "f32", 2, 128), src, w)
    c = _FakeCache()
    a = 0x7e0000000000
    assert _raw_append(plan, c, 1, a, a, 1, a, 1) == K.KVS_ERR_NOT_SOURCE
    assert _raw_append(plan, c, 7, a, a, 1, a, 1) == K.KVS_ERR_ARG
    assert _raw_append(plan, c, 0, a, a, 1, a, 3) == K.KVS_ERR_RANGE
    assert _raw_append(plan, c, 0, a, a, 129, a, 1) == K.KVS_ERR_RANGE
    assert _raw_append(plan, c, 0, a + 8, a, 1, a, 1) == K.KVS_ERR_ALIGN
    assert _raw_append(plan, _FakeCache(misalign=True), 0, a, a, 1, a, 1) == K.KVS_ERR_ALIGN
    assert _raw_append(plan, c, 0, None, a, 1, a, 1) == K.KVS_ERR_ARG
    ws = K.kvs_decode_workspace_size(plan, 1, 2)
    assert _raw_decode(plan, c, 1, a, a, 1, 128, 2, a, 0, a, ws - 4) == K.KVS_ERR_RANGE
    assert _raw_decode(plan, c, 1, a, a, 1, 128, 2, a, 5, a, ws) == K.KVS_ERR_ARG
    assert _raw_decode(plan, c, 1, a + 4, a, 1, 128, 2, a, 0, a, ws) == K.KVS_ERR_ALIGN
    assert _raw_decode(plan, c, 1, a, a, 1, 128, 5000, a, 0, a, 1 << 40) == K.KVS_ERR_RANGE
    assert _raw_decode(plan, c, 1, a, None, 1, 128, 2, a, 0, a, ws) == K.KVS_ERR_ARG
    assert "null" in K.lib().kvs_last_error().decode()
    # the last error names the failed check of the call that set it
    assert _raw_decode(plan, c, 1, a, a, 1, 128, 2, a, 0, a, ws - 4) == K.KVS_ERR_RANGE
    msg = K.lib().kvs_last_error().decode()
    assert "workspace too small" in msg and str(ws) in msg
