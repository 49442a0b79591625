"""C-ABI checks that need no GPU: the library loads, exports every declared symbol,
validates arguments before touching the device, and packs host pages in the
documented layout."""
import ctypes
import os
import re

import numpy as np
import pytest

from lookahead_sparse_kv_draft_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oasiskv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(oasis_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_set():
    assert declared_functions() == sorted(L.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(L.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def _shape(**kw):
    base = dict(batch=2, kv_heads=2, group=4, head_dim=128, max_blocks=64, budget_blocks=16,
                n_draft=4, fetch_cap=4, dtype=L.OASIS_BF16)
    base.update(kw)
    return base


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), L.OASIS_EINVAL),
    (dict(budget_blocks=1), L.OASIS_EINVAL),
    (dict(budget_blocks=2000), L.OASIS_EINVAL),
    (dict(fetch_cap=-1), L.OASIS_EINVAL),
    (dict(head_dim=96), L.OASIS_EUNSUPPORTED),
    (dict(block_size=32), L.OASIS_EUNSUPPORTED),
    (dict(dtype=7), L.OASIS_EUNSUPPORTED),
    (dict(group=16, n_draft=4), L.OASIS_EUNSUPPORTED),   # 80 query rows
    (dict(max_blocks=70000), L.OASIS_EUNSUPPORTED),
])
def test_create_rejects_bad_shapes(kw, code):
    with pytest.raises(L.OasisError) as e:
        L.oasis_create(**_shape(**kw))
    assert e.value.code == code
    assert L.oasis_last_error()


def test_launch_options_resolve_and_validate():
    """The launch options a handle resolves (host only, no device call): the
    in-launch split merge where it was asked for and 2 to 8 splits run beside
    the scoring, the combine otherwise (by default, 1 split, too many splits,
    fp32); the default split count beside the scoring (about 512 attention
    wavefronts, fewer where the scoring reads most of the launch's bytes);
    out-of-range values are EINVAL."""
    def resolved(opts, **kw):
        h = L.oasis_create_with_options(**_shape(**kw), options=opts)
        try:
            return L.oasis_get_launch_options(h)
        finally:
            L.oasis_destroy(h)

    assert resolved(dict(attn_splits=4))["attn_merge"] == 1                  # default: the combine
    assert resolved(dict(attn_splits=8))["attn_merge"] == 1
    assert resolved(dict(attn_splits=8, attn_merge=1))["attn_merge"] == 1
    assert resolved(dict(attn_splits=4, attn_merge=2)) == dict(resolved(dict(attn_splits=4)), attn_merge=2)
    assert resolved(dict(attn_splits=4, attn_merge=3))["attn_merge"] == 3
    assert resolved(dict(attn_splits=8, attn_merge=2))["attn_merge"] == 2
    assert resolved(dict(attn_splits=1, attn_merge=2))["attn_merge"] == 1    # nothing to merge
    nine = resolved(dict(attn_splits=9, attn_merge=2), budget_blocks=72, max_blocks=128)
    assert nine["attn_splits"] == 9 and nine["attn_merge"] == 1             # more than 8 splits
    assert resolved(dict(attn_splits=4, attn_merge=2), dtype=L.OASIS_F32)["attn_merge"] == 1
    # partials of 2 GiB or more (batch 65536, 8 KV heads, 20 rows, 8 splits): the combine
    big = resolved(dict(attn_splits=8, attn_merge=2), batch=65536, kv_heads=8, budget_blocks=128, max_blocks=128)
    assert big["attn_splits"] == 8 and big["attn_merge"] == 1
    # 64 units, k = 128: 4 splits with 2048 blocks of metadata per unit (even
    # share), 2 with 8192 (share 0.2: about 205 attention wavefronts)
    assert resolved(None, batch=8, kv_heads=8, budget_blocks=128, max_blocks=2048)["attn_splits"] == 4
    assert resolved(None, batch=8, kv_heads=8, budget_blocks=128, max_blocks=8192)["attn_splits"] == 2
    for bad in (dict(attn_merge=4), dict(attn_merge=-1), dict(attn_pf=3), dict(step_launches=1)):
        with pytest.raises(L.OasisError) as e:
            resolved(bad)
        assert e.value.code == L.OASIS_EINVAL, bad
    # the workspace holds the partials and then one arrival counter per unit
    h1 = L.oasis_create_with_options(**_shape(), options=dict(attn_splits=4))
    h2 = L.oasis_create_with_options(**_shape(), options=dict(attn_splits=4, attn_merge=2))
    try:
        assert L.oasis_workspace_bytes(h1) == L.oasis_workspace_bytes(h2)
        assert L.oasis_workspace_bytes(h1) % 256 == 0
    finally:
        L.oasis_destroy(h1)
        L.oasis_destroy(h2)


@pytest.mark.parametrize("kw,splits,tpw,pf_step", [
    # llama8b_32k: batch 8, 32q/8kv, 2048 blocks; the attention moves half of the first launch's bytes
    (dict(batch=8, kv_heads=8, group=4, max_blocks=2048, n_draft=4), 4, 2, 2),
    # qwen32b_32k: batch 16, 64q/8kv (40 attention rows), 2048 blocks
    (dict(batch=16, kv_heads=8, group=8, max_blocks=2048, n_draft=4), 2, 2, 2),
    # llama8b_128k: batch 4, 8192 blocks; the attention moves a fifth of the bytes
    (dict(batch=4, kv_heads=8, group=4, max_blocks=8192, n_draft=4), 4, 4, 2),
    # qwen8b_reason: batch 64, 528 blocks; one split of 64-block runs
    (dict(batch=64, kv_heads=8, group=4, max_blocks=528, n_draft=5), 1, 2, 2),
])
def test_default_launch_shapes_of_the_workloads(kw, splits, tpw, pf_step):
    """The launch shape the library picks by default for each benchmark
    workload (attention splits and scoring runs of the fused first launch;
    the ring stays 2 pages there), as measured best on MI355X."""
    h = L.oasis_create_with_options(head_dim=128, budget_blocks=128, fetch_cap=32, dtype=L.OASIS_BF16, **kw)
    try:
        o = L.oasis_get_launch_options(h)
    finally:
        L.oasis_destroy(h)
    assert (o["attn_splits"], o["score_tpw"], o["attn_pf"], o["attn_waves"], o["attn_merge"]) == \
        (splits, tpw, pf_step, 2, 1), o


def test_sizes_and_null_checks():
    h = L.oasis_create(**_shape())
    try:
        assert L.oasis_version() == 2
        assert L.oasis_page_bytes(h) == 2 * 16 * 128 * 2
        assert L.oasis_meta_bytes(h) == 4 * 64 * 2 * 128 * 2
        assert L.oasis_pool_bytes(h) == 4 * 16 * 8192
        assert L.oasis_host_tier_bytes(h) == 4 * 64 * 8192
        assert L.oasis_workspace_bytes(h) > 0
        lib = L.load()
        # null pointers are rejected before any device work
        assert lib.oasis_lookahead_score(h, None, None, None, None, None) == L.OASIS_EINVAL
        assert lib.oasis_verify_score(h, 18, 32, 16, 16, None) == L.OASIS_EINVAL  # misaligned q
        assert lib.oasis_verify_score(h, None, None, None, None, None) == L.OASIS_EINVAL
        assert lib.oasis_admit(h, *([None] * 8)) == L.OASIS_EINVAL
        assert lib.oasis_admit(h, 16, 16, 16, 16, 16, 16, None, None) == L.OASIS_EINVAL  # pool without the map
        assert "null" in L.oasis_last_error()
        assert lib.oasis_topk_select(h, None, None, None, None) == L.OASIS_EINVAL
        assert lib.oasis_resident_diff_cap_evict(h, *([None] * 10)) == L.OASIS_EINVAL
        assert lib.oasis_sparse_paged_decode_attn(h, None, None, None, None, None, None, None, None) == L.OASIS_EINVAL
        assert lib.oasis_block_meta_update(h, None, None, None, None, None, None, None, None) == L.OASIS_EINVAL
        assert lib.oasis_block_meta_build(h, None, None, 0, None, None, None, None, None) == L.OASIS_EINVAL
        # token ranges outside [0, max_blocks * 16] (64 blocks here)
        for tb, te in ((-1, 16), (32, 16), (0, 64 * 16 + 1)):
            assert lib.oasis_block_meta_build_rows(h, 256, tb, te, 256, 256, None) == L.OASIS_EINVAL, (tb, te)
        assert lib.oasis_block_meta_build_rows(h, None, 0, 16, 256, 256, None) == L.OASIS_EINVAL
        assert lib.oasis_block_meta_export(h, None, 256, None) == L.OASIS_EINVAL
        assert lib.oasis_block_meta_import(h, 256, None, None) == L.OASIS_EINVAL
        assert lib.oasis_block_meta_export(h, 256, 256, None) == L.OASIS_EINVAL  # not in place
        assert lib.oasis_block_meta_import(h, 256, 264, None) == L.OASIS_EINVAL  # misaligned
        assert lib.oasis_lookahead_score(None, 16, 16, 16, 16, None) == L.OASIS_EINVAL
        assert lib.oasis_select_and_diff(h, *([None] * 11)) == L.OASIS_EINVAL
        assert lib.oasis_decode_step(h, *([None] * 17)) == L.OASIS_EINVAL
        assert lib.oasis_sparse_paged_decode_attn_list(h, *([None] * 8)) == L.OASIS_EINVAL
        assert lib.oasis_fetch_gather(h, None, None, None, None, None) == L.OASIS_EINVAL
        assert lib.oasis_attend_and_score(h, *([None] * 13)) == L.OASIS_EINVAL
        assert lib.oasis_attn_combine(h, None, None, None) == L.OASIS_EINVAL
        assert lib.oasis_select_diff_combine(h, *([None] * 13)) == L.OASIS_EINVAL
        assert lib.oasis_select_and_diff_lru(h, *([None] * 6), 0, *([None] * 6)) == L.OASIS_EINVAL
        assert lib.oasis_select_diff_combine_lru(h, *([None] * 6), 0, *([None] * 8)) == L.OASIS_EINVAL
        # LRU needs the stamps
        assert lib.oasis_select_and_diff_lru(h, *([256] * 5), None, 3, *([256] * 3), None, None, None) \
            == L.OASIS_EINVAL
        # attention inputs: the maps are needed when no attended list is given
        assert lib.oasis_attend_and_score(h, *([256] * 5), None, None, None, None, 256, 256, 256, None) \
            == L.OASIS_EINVAL
        assert lib.oasis_attn_combine(h, 272, 256, None) == L.OASIS_EINVAL  # misaligned workspace
        # the attended list and its length come together or not at all
        assert lib.oasis_select_and_diff(h, *([256] * 8), 256, None, None) == L.OASIS_EINVAL
        assert "attend" in L.oasis_last_error()
        assert lib.oasis_resident_diff_cap_evict(h, *([256] * 7), None, 256, None) == L.OASIS_EINVAL
        # a host tier that is not pinned, device-mapped memory is refused before any launch
        plain = np.zeros(4096, dtype=np.uint8)
        assert lib.oasis_fetch_gather(h, plain.ctypes.data, 256, 256, 256, None) == L.OASIS_EINVAL
        # one missing pointer among valid-looking ones, and a misaligned workspace
        good = [256] * 17
        for i in range(11):  # q .. workspace, then n_fetch
            args = list(good)
            args[i] = None
            assert lib.oasis_decode_step(h, *args) == L.OASIS_EINVAL, i
        args = list(good)
        args[10] = 272  # workspace 16- but not 256-byte aligned
        assert lib.oasis_decode_step(h, *args) == L.OASIS_EINVAL
        assert "workspace" in L.oasis_last_error()
        args = list(good)
        args[15] = None  # n_attend without attend's partner
        assert lib.oasis_decode_step(h, *args) == L.OASIS_EINVAL
        # misaligned device pointers
        assert lib.oasis_lookahead_score(h, 18, 32, 16, 16, None) == L.OASIS_EINVAL
        assert "aligned" in L.oasis_last_error()
        # aliasing context buffers
        assert lib.oasis_block_meta_update(h, 16, 16, 64, 64, 16, 16, 16, None) == L.OASIS_EINVAL
    finally:
        L.oasis_destroy(h)


def test_fetch_issue_validates_every_entry_first():
    h = L.oasis_create(**_shape())
    try:
        fetch = np.full((4, 4, 2), -1, dtype=np.int32)
        nf = np.array([1, 0, 0, 0], dtype=np.int32)
        fetch[0, 0] = (64, 0)  # block out of range
        with pytest.raises(L.OasisError) as e:
            L.oasis_fetch_issue(h, 16, 16, fetch, nf, 0)
        assert e.value.code == L.OASIS_EINVAL
        fetch[0, 0] = (3, 16)  # slot out of range
        with pytest.raises(L.OasisError):
            L.oasis_fetch_issue(h, 16, 16, fetch, nf, 0)
        nf[0] = 5  # more entries than the cap
        with pytest.raises(L.OasisError):
            L.oasis_fetch_issue(h, 16, 16, fetch, nf, 0)
        nf[:] = 0
        L.oasis_fetch_issue(h, 16, 16, fetch, nf, 0)  # nothing to copy: no device work
    finally:
        L.oasis_destroy(h)


@pytest.mark.parametrize("dtype", [L.OASIS_BF16, L.OASIS_F32])
def test_pack_pages_layout(dtype):
    """Page = K rows token-major [16][d], then V channel-major [d][16]."""
    d, Nmax = 64, 6
    h = L.oasis_create(**_shape(head_dim=d, max_blocks=Nmax, dtype=dtype))
    try:
        et = np.uint16 if dtype == L.OASIS_BF16 else np.float32
        rng = np.random.default_rng(0)
        K = rng.integers(0, 60000, size=(3 * 16, d)).astype(et)
        V = rng.integers(0, 60000, size=(3 * 16, d)).astype(et)
        pages = np.zeros((4, Nmax, 2 * 16 * d), dtype=et)
        blocks = np.array([4, 0, 2], dtype=np.int32)
        L.oasis_pack_pages(h, K, V, blocks, 3, 2, pages)
        for i, b in enumerate(blocks):
            kp = pages[2, b, : 16 * d].reshape(16, d)
            vt = pages[2, b, 16 * d:].reshape(d, 16)
            assert np.array_equal(kp, K[16 * i: 16 * i + 16])
            assert np.array_equal(vt, V[16 * i: 16 * i + 16].T)
        assert not pages[2, 1].any() and not pages[2, 3].any() and not pages[0].any()
        # K only: V half untouched
        K2 = K + 1
        L.oasis_pack_pages(h, K2[:16], None, np.array([4], dtype=np.int32), 1, 2, pages)
        assert np.array_equal(pages[2, 4, : 16 * d].reshape(16, d), K2[:16])
        assert np.array_equal(pages[2, 4, 16 * d:].reshape(d, 16), V[:16].T)
        with pytest.raises(L.OasisError):
            L.oasis_pack_pages(h, K, V, np.array([6], dtype=np.int32), 1, 0, pages)
        # host append: token 35 (block 2, row 3) of request 1 -> units 2, 3
        kn = rng.integers(0, 60000, size=(2, 2, d)).astype(et)
        vn = rng.integers(0, 60000, size=(2, 2, d)).astype(et)
        L.oasis_host_tier_append(h, kn, vn, np.array([0, 35], dtype=np.int32), pages)
        assert np.array_equal(pages[3, 2, : 16 * d].reshape(16, d)[3], kn[1, 1])
        assert np.array_equal(pages[3, 2, 16 * d:].reshape(d, 16)[:, 3], vn[1, 1])
        assert np.array_equal(pages[1, 0, : 16 * d].reshape(16, d)[0], kn[0, 1])
    finally:
        L.oasis_destroy(h)


def test_noalloc_attention_rejects_a_workspace_beyond_its_scratch():
    # 512 units x 64 rows x 4 splits of k = 256 need 64 MiB of partials: more than
    # the 16 MiB scratch; rejected on the host, before any device work
    h = L.oasis_create(**_shape(batch=64, kv_heads=8, group=16, n_draft=3, max_blocks=4096, budget_blocks=256))
    try:
        assert L.oasis_workspace_bytes(h) > 16 << 20
        lib = L.load()
        assert lib.oasis_sparse_paged_decode_attn_noalloc(h, 16, 16, 16, 16, 16, 16, None) == L.OASIS_EINVAL
        assert "scratch" in L.oasis_last_error()
        assert lib.oasis_sparse_paged_decode_attn_noalloc(h, None, 16, 16, 16, 16, 16, None) == L.OASIS_EINVAL
    finally:
        L.oasis_destroy(h)


def test_decode_step_gather_rejects_its_own_pool():
    # the transfer's pool is the step's pool: the attention would read what the
    # move writes; rejected before anything is enqueued
    h = L.oasis_create(**_shape())
    try:
        lib = L.load()
        tr = L.oasis_transfer(host_tier=256, pool=512, fetch=768, n_fetch=1024)
        args = [h, 256, 512, 256] + [256] * 13
        assert lib.oasis_decode_step_gather(*args, ctypes.byref(tr), None) == L.OASIS_EINVAL
        assert "pool" in L.oasis_last_error()
    finally:
        L.oasis_destroy(h)


def test_decode_step_append_rejects_before_any_launch():
    """The step that carries the token append: missing pointers (the step's
    own and the token's), a misaligned workspace and a grown context that
    aliases the positions are EINVAL, on the host, before any launch."""
    lib = L.load()
    # q, pool, meta, ctx_in, ctx_out, sel, b2s, s2b, scores, out, workspace, fetch, n_fetch, evict, attend,
    # n_attend, k_new, v_new (fake device addresses: nothing is launched)
    args = list(range(256, 256 * 19, 256))
    h = L.oasis_create(**_shape())
    try:
        for i in (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 12, 16, 17):
            a = list(args)
            a[i] = None
            assert lib.oasis_decode_step_append(h, *a, None) == L.OASIS_EINVAL, i
        a = list(args)
        a[10] = 272  # workspace not 256-byte aligned
        assert lib.oasis_decode_step_append(h, *a, None) == L.OASIS_EINVAL
        a = list(args)
        a[4] = a[3]  # ctx_out aliases ctx_in
        assert lib.oasis_decode_step_append(h, *a, None) == L.OASIS_EINVAL
        assert "aliases" in L.oasis_last_error()
        a = list(args)
        a[14] = None  # attend without n_attend
        assert lib.oasis_decode_step_append(h, *a, None) == L.OASIS_EINVAL
    finally:
        L.oasis_destroy(h)


def test_decode_step_carry_rejects_before_any_launch():
    """The step that carries another state's selection: missing pointers, a job
    that is this step's own state, and a transfer reading the fetch list the
    job writes are EINVAL; shapes outside its kernels EUNSUPPORTED; all on the
    host, before any launch."""
    lib = L.load()
    # q, pool, meta, ctx_attn, ctx_score, attend, n_attend, scores, out, workspace
    args = list(range(256, 256 * 11, 256))
    job_fields = list(range(256 * 20, 256 * 30, 256))  # scores .. n_attend of another state

    def job(**kw):
        j = L.oasis_select_job(*job_fields)
        for k, v in kw.items():
            setattr(j, k, v)
        return ctypes.byref(j)

    h = L.oasis_create(**_shape())
    try:
        for i in (0, 5, 6, 7, 9):
            a = list(args)
            a[i] = None
            assert lib.oasis_decode_step_carry(h, *a, None, None, None) == L.OASIS_EINVAL, i
        a = list(args)
        a[9] = 272  # workspace not 256-byte aligned
        assert lib.oasis_decode_step_carry(h, *a, None, None, None) == L.OASIS_EINVAL
        assert lib.oasis_decode_step_carry(h, *args, job(scores=None), None, None) == L.OASIS_EINVAL
        assert lib.oasis_decode_step_carry(h, *args, job(scores=args[7]), None, None) == L.OASIS_EINVAL
        assert "own state" in L.oasis_last_error()
        assert lib.oasis_decode_step_carry(h, *args, job(attend=args[5]), None, None) == L.OASIS_EINVAL
        assert lib.oasis_decode_step_carry(h, *args, job(n_attend=args[6]), None, None) == L.OASIS_EINVAL
    finally:
        L.oasis_destroy(h)
    for kw in (dict(budget_blocks=256, fetch_cap=4), dict(head_dim=64), dict(dtype=L.OASIS_F32),
               dict(max_blocks=9000)):
        h = L.oasis_create(**_shape(**kw))
        try:
            assert lib.oasis_decode_step_carry(h, *args, job(), None, None) == L.OASIS_EUNSUPPORTED, kw
        finally:
            L.oasis_destroy(h)
