"""CPU tests of the C ABI: the library loads, exports what the header declares,
the host scheduler matches the oracle bit for bit, and bad arguments are
rejected with the documented codes before any GPU work."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import variable_length_sequence_amd as vl
import workloads
from oracle import schedule as osched

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "varlen.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"VL_API\s+[\w\s\*]+?\b(\w+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = _declared()
    assert set(names) == set(vl.EXPORTS)
    for n in ("varlen_attn_fwd", "varlen_attn_bwd", "attn_lse_merge", "sp_seq2head", "sp_head2seq"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = vl.lib()
    for n in _declared():
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", vl.LIB_PATH], capture_output=True, text=True)
    exported = {ln.split()[-1] for ln in out.stdout.splitlines() if " T " in ln}
    assert exported == set(_declared())
    assert vl.version() == 1


def _cu(lengths):
    return workloads.cu_seqlens(lengths)


def _check_against_oracle(cq, ck, causal, d):
    for p in (0, 1):
        r = vl.varlen_schedule_export(cq, ck, causal, p, d)
        fn = osched.fwd_items if p == 0 else osched.bwd_items
        ref = fn(cq, ck, causal, r["bq"], r["bk"])
        assert np.array_equal(r["items"], ref.reshape(-1, 4)), (p, causal)
        assert r["useful_pairs"] == osched.visible_pairs(cq, ck, causal)
        assert r["issued_pairs"] == osched.issued_pairs(ref, r["bq"], r["bk"])


@pytest.mark.parametrize("name", ["tiny_256", "longtail_16k", "ulysses_384k", "mixed_128k"])
def test_schedule_matches_oracle_on_workloads(name):
    w = workloads.ALL[name]()
    cu = w.cu
    _check_against_oracle(cu, cu, True, w.d)


def test_schedule_matches_oracle_ring_chunks():
    c = 32768
    _check_against_oracle(np.array([0, c], np.int32), np.array([0, c], np.int32), False, 128)
    _check_against_oracle(np.array([0, c], np.int32), np.array([0, 8 * c], np.int32), True, 128)


def test_schedule_matches_oracle_random(rng):
    for _ in range(60):
        n = int(rng.integers(1, 9))
        lq = rng.integers(0, 700, size=n)
        lk = lq.copy() if rng.random() < 0.5 else rng.integers(0, 700, size=n)
        for causal in (True, False):
            _check_against_oracle(_cu(lq), _cu(lk), causal, 128 if rng.random() < 0.5 else 64)


def _check_dkdv_split(cq, ck, causal, hq, hkv, n_cu):
    """The dK/dV list with its q-head split: every q head of every kv tile
    exactly once, only tiles over the per-CU share cut, into the fewest
    power-of-two slices that fit (at most min(4, group)), longest first."""
    ent = vl.varlen_schedule_export_dkdv(cq, ck, causal, hq, hkv, n_cu)
    items = osched.bwd_items(cq, ck, causal, 32, 128).reshape(-1, 4)
    grp = hq // hkv
    max_split = 1
    while max_split < grp and grp % (2 * max_split) == 0 and 2 * max_split <= 4:
        max_split *= 2
    per_cu = grp * hkv * int(items[:, 3].sum()) / n_cu
    by_tile = {}
    for doc, tile, first, count, sl, ns in ent.tolist():
        by_tile.setdefault((doc, tile, first, count), []).append((sl, ns))
    assert sorted(by_tile) == sorted(map(tuple, items.tolist()))
    for (doc, tile, first, count), sl in by_tile.items():
        ns = sl[0][1]
        assert all(n == ns for _, n in sl) and sorted(s for s, _ in sl) == list(range(ns))
        assert ns <= max_split and grp % ns == 0
        want = 1
        while want < max_split and count * grp / want > per_cu:
            want *= 2
        assert ns == want, (doc, tile, count, ns, want)
    work = ent[:, 3].astype(np.int64) * grp // ent[:, 5]
    assert np.all(work[:-1] >= work[1:])
    return int(ent[:, 5].max()) if len(ent) else 1


def test_dkdv_split_schedule():
    for w in (workloads.longtail_16k(), workloads.mixed_128k(), workloads.tiny()):
        cu = w.cu
        top = _check_dkdv_split(cu, cu, True, w.hq, w.hkv, 256)
        # the backward workspace holds as many fp32 partials as the largest cut
        delta = _align256(w.total * w.hq * 4)
        part = _align256(top * 2 * w.total * w.hkv * w.d * 4) if top > 1 else 0
        assert vl.bwd_workspace_bytes_cu(cu, cu, w.hq, w.hkv, w.d) == delta + part, w.name
    # the long-tail batch cuts only its longest key tiles
    cu = workloads.longtail_16k().cu
    ent = vl.varlen_schedule_export_dkdv(cu, cu, True, 32, 4, 256)
    cut = {(d, t) for d, t, *_, ns in ent.tolist() if ns > 1}
    assert 0 < len(cut) < len({(d, t) for d, t, *_ in ent.tolist()}) // 2
    rng = np.random.default_rng(5)
    for _ in range(40):
        n = int(rng.integers(1, 12))
        lq = rng.integers(0, 3000, size=n)
        hkv = int(rng.choice([1, 2, 4]))
        hq = hkv * int(rng.choice([1, 2, 3, 4, 8]))
        _check_dkdv_split(_cu(lq), _cu(lq), bool(rng.integers(0, 2)), hq, hkv,
                          int(rng.choice([8, 64, 256])))
    with pytest.raises(vl.VarlenError):
        vl.varlen_schedule_export_dkdv(_cu([5]), _cu([5]), True, 6, 4, 256)


def test_tiny_schedule_values():
    r = vl.varlen_schedule_export(_cu([17, 64, 128, 47]), _cu([17, 64, 128, 47]), True, 0, 64)
    assert r["useful_pairs"] == 11617
    assert r["bq"] == 128 and r["bk"] == 64


# ------------------------------------------------------------------ error codes
FAKE = 1 << 20  # a 256-aligned non-null address; never dereferenced on these paths


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu_q=np.array([0, 4], np.int32), cu_k=np.array([0, 4], np.int32),
             n_docs=1, tq=4, tk=4, hq=4, hkv=2, d=128, scale=0.0, causal=1, od=0, out=FAKE, lse=FAKE)
    a.update(kw)
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    ip = lambda x: None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    rc = vl.lib().varlen_attn_fwd(p(a["q"]), p(a["k"]), p(a["v"]), ip(a["cu_q"]), ip(a["cu_k"]),
                                  a["n_docs"], a["tq"], a["tk"], a["hq"], a["hkv"], a["d"],
                                  a["scale"], a["causal"], a["od"], p(a["out"]), p(a["lse"]), None)
    return rc, vl.lib().varlen_last_error().decode()


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1),
    (dict(out=None), -1),
    (dict(od=7), -1),
    (dict(hkv=3), -2),
    (dict(hq=0), -2),
    (dict(d=96), -4),
    (dict(cu_q=np.array([1, 4], np.int32)), -3),
    (dict(cu_q=np.array([0, 5], np.int32)), -3),
    (dict(cu_k=np.array([0, 2, 1], np.int32), n_docs=2, tk=1,
          cu_q=np.array([0, 2, 4], np.int32)), -3),
    (dict(q=FAKE + 2), -1),
])
def test_fwd_rejects_bad_arguments(kw, code):
    rc, msg = _fwd(**kw)
    assert rc == code and msg


def _align256(x):
    return (x + 255) // 256 * 256


def test_bwd_workspace_sizes():
    L = vl.lib()
    # one short document: its only key tile outlasts the per-CU share of the
    # pass, so the group of two q heads is split in two, which is also the bound
    cu = np.array([0, 8], np.int32)
    ip = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    two = _align256(8 * 4 * 4) + _align256(2 * 2 * 8 * 2 * 64 * 4)
    assert L.varlen_attn_bwd_workspace_size_cu(ip, ip, 1, 8, 8, 4, 2, 64, 1) == two
    assert L.varlen_attn_bwd_workspace_size(8, 8, 4, 2, 64) == two
    # 120 equal short documents spread over the device: no split, D only
    cu120 = np.arange(0, 121 * 200, 200, dtype=np.int32)
    p120 = cu120.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert L.varlen_attn_bwd_workspace_size_cu(p120, p120, 120, 24000, 24000, 32, 4, 128, 1) == _align256(24000 * 32 * 4)
    # any batch: D plus 0, 2 or 4 fp32 dK/dV partials, never above the bound
    for w in (workloads.longtail_16k(), workloads.mixed_128k(), workloads.ulysses_384k()):
        cu = np.asarray(w.cu, np.int32)
        ip = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        got = L.varlen_attn_bwd_workspace_size_cu(ip, ip, len(cu) - 1, w.total, w.total, w.hq, w.hkv, w.d, 1)
        delta = _align256(w.total * w.hq * 4)
        part = w.total * w.hkv * w.d * 4
        assert got in {delta, delta + _align256(2 * 2 * part), delta + _align256(4 * 2 * part)}, w.name
        assert got <= L.varlen_attn_bwd_workspace_size(w.total, w.total, w.hq, w.hkv, w.d)
        assert vl.bwd_workspace_bytes_cu(w.cu, w.cu, w.hq, w.hkv, w.d) == got
    # invalid arguments give 0
    bad = np.array([0, 9], np.int32)
    bp = bad.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert L.varlen_attn_bwd_workspace_size_cu(bp, bp, 1, 8, 8, 4, 2, 64, 1) == 0
    assert L.varlen_attn_bwd_workspace_size_cu(ip, ip, 1, 8, 8, 4, 3, 64, 1) == 0


def test_bwd_rejects_small_workspace():
    L = vl.lib()
    cu = np.array([0, 8], np.int32)
    ip = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    f = ctypes.c_void_p(FAKE)
    need = L.varlen_attn_bwd_workspace_size_cu(ip, ip, 1, 8, 8, 4, 2, 64, 1)
    assert need > 0
    rc = L.varlen_attn_bwd(f, f, f, f, f, f, ip, ip, 1, 8, 8, 4, 2, 64, 0.0, 1, f, f, f, f, need - 1, None)
    assert rc == -6
    rc = L.varlen_attn_bwd(f, f, f, f, f, f, ip, ip, 1, 8, 8, 4, 2, 64, 0.0, 1, f, f, f, None, need, None)
    assert rc == -6


def test_permute_and_merge_reject_bad_arguments():
    L = vl.lib()
    f = ctypes.c_void_p(FAKE)
    g = ctypes.c_void_p(FAKE * 64)
    assert L.sp_seq2head(f, g, 16, 6, 128, 4, 2, None) == -2      # 4 does not divide 6
    assert L.sp_seq2head(f, g, 16, 8, 128, 4, 3, None) == -1      # element size
    assert L.sp_seq2head(f, f, 16, 8, 128, 4, 2, None) == -1      # overlap
    assert L.sp_head2seq(None, g, 16, 8, 128, 4, 2, None) == -1
    arr = (ctypes.c_void_p * 2)(FAKE, FAKE * 2)
    assert L.attn_lse_merge(0, arr, arr, 1, 4, 2, 128, g, g, 1, None) == -1
    assert L.attn_lse_merge(65, arr, arr, 1, 4, 2, 128, g, g, 1, None) == -1
    assert L.attn_lse_merge(2, arr, arr, 1, 4, 2, 96, g, g, 1, None) == -4
    assert L.attn_lse_merge(2, arr, arr, 5, 4, 2, 128, g, g, 1, None) == -1
    assert L.attn_lse_merge(2, arr, arr, 1, 4, 2, 128, ctypes.c_void_p(FAKE), g, 1, None) == -1


def test_schedule_export_rejects():
    L = vl.lib()
    bad = np.array([0, 3, 2], np.int32)
    ok = np.array([0, 3, 5], np.int32)
    n = ctypes.c_int64()
    ip = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    assert L.varlen_schedule_export(ip(bad), ip(ok), 2, 1, 0, 128, None, 0, ctypes.byref(n),
                                    None, None, None, None) == -3
    assert L.varlen_schedule_export(ip(ok), ip(ok), 2, 1, 2, 128, None, 0, ctypes.byref(n),
                                    None, None, None, None) == -1
    items = np.zeros(4, np.int32)
    assert L.varlen_schedule_export(ip(ok), ip(ok), 2, 1, 0, 128, ip(items), 0, ctypes.byref(n),
                                    None, None, None, None) == -6


# ---------------------------------------------------------------- ring blocks
def _brute_block(cu, qr, kr):
    """Visible pairs of a (query chunk, key chunk) block of the packed causal
    batch with document mask, straight from the definition."""
    a = np.asarray(cu)
    doc = np.searchsorted(a, np.arange(int(a[-1])), side="right") - 1
    x = np.arange(*qr)
    y = np.arange(*kr)
    return (doc[x][:, None] == doc[y][None, :]) & (y[None, :] <= x[:, None])


def _block_from_call(cu_q, cu_k, causal):
    """Visible pairs of the attention call varlen_ring_block describes."""
    lq = np.diff(cu_q)
    lk = np.diff(cu_k)
    vis = np.zeros((int(cu_q[-1]), int(cu_k[-1])), dtype=bool)
    for b in range(len(lq)):
        for i in range(lq[b]):
            for j in range(lk[b]):
                if not causal or j <= i + lk[b] - lq[b]:
                    vis[cu_q[b] + i, cu_k[b] + j] = True
    return vis


def test_ring_blocks_reproduce_hsap_figure3():
    lines = [ln.split() for ln in open(os.path.join(ROOT, "tests", "golden", "hsap_fig3_step1.txt"))
             if ln.strip() and not ln.startswith("#")]
    cu = [int(x) for x in lines[0][1:]]
    chunk = int(lines[1][1])
    fig = lines[2:]
    n = int(cu[-1]) // chunk
    for r in range(n):
        for s in range(n):
            cq, ck, causal, cls = vl.varlen_ring_block(cu, (r * chunk, (r + 1) * chunk),
                                                       (s * chunk, (s + 1) * chunk))
            assert cls == fig[r][s], (r, s, cls, fig[r][s])
            vis = _brute_block(cu, (r * chunk, (r + 1) * chunk), (s * chunk, (s + 1) * chunk))
            if cls != "N":
                assert np.array_equal(_block_from_call(cq, ck, causal), vis), (r, s)
            else:
                assert not vis.any()


def test_ring_blocks_random_packings_match_brute_force():
    rng = np.random.default_rng(7)
    for trial in range(30):
        lens = workloads.random_lengths(rng, int(rng.integers(1, 7)), 0, 40)
        cu = _cu(lens)
        total = int(cu[-1])
        if total == 0:
            continue
        n = int(rng.integers(1, 6))
        bounds = np.linspace(0, total, n + 1).astype(int)
        for r in range(n):
            for s in range(n):
                qr, kr = (bounds[r], bounds[r + 1]), (bounds[s], bounds[s + 1])
                cq, ck, causal, cls = vl.varlen_ring_block(cu, qr, kr)
                assert cq[-1] == qr[1] - qr[0] and ck[-1] == kr[1] - kr[0]
                vis = _brute_block(cu, qr, kr)
                assert causal == (tuple(qr) == tuple(kr))   # equal ranges: the diagonal
                if cls == "N":
                    assert not vis.any()
                else:
                    assert np.array_equal(_block_from_call(cq, ck, causal), vis), (trial, r, s)
                # the class names the pattern (oracle's classifier on equal chunks)
                if not causal and cls != "N":
                    rows, cols = vis.any(axis=1), vis.any(axis=0)
                    assert (cls == "A2") == bool(vis.all())
                    assert (cls in ("A2", "A3")) == bool(cols.all())
                    assert (cls in ("A2", "A4")) == bool(rows.all())


def test_ring_block_rejects_overlapping_unequal_chunks():
    cu = [0, 10, 30]
    with pytest.raises(vl.VarlenError) as e:
        vl.varlen_ring_block(cu, (0, 20), (10, 30))
    assert e.value.code == -1
    with pytest.raises(vl.VarlenError):
        vl.varlen_ring_block(cu, (0, 40), (0, 40))
    with pytest.raises(vl.VarlenError) as e:
        vl.varlen_ring_block([0, 5, 3], (0, 3), (0, 3))
    assert e.value.code == -3


def test_qkv_permute_rejects_bad_arguments():
    L = vl.lib()
    a, b, c = (ctypes.c_void_p(FAKE * m) for m in (1, 64, 128))
    x, y, z = (ctypes.c_void_p(FAKE * m) for m in (256, 512, 1024))
    ok = (a, b, c, x, y, z)
    for fn in (L.sp_qkv_seq2head, L.sp_qkv_head2seq):
        assert fn(*ok, 16, 6, 2, 128, 4, 0, None) == -2        # 4 does not divide Hq = 6
        assert fn(*ok, 16, 8, 3, 128, 4, 0, None) == -2        # Hkv = 3 does not divide 8
        assert fn(*ok, 16, 12, 3, 128, 2, 0, None) == -2       # neither of 2, 3 divides the other
        assert fn(*ok, 16, 8, 2, 128, 4, 2, None) == -1        # dtype
        assert fn(*ok, 16, 8, 2, 1, 4, 0, None) == -4          # a bf16 head of 2 bytes
        assert fn(None, b, c, x, y, z, 16, 8, 2, 128, 4, 0, None) == -1
        assert fn(a, b, c, x, y, ctypes.c_void_p(FAKE * 1024 + 2), 16, 8, 2, 128, 4, 0,
                  None) == -1                                  # misaligned
        assert fn(a, b, c, x, x, z, 16, 8, 2, 128, 4, 0, None) == -1   # outputs overlap
        assert fn(a, b, c, a, y, z, 16, 8, 2, 128, 4, 0, None) == -1   # output on an input
        assert fn(*ok, -1, 8, 2, 128, 4, 0, None) == -2
        assert fn(*ok, 0, 8, 2, 128, 4, 0, None) == 0           # nothing to do


@pytest.mark.parametrize("N,B", [(1, 1), (8, 1), (8, 2), (8, 4), (8, 8), (6, 3), (4, 8), (2, 6)])
def test_basp_shard_matches_oracle(N, B):
    from oracle import sp_groups
    L = 48
    K = sp_groups.group_size(N, B)
    for r in range(N):
        got = vl.basp_shard(r, N, B, L)
        assert (got["seq_begin"], got["seq_end"], got["tok_begin"], got["tok_end"]) == \
            sp_groups.shard(r, N, B, L)
        assert got["group_size"] == K
        assert r in sp_groups.groups(N, B)[got["group"]]


@pytest.mark.parametrize("args", [(0, 4, 3, 12), (0, 3, 2, 12), (0, 8, 2, 10), (0, 4, 6, 8),
                                  (4, 4, 2, 8), (-1, 4, 2, 8), (0, 0, 1, 4), (0, 4, 2, -2)])
def test_basp_shard_rejects(args):
    with pytest.raises(vl.VarlenError) as e:
        vl.basp_shard(*args)
    assert e.value.code == -2


def test_plan_cache_switch_returns_previous_setting():
    # the switch itself touches no device
    prev = vl.set_plan_cache(False)
    try:
        assert vl.set_plan_cache(False) is False
        assert vl.set_plan_cache(True) is False
        assert vl.set_plan_cache(True) is True
    finally:
        vl.set_plan_cache(prev)


# ---------------------------------------------------------------- binding argument checks
# The C ABI derives every size from q and k; the binding checks the other
# tensors' shapes and dtypes before any pointer reaches the library.  CPU
# tensors are enough: the checks fire before the GPU-placement check.
def _bf(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.bfloat16)


def _f32(*shape):
    import torch
    return torch.zeros(shape, dtype=torch.float32)


def test_fwd_binding_rejects_mismatched_tensors():
    cu = np.array([0, 8], np.int32)
    q, k, v = _bf(8, 4, 64), _bf(8, 2, 64), _bf(8, 2, 64)
    with pytest.raises(ValueError, match="v must have shape"):
        vl.varlen_attn_fwd(q, k, _bf(8, 1, 64), cu, cu)
    with pytest.raises(TypeError, match="k must be bfloat16"):
        vl.varlen_attn_fwd(q, k.float(), v, cu, cu)
    with pytest.raises(ValueError, match="share head_dim"):
        vl.varlen_attn_fwd(q, _bf(8, 2, 128), _bf(8, 2, 128), cu, cu)
    with pytest.raises(ValueError, match="out must have shape"):
        vl.varlen_attn_fwd(q, k, v, cu, cu, out=_bf(8, 4, 32))
    with pytest.raises(ValueError, match="lse must have shape"):
        vl.varlen_attn_fwd(q, k, v, cu, cu, lse=_f32(8, 4))
    with pytest.raises(TypeError, match="lse must be float32"):
        vl.varlen_attn_fwd(q, k, v, cu, cu, lse=_bf(4, 8))
    with pytest.raises(TypeError, match="out_dtype"):
        import torch
        vl.varlen_attn_fwd(q, k, v, cu, cu, out_dtype=torch.float16)
    with pytest.raises(ValueError, match="lse_acc must have shape"):
        vl.varlen_attn_fwd_acc(q, k, v, cu, cu, _f32(8, 4, 64), _f32(8, 4))


def test_bwd_binding_rejects_mismatched_tensors():
    cu = np.array([0, 8], np.int32)
    q, k, v = _bf(8, 4, 64), _bf(8, 2, 64), _bf(8, 2, 64)
    o, do, lse = _bf(8, 4, 64), _bf(8, 4, 64), _f32(4, 8)
    # an fp32 O (what out_dtype=float32 returns) would be read as bf16 pairs
    with pytest.raises(TypeError, match="o must be bfloat16"):
        vl.varlen_attn_bwd(q, k, v, o.float(), do, lse, cu, cu)
    with pytest.raises(ValueError, match="do must have shape"):
        vl.varlen_attn_bwd(q, k, v, o, _bf(8, 2, 64), lse, cu, cu)
    with pytest.raises(ValueError, match="lse must have shape"):
        vl.varlen_attn_bwd(q, k, v, o, do, _f32(2, 8), cu, cu)
    with pytest.raises(ValueError, match="v must have shape"):
        vl.varlen_attn_bwd(q, k, _bf(7, 2, 64), o, do, lse, cu, cu)
    with pytest.raises(ValueError, match="dk must have shape"):
        vl.varlen_attn_bwd(q, k, v, o, do, lse, cu, cu, dk=_bf(8, 4, 64))
    with pytest.raises(TypeError, match="dv must be bfloat16"):
        vl.varlen_attn_bwd(q, k, v, o, do, lse, cu, cu, dv=_f32(8, 2, 64))
    with pytest.raises(ValueError, match="dq must have shape"):
        vl.varlen_attn_bwd(q, k, v, o, do, lse, cu, cu, dq=_bf(8, 2, 64))
    with pytest.raises(TypeError, match="workspace"):
        vl.varlen_attn_bwd(q, k, v, o, do, lse, cu, cu, workspace=_f32(1 << 16))


def test_merge_and_permute_bindings_reject_mismatched_tensors():
    o1, o2 = _f32(8, 2, 16), _f32(8, 2, 16)
    l1, l2 = _f32(2, 8), _f32(2, 8)
    with pytest.raises(ValueError, match=r"lse_parts\[1\] must have shape"):
        vl.attn_lse_merge([o1, o2], [l1, _f32(8, 2)])
    with pytest.raises(TypeError, match=r"o_parts\[1\] must be float32"):
        vl.attn_lse_merge([o1, o2.bfloat16()], [l1, l2])
    with pytest.raises(ValueError, match="out must have shape"):
        vl.attn_lse_merge([o1, o2], [l1, l2], out=_bf(8, 2, 8))
    with pytest.raises(ValueError, match="lse_out must have shape"):
        vl.attn_lse_merge([o1, o2], [l1, l2], lse_out=_f32(8, 2))
    x = _bf(16, 8, 32)
    with pytest.raises(ValueError, match="out must have shape"):
        vl.sp_seq2head(x, 4, out=_bf(4, 16, 4, 32))
    with pytest.raises(TypeError, match="out must be bfloat16"):
        vl.sp_seq2head(x, 4, out=_f32(4, 16, 2, 32))
    with pytest.raises(ValueError, match="out must have shape"):
        vl.sp_head2seq(_bf(4, 16, 2, 32), out=_bf(16, 4, 32))
    q, k, v = _bf(16, 8, 32), _bf(16, 2, 32), _bf(16, 2, 32)
    with pytest.raises(ValueError, match=r"out\[1\] must have shape"):
        vl.sp_qkv_seq2head(q, k, v, 4, out=(_bf(4, 16, 2, 32), _bf(4, 16, 2, 32), _bf(4, 16, 1, 32)))
    yq, yk = _bf(4, 16, 2, 32), _bf(4, 16, 1, 32)
    with pytest.raises(ValueError, match="yk must have shape"):
        vl.sp_qkv_head2seq(yq, _bf(4, 16, 2, 32), _bf(4, 16, 2, 32), 2)
    with pytest.raises(ValueError, match=r"out\[2\] must have shape"):
        vl.sp_qkv_head2seq(yq, yk, yk, 2, out=(_bf(16, 8, 32), _bf(16, 2, 32), _bf(16, 4, 32)))
