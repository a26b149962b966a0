"""CPU tests of the C ABI: the library loads, exports what the header declares,
and its split-KV planner (host-only plans, no device) covers every token once,
cuts on the granularity, numbers partial slots consecutively, is a pure
function of the lengths, and rejects malformed page tables."""
import ctypes
import os
import re

import numpy as np
import pytest

import mla_paged_kv_decode_amd as mla
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mla.LIB_PATH):
        from mla_paged_kv_decode_amd import build
        build.build()
    return mla.load_library()


def test_exports_match_header(lib):
    hdr = open(os.path.join(ROOT, "include", "mla_decode.h")).read()
    hdr += open(os.path.join(ROOT, "include", "mla_peaks.h")).read()
    declared = set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", hdr))
    assert declared == set(mla.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4, -5):
        assert lib.mla_status_string(st)


def _table(lengths, P):
    rng = np.random.default_rng(0)
    ip, ix, lp, _ = synth.page_table(lengths, P, rng)
    return ip, lp


def _check_plan(plan, lengths, gran):
    seg, wp = plan.segments()
    info = plan.info()
    hs = info["head_split"]
    lengths = [L for L in lengths for _ in range(hs)]  # row r reads request r // hs
    assert wp[0] == 0 and wp[-1] == len(seg) and np.all(np.diff(wp) > 0)
    covered = {}
    for b, t0, t1, slot in seg:
        covered.setdefault(int(b), []).append((int(t0), int(t1), int(slot)))
    slots_seen = set()
    for b, L in enumerate(lengths):
        pieces = sorted(covered[b])
        if L == 0:
            assert pieces == [(0, 0, -1)]
            continue
        assert pieces[0][0] == 0 and pieces[-1][1] == L
        for (a0, a1, _), (b0, _, _) in zip(pieces, pieces[1:]):
            assert a1 == b0
        for t0, t1, _ in pieces:
            assert t1 > t0 and t0 % gran == 0
        if len(pieces) == 1:
            assert pieces[0][2] == -1
        else:
            sl = [p[2] for p in pieces]
            assert sl == list(range(sl[0], sl[0] + len(sl)))
            slots_seen.update(sl)
    assert len(slots_seen) == info["num_partials"]
    return seg, wp, info


@pytest.mark.parametrize("heads,P,lengths", [
    (16, 64, [4096] * 64),
    (128, 64, [4096] * 64),
    (64, 16, list(np.random.default_rng(4).integers(1, 2049, 768))),
    (16, 16, [256] * 4),
    (32, 32, [0, 1, 17, 5000, 33, 0, 64]),
])
def test_plan_covers_each_token_once(lib, heads, P, lengths):
    ip, lp = _table(lengths, P)
    plan = mla.Plan(ip, lp, heads, P, num_cus=256)
    _check_plan(plan, lengths, plan.info()["granularity"])
    assert plan.info()["num_workers"] <= 256


def test_plan_balances_uniform_batch(lib):
    ip, lp = _table([4096] * 64, 64)
    plan = mla.Plan(ip, lp, 16, 64, num_cus=256)
    seg, wp, info = _check_plan(plan, [4096] * 64, plan.info()["granularity"])
    assert info["num_workers"] == 256
    assert set((seg[:, 2] - seg[:, 1]).tolist()) == {1024}


def _worker_loads(seg, wp, heads, lengths):
    # the planner's cost model: tokens + 64 + H per piece, + 4H per piece of a
    # request cut into several
    nsplit = np.bincount(seg[:, 0], minlength=len(lengths))
    cost = (seg[:, 2] - seg[:, 1]) + 64 + heads + np.where(nsplit[seg[:, 0]] > 1, 4 * heads, 0)
    return np.array([cost[wp[i]:wp[i + 1]].sum() for i in range(len(wp) - 1)])


def test_plan_balances_variable_lengths(lib):
    # 768 requests of 1..2048 tokens on 256 workers, about three each: the
    # longest-first assignment alone leaves the busiest worker ~9% above the
    # mean; the refinement brings it within 1%
    lengths = [int(x) for x in np.random.default_rng(4).integers(1, 2049, 768)]
    ip, lp = _table(lengths, 16)
    plan = mla.Plan(ip, lp, 64, 16, num_cus=256)
    seg, wp, info = _check_plan(plan, lengths, plan.info()["granularity"])
    loads = _worker_loads(seg, wp, 64, lengths)
    assert info["num_workers"] == 256
    assert loads.max() <= 1.01 * loads.mean(), (loads.max(), loads.mean())


def test_plan_is_pure_function_of_lengths(lib):
    lengths = list(np.random.default_rng(9).integers(1, 3000, 300))
    ip, lp = _table(lengths, 16)
    a = mla.Plan(ip, lp, 64, 16, num_cus=256).segments()
    b = mla.Plan(ip.copy(), lp.copy(), 64, 16, num_cus=256).segments()
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_force_splits(lib):
    lengths = [1000, 64, 1, 0]
    ip, lp = _table(lengths, 16)
    plan = mla.Plan(ip, lp, 16, 16, num_cus=8, force_splits=3)
    seg, wp, info = _check_plan(plan, lengths, plan.info()["granularity"])
    counts = {b: int((seg[:, 0] == b).sum()) for b in range(4)}
    g = info["granularity"]

    def pieces(L):  # near-equal chunks on multiples of the granularity
        if L == 0:
            return 1
        n = min(3, -(-L // g))
        step = -(-(-(-L // n)) // g) * g
        return -(-L // step)
    assert counts == {b: pieces(L) for b, L in enumerate(lengths)}
    assert counts[0] == 3


def test_workspace_bound_covers_plan(lib):
    lengths = list(np.random.default_rng(5).integers(1, 5000, 100))
    ip, lp = _table(lengths, 64)
    for heads in (16, 128):
        n = mla.workspace_bytes(100, heads, num_cus=256)
        plan = mla.Plan(ip, lp, heads, 64, num_cus=256)
        info = plan.info()
        need = info["num_partials"] * heads * (512 + 1) * 4 + info["num_segments"] * 16
        assert n >= need


@pytest.mark.parametrize("bad", ["indptr_start", "indptr_decreasing", "last_zero", "last_big"])
def test_malformed_tables_rejected(lib, bad):
    ip = np.array([0, 2, 4], np.int32)
    lp = np.array([16, 3], np.int32)
    if bad == "indptr_start":
        ip[0] = 1
    elif bad == "indptr_decreasing":
        ip = np.array([0, 3, 2], np.int32)
    elif bad == "last_zero":
        lp[1] = 0
    else:
        lp[0] = 17
    with pytest.raises(mla.MlaError) as e:
        mla.Plan(ip, lp, 16, 16, num_cus=4)
    assert e.value.status == -1


@pytest.mark.parametrize("heads,P", [(8, 16), (48, 16), (16, 8), (16, 128)])
def test_unsupported_shapes_rejected(lib, heads, P):
    with pytest.raises(mla.MlaError) as e:
        mla.Plan(np.array([0, 1], np.int32), np.array([1], np.int32), heads, P, num_cus=4)
    assert e.value.status == -2


def test_run_without_workspace_is_refused(lib):
    plan = mla.Plan(np.array([0, 1], np.int32), np.array([1], np.int32), 16, 16, num_cus=4)
    P = ctypes.c_void_p
    st = lib.mla_decode_run(plan._h, P(1), P(1), P(1), P(1), None, P(1), P(1), P(1),
                            ctypes.c_float(0.1), P(1), P(1), None)
    assert st == -5


def test_head_split_automatic_choice(lib):
    # bf16 keeps every head of a request in one workgroup
    ip, lp = _table([4096] * 64, 64)
    info = mla.Plan(ip, lp, 128, 64, num_cus=256).info()
    assert info["head_split"] == 1 and info["kernel_heads"] == 128
    lengths = list(np.random.default_rng(4).integers(1, 2049, 768))
    ip, lp = _table(lengths, 16)
    info = mla.Plan(ip, lp, 64, 16, num_cus=256).info()
    assert info["head_split"] == 1 and info["kernel_heads"] == 64
    # 8-bit caches: 16 and 128 heads in one workgroup, 32 and 64 as 16-head rows
    ip, lp = _table([8192] * 64, 64)
    for heads in (16, 32, 64, 128):
        for kvd in (mla.KV_FP8_E4M3, mla.KV_INT8):
            info = mla.Plan(ip, lp, heads, 64, kvd, num_cus=256).info()
            hs = 1 if heads in (16, 128) else heads // 16
            assert info["head_split"] == hs and info["kernel_heads"] == heads // hs
    plan = mla.Plan(ip, lp, 64, 64, mla.KV_FP8_E4M3, num_cus=256)
    _check_plan(plan, [8192] * 64, plan.info()["granularity"])


def test_8bit_rejects_unserved_rows(lib):
    ip, lp = _table([100], 16)
    for hs in (2, 4):  # 64- and 32-head rows have no 8-bit kernel
        with pytest.raises(mla.MlaError) as e:
            mla.Plan(ip, lp, 128, 16, mla.KV_INT8, num_cus=8, head_split=hs)
        assert e.value.status == -2
    for hs in (1, 8):
        assert mla.Plan(ip, lp, 128, 16, mla.KV_INT8, num_cus=8, head_split=hs).info()[
            "head_split"] == hs
    with pytest.raises(mla.MlaError):
        mla.Plan(ip, lp, 16, 16, 6, num_cus=8)


def test_workspace_bound_covers_8bit_plans(lib):
    lengths = list(np.random.default_rng(6).integers(1, 9000, 64))
    ip, lp = _table(lengths, 64)
    for heads in (16, 128):
        n = mla.workspace_bytes(64, heads, num_cus=256)
        info = mla.Plan(ip, lp, heads, 64, mla.KV_FP8_E4M3, num_cus=256).info()
        need = info["num_partials"] * 16 * (512 + 1) * 4 + info["num_segments"] * 16
        assert n >= need


@pytest.mark.parametrize("heads,hs", [(128, 1), (128, 2), (128, 4), (64, 2), (32, 2)])
def test_head_split_explicit(lib, heads, hs):
    lengths = [333, 4096, 17, 0, 1000]
    ip, lp = _table(lengths, 32)
    plan = mla.Plan(ip, lp, heads, 32, num_cus=64, head_split=hs)
    info = plan.info()
    assert info["head_split"] == hs and info["kernel_heads"] == heads // hs
    _check_plan(plan, lengths, info["granularity"])


def test_head_split_rows_share_an_xcd(lib):
    ip, lp = _table([4096] * 64, 64)
    plan = mla.Plan(ip, lp, 128, 64, num_cus=256, head_split=4)
    seg, wp = plan.segments()
    xcd_of_request = {}
    for w in range(len(wp) - 1):
        for s_ in seg[wp[w]:wp[w + 1]]:
            xcd_of_request.setdefault(int(s_[0]) // 4, set()).add(w % 8)
    assert len(xcd_of_request) == 64
    assert all(len(x) == 1 for x in xcd_of_request.values())


@pytest.mark.parametrize("heads,kvd", [(16, mla.KV_BF16), (128, mla.KV_BF16),
                                       (128, mla.KV_FP8_E4M3)])
def test_chunks_of_a_request_share_an_xcd(lib, heads, kvd):
    # one row per request, cut into 4 token chunks: the chunks read the same
    # query rows, so they get launch positions congruent mod 8 (one L2), and
    # the kernels still find each segment's request from its index alone
    ip, lp = _table([4096] * 64, 64)
    plan = mla.Plan(ip, lp, heads, 64, kvd, num_cus=256)
    info = plan.info()
    assert info["head_split"] == 1
    seg, wp, _ = _check_plan(plan, [4096] * 64, info["granularity"])
    assert len(seg) == 256 and info["num_workers"] == 256
    xcd = {}
    for w in range(len(wp) - 1):
        for s_ in seg[wp[w]:wp[w + 1]]:
            xcd.setdefault(int(s_[0]), set()).add(w % 8)
    assert len(xcd) == 64 and all(len(x) == 1 for x in xcd.values())
    # the fast path's closed form: segment i reads request rank(i) / c
    assert info["one_seg"] == 1 and info["req_div"] == 4 and info["req_deal"] == 8
    n, X = info["num_workers"], info["req_deal"]
    rank = [(i % X) * (n // X) + i // X for i in range(n)]
    assert [int(seg[i, 0]) for i in range(n)] == [r // info["req_div"] for r in rank]
    # without placement: launch order is request order
    flat = mla.Plan(ip, lp, heads, 64, kvd, num_cus=256, l2_domains=1).info()
    assert flat["req_div"] == 4 and flat["req_deal"] == 0


@pytest.mark.parametrize("heads,q,kvd", [(128, 2, mla.KV_BF16), (64, 1, mla.KV_FP8_E4M3),
                                         (16, 4, mla.KV_INT8)])
def test_rows_of_a_request_share_an_xcd_with_token_splits(lib, heads, q, kvd):
    # rows of one request (several per request, each also cut into token
    # chunks) get launch positions congruent mod 8, i.e. one L2 domain
    ip, lp = _table([4096] * 64, 64)
    plan = mla.Plan(ip, lp, heads, 64, kvd, num_cus=256, qo_len=q)
    hs = plan.info()["head_split"]
    assert hs > 1
    seg, wp = plan.segments()
    assert len(seg) >= 64 * hs  # (128 heads x 2 queries: rows also cut into chunks)
    xcd = {}
    for w in range(len(wp) - 1):
        for s_ in seg[wp[w]:wp[w + 1]]:
            xcd.setdefault(int(s_[0]) // hs, set()).add(w % 8)
    # (each workgroup serves one request here, and the domains hold whole requests)
    assert len(xcd) == 64 and all(len(x) == 1 for x in xcd.values())
    # l2_domains = 1 turns the placement off (same segments, other order)
    flat = mla.Plan(ip, lp, heads, 64, kvd, num_cus=256, qo_len=q, l2_domains=1)
    seg1, _ = flat.segments()
    assert sorted(map(tuple, seg1.tolist())) == sorted(map(tuple, seg.tolist()))
    with pytest.raises(mla.MlaError):
        mla.Plan(ip, lp, heads, 64, kvd, num_cus=256, qo_len=q, l2_domains=-1)


def test_bad_head_split_rejected(lib):
    ip, lp = _table([10], 16)
    for heads, hs in ((128, 3), (16, 2), (64, 8)):
        with pytest.raises(mla.MlaError):
            mla.Plan(ip, lp, heads, 16, num_cus=8, head_split=hs)


@pytest.mark.parametrize("heads,q,kvd,width", [
    (16, 1, mla.KV_BF16, 16), (16, 2, mla.KV_BF16, 32), (16, 3, mla.KV_BF16, 16),
    (16, 4, mla.KV_BF16, 64), (16, 8, mla.KV_BF16, 128), (16, 16, mla.KV_BF16, 128),
    (128, 2, mla.KV_BF16, 128), (32, 3, mla.KV_BF16, 32), (16, 2, mla.KV_FP8_E4M3, 16),
    (16, 1, mla.KV_FP8_E4M3_KPE_BF16, 16), (128, 1, mla.KV_INT8_KPE_BF16, 128),
    (64, 1, mla.KV_FP8_E4M3_KPE_BF16, 16), (64, 2, mla.KV_INT8_KPE_BF16, 128),
    (16, 1, mla.KV_FP16, 16), (32, 1, mla.KV_FP16, 16), (128, 1, mla.KV_FP16, 128),
    (64, 2, mla.KV_INT8, 128), (16, 6, mla.KV_INT8, 16), (128, 4, mla.KV_FP8_E4M3, 128)])
def test_multiquery_rows(lib, heads, q, kvd, width):
    # the qo_len * heads query vectors of a request run as rows of the largest
    # served width that divides them, each row reading the request's cache
    lengths = [333, 4096, 17, 0, 1000, 2]
    ip, lp = _table(lengths, 32)
    plan = mla.Plan(ip, lp, heads, 32, kvd, num_cus=64, qo_len=q)
    info = plan.info()
    assert info["qo_len"] == q and info["kernel_heads"] == width
    assert info["head_split"] == heads * q // width
    _check_plan(plan, lengths, info["granularity"])
    n = mla.workspace_bytes(len(lengths), heads, num_cus=64, qo_len=q)
    need = info["num_partials"] * width * (512 + 1) * 4 + info["num_segments"] * 32
    assert n >= need


def test_multiquery_bad_qo_len_rejected(lib):
    ip, lp = _table([10, 20], 16)
    for q in (-1, 65):
        with pytest.raises(mla.MlaError) as e:
            mla.Plan(ip, lp, 16, 16, num_cus=8, qo_len=q)
        assert e.value.status == -1
    with pytest.raises(mla.MlaError):
        mla.workspace_bytes(2, 16, num_cus=8, qo_len=65)
    assert mla.Plan(ip, lp, 16, 16, num_cus=8, qo_len=0).info()["qo_len"] == 1
    # a head split that does not divide the query vectors
    with pytest.raises(mla.MlaError):
        mla.Plan(ip, lp, 16, 16, num_cus=8, qo_len=3, head_split=2)


def test_cache_append_rejects_bad_arguments(lib):
    # every check happens before any HIP call, so this runs without a GPU
    Pp = ctypes.c_void_p
    assert lib.mla_cache_append(Pp(1), Pp(1), Pp(1), -1, 0, Pp(1), Pp(1), None, None) == -1
    assert lib.mla_cache_append(Pp(1), Pp(1), Pp(1), 4, 6, Pp(1), Pp(1), None, None) == -2
    assert lib.mla_cache_append(Pp(1), Pp(1), Pp(1), 4, 5, Pp(1), Pp(1), Pp(1), None) == -1
    assert lib.mla_cache_append(Pp(1), Pp(1), Pp(1), 4, -1, Pp(1), Pp(1), None, None) == -2
    assert lib.mla_cache_append(Pp(1), Pp(1), Pp(1), 4, 3, Pp(1), Pp(1), None, None) == -1
    assert lib.mla_cache_append(Pp(1), Pp(1), Pp(1), 4, 1, Pp(1), Pp(1), None, None) == -1
    assert lib.mla_cache_append(Pp(1), Pp(1), Pp(1), 4, 0, Pp(1), Pp(1), Pp(1), None) == -1
    assert lib.mla_cache_append(None, None, Pp(1), 4, 0, Pp(1), Pp(1), None, None) == -1
    assert lib.mla_cache_append(None, None, None, 0, 1, None, None, None, None) == 0


def test_run_rejects_metadata_that_differs_from_the_plan():
    # the binding checks the device metadata's sizes against the plan's host
    # copies before anything reaches the library (CPU tensors suffice: the
    # check comes first)
    torch = pytest.importorskip("torch")
    import mla_paged_kv_decode_amd as mla
    indptr = np.array([0, 2, 5], np.int32)
    last = np.array([3, 16], np.int32)
    plan = mla.Plan(indptr, last, 16, 16, num_cus=8)
    B, H = 2, 16
    q_nope = torch.zeros((B, H, 512), dtype=torch.bfloat16)
    q_pe = torch.zeros((B, H, 64), dtype=torch.bfloat16)
    ckv = torch.zeros((5, 16, 512), dtype=torch.bfloat16)
    kpe = torch.zeros((5, 16, 64), dtype=torch.bfloat16)
    o = torch.zeros((B, H, 512), dtype=torch.bfloat16)
    lse = torch.zeros((B, H), dtype=torch.float32)
    i32 = lambda a: torch.tensor(a, dtype=torch.int32)
    good = (i32(indptr), i32(np.arange(5)), i32(last))
    bad = [(i32(indptr[:2]), good[1], good[2]),          # kv_indptr too short
           (good[0], good[1], i32(last[:1])),            # kv_last_page_len too short
           (good[0], i32(np.arange(4)), good[2])]        # fewer kv_indices than pages
    for ip, ix, lp in bad:
        with pytest.raises(ValueError):
            plan.run(q_nope, q_pe, ckv, kpe, None, ip, ix, lp, 0.07, o, lse)
    # with the right sizes, the next check is the device one
    with pytest.raises(ValueError, match="device"):
        plan.run(q_nope, q_pe, ckv, kpe, None, *good, 0.07, o, lse)


C_PROGRAM = r"""
#include <stdio.h>
#include <stdlib.h>
#include "mla_decode.h"
#include "mla_peaks.h"

/* a host-only plan through the public header, from C: three requests of
   1000, 0 and 33 tokens in 16-token pages; every token planned once */
int main(void) {
  const int32_t indptr[4] = {0, 63, 63, 66};
  const int32_t last[3] = {8, 1, 1};
  mla_plan_opts opts = {0};
  opts.num_cus = 256;
  size_t ws = mla_decode_workspace_bytes(3, 64, &opts);
  mla_plan_t plan = NULL;
  mla_status st = mla_decode_plan(&plan, indptr, last, 3, 64, 16, MLA_KV_BF16, &opts, NULL, 0,
                                  NULL);
  if (ws == 0 || st != MLA_OK) {
    printf("plan failed: %s %s\n", mla_status_string(st), mla_last_error());
    return 1;
  }
  int32_t info[16];
  if (mla_decode_plan_info(plan, info) != MLA_OK) return 2;
  int32_t* seg = (int32_t*)malloc(sizeof(int32_t) * 4 * (size_t)(info[5] > 0 ? info[5] : 1));
  int32_t* wp = (int32_t*)malloc(sizeof(int32_t) * (size_t)(info[4] + 1));
  if (mla_decode_plan_segments(plan, seg, wp) != MLA_OK) return 3;
  long covered[3] = {0, 0, 0};
  for (int i = 0; i < info[5]; ++i) covered[seg[4 * i]] += seg[4 * i + 2] - seg[4 * i + 1];
  printf("%ld %ld %ld %d\n", covered[0], covered[1], covered[2], info[4]);
  free(seg);
  free(wp);
  mla_decode_plan_destroy(plan);
  /* an invalid kv_dtype is an error, not undefined behaviour */
  st = mla_decode_plan(&plan, indptr, last, 3, 64, 16, 99, &opts, NULL, 0, NULL);
  return st == MLA_OK ? 4 : 0;
}
"""


def test_header_is_plain_c_and_plans_from_c(lib, tmp_path):
    # the public headers compile as C99 with warnings as errors, and a C
    # program linked to the library plans a batch (host only)
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc missing")
    src = tmp_path / "plan.c"
    src.write_text(C_PROGRAM)
    exe = str(tmp_path / "plan")
    libdir = os.path.dirname(mla.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", exe,
                    "-L", libdir, "-l:libmla_decode.so", "-Wl,-rpath," + libdir],
                   check=True, capture_output=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    covered = [int(x) for x in r.stdout.split()]
    assert covered[:3] == [1000, 0, 33] and covered[3] > 0
