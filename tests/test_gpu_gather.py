"""GPU anchor gather (sr_gather_suffix): bit-exact against the oracle's
fancy indexing, with cu_seqlens, page-boundary crossings, empty replays,
whole-prefix replays, and a sentinel showing nothing outside the packed rows
is written."""
import numpy as np
import pytest

import oracle
from replay_inputs import PAGE, suffix_pool_case
from tests.util import to_dev

pytestmark = pytest.mark.gpu


def _run(pc, pool_np, total=None, packed_rows=None):
    import torch
    import linear_attention_state_anchor_amd as sr
    pool = to_dev(pool_np)
    total = int(pc.suffix_len.sum()) if total is None else total
    rows = total if packed_rows is None else packed_rows
    packed = torch.full((rows, pc.hidden), -1, dtype=torch.int16, device="cuda").view(
        pool.dtype)
    out, cu = sr.gather_suffix(pool, to_dev(pc.page_table), to_dev(pc.matched_len),
                               to_dev(pc.suffix_len), total, packed=packed)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), cu.cpu().numpy()


def test_gather_small_bit_exact():
    print("[gather] small", flush=True)
    pc = suffix_pool_case(7, 65, 700, 0.05, 0.6, 128, seed=3, spare_pages=5)
    pool = pc.pool()
    got, cu = _run(pc, pool)
    ref, cu_ref = oracle.gather_suffix(pool, pc.page_table, pc.matched_len, pc.suffix_len)
    np.testing.assert_array_equal(cu, cu_ref)
    np.testing.assert_array_equal(got, ref)


def test_gather_edge_requests_and_sentinel():
    print("[gather] edges", flush=True)
    pc = suffix_pool_case(5, 64, 200, 0.1, 0.2, 64, seed=5)
    # k = 0, k = m (whole prefix), a suffix ending exactly on a page edge,
    # one starting exactly on a page edge
    pc.suffix_len[:] = [0, pc.matched_len[1], 64, 1, 65]
    pc.matched_len[2] = 128
    pool = pc.pool()
    total = int(pc.suffix_len.sum())
    got, cu = _run(pc, pool, total=total, packed_rows=total + 9)
    ref, cu_ref = oracle.gather_suffix(pool, pc.page_table, pc.matched_len, pc.suffix_len)
    np.testing.assert_array_equal(cu, cu_ref)
    np.testing.assert_array_equal(got[:total], ref)
    assert np.all(got[total:] == 0xFFFF)


def test_gather_fp32_elements():
    print("[gather] fp32", flush=True)
    pc = suffix_pool_case(3, 100, 300, 0.2, 0.5, 32, seed=9)
    rng = np.random.default_rng(2)
    pool = rng.standard_normal((pc.n_pages, PAGE, 32)).astype(np.float32)
    import torch
    import linear_attention_state_anchor_amd as sr
    out, cu = sr.gather_suffix(to_dev(pool), to_dev(pc.page_table), to_dev(pc.matched_len),
                               to_dev(pc.suffix_len))
    ref, _ = oracle.gather_suffix(pool, pc.page_table, pc.matched_len, pc.suffix_len)
    np.testing.assert_array_equal(out.cpu().numpy(), ref)


def test_gather_full_size_every_row():
    """64 hits, m ~ U{8192..32768}, k = ceil(r m), r ~ U[0.05, 0.10], hidden
    2560, pool of full prefixes with shuffled pages.  The pool is filled on
    the device from a seeded generator; the oracle computes the source row of
    every packed row (fancy indexing of a pool of row indices), and every
    packed row is compared bit for bit on the device."""
    import torch
    import linear_attention_state_anchor_amd as sr
    print("[gather] full size", flush=True)
    pc = suffix_pool_case(64, 8192, 32768, 0.05, 0.10, 2560, seed=105)
    gen = torch.Generator(device="cuda").manual_seed(105)
    pool = torch.randint(-32768, 32767, (pc.n_pages, PAGE, 2560), dtype=torch.int16,
                         device="cuda", generator=gen).view(torch.bfloat16)
    total = int(pc.suffix_len.sum())
    packed = torch.full((total + 7, 2560), -1, dtype=torch.int16, device="cuda")
    packed_bf, cu = sr.gather_suffix(pool, to_dev(pc.page_table), to_dev(pc.matched_len),
                                     to_dev(pc.suffix_len), total,
                                     packed=packed.view(torch.bfloat16))
    idx_pool = np.arange(pc.n_pages * PAGE, dtype=np.int64).reshape(pc.n_pages, PAGE, 1)
    src, cu_ref = oracle.gather_suffix(idx_pool, pc.page_table, pc.matched_len,
                                       pc.suffix_len)
    np.testing.assert_array_equal(cu.cpu().numpy(), cu_ref)
    assert src.shape[0] == total
    flat = pool.view(torch.int16).view(-1, 2560)
    want = flat[torch.from_numpy(src[:, 0]).cuda()]
    assert torch.equal(want, packed[:total]), "a packed row differs from its source row"
    assert bool((packed[total:] == -1).all()), "rows past the packed total were written"
    print(f"    {total} rows bit-exact", flush=True)


# ---------------------------------------------------------------------------
# token-wise sparse anchors ("SuffixReplay", Algorithm Design 2-3): each
# 64-token page keeps an anchor block of A rows at fixed in-page offsets, and
# the replay takes the last k = min(ceil(0.05 n), k_max) anchors
# ---------------------------------------------------------------------------
NEAR = (60, 61, 62, 63)     # density 1/16 next to the page boundary
UNIFORM = (15, 31, 47, 63)  # density 1/16 spread over the page


def _sparse_case(n_req, m_lo, m_hi, offs, k_max, hidden, seed):
    pc = suffix_pool_case(n_req, m_lo, m_hi, 0.05, 0.10, hidden, seed)
    n_anchor = [len(oracle.anchor_positions(int(m), offs)) for m in pc.matched_len]
    k = np.asarray(oracle.replay_budget(n_anchor, 0.05, k_max), np.int32)
    return pc, n_anchor, k


@pytest.mark.parametrize("offs", [NEAR, UNIFORM, (0, 17, 33)])
def test_sparse_gather_small_bit_exact(offs):
    import torch
    import linear_attention_state_anchor_amd as sr
    print(f"[gather] sparse small offsets={offs}", flush=True)
    pc, n_anchor, k = _sparse_case(9, 1, 5000, offs, 128, 128, seed=11)
    k[0] = n_anchor[0]                              # one request replays all its anchors
    assert sr.replay_budget(n_anchor[1:], 0.05, 128) == list(k[1:])
    rng = np.random.default_rng(4)
    pool = rng.integers(0, 2 ** 16, size=(pc.n_pages, len(offs), 128), dtype=np.uint16)
    total = int(k.sum())
    packed = torch.full((total + 5, 128), -1, dtype=torch.int16, device="cuda")
    out, cu, pos = sr.gather_anchors(to_dev(pool), offs, to_dev(pc.page_table),
                                     to_dev(pc.matched_len), to_dev(k), total,
                                     packed=packed.view(torch.bfloat16))
    torch.cuda.synchronize()
    ref, cu_ref, pos_ref = oracle.gather_anchors(pool, offs, pc.page_table, pc.matched_len, k)
    np.testing.assert_array_equal(cu.cpu().numpy(), cu_ref)
    np.testing.assert_array_equal(pos.cpu().numpy(), pos_ref)
    got = packed.cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got[:total], ref)
    assert np.all(got[total:] == 0xFFFF)


@pytest.mark.parametrize("k_max", [256, 512])
def test_sparse_gather_full_size_every_row(k_max):
    """64 hits, m ~ U{8192..32768}, density 1/16 next to the page boundary,
    k = min(ceil(0.05 n), k_max) anchors, hidden 2560: every packed row and
    every position bit-exact against the oracle's source indices."""
    import torch
    import linear_attention_state_anchor_amd as sr
    print(f"[gather] sparse full size k_max={k_max}", flush=True)
    pc, n_anchor, k = _sparse_case(64, 8192, 32768, NEAR, k_max, 2560, seed=105)
    gen = torch.Generator(device="cuda").manual_seed(106)
    pool = torch.randint(-32768, 32767, (pc.n_pages, 4, 2560), dtype=torch.int16,
                         device="cuda", generator=gen)
    total = int(k.sum())
    packed, cu, pos = sr.gather_anchors(pool.view(torch.bfloat16), NEAR, to_dev(pc.page_table),
                                        to_dev(pc.matched_len), to_dev(k), total)
    idx_pool = np.arange(pc.n_pages * 4, dtype=np.int64).reshape(pc.n_pages, 4, 1)
    src, cu_ref, pos_ref = oracle.gather_anchors(idx_pool, NEAR, pc.page_table,
                                                 pc.matched_len, k)
    np.testing.assert_array_equal(cu.cpu().numpy(), cu_ref)
    np.testing.assert_array_equal(pos.cpu().numpy(), pos_ref)
    want = pool.view(-1, 2560)[torch.from_numpy(src[:, 0]).cuda()]
    assert torch.equal(want, packed.view(torch.int16))
    print(f"    {total} rows and positions bit-exact", flush=True)


# ---------------------------------------------------------------------------
# device-side precondition checks (sr_check_gather_inputs and the SR_DEBUG
# path); the bad inputs only ever reach the validation kernels
# ---------------------------------------------------------------------------
def test_check_gather_inputs_flags_bad_data():
    import linear_attention_state_anchor_amd as sr
    print("[gather] precondition checks", flush=True)
    pc = suffix_pool_case(6, 100, 900, 0.05, 0.5, 64, seed=8)
    pt, m, k = pc.page_table.copy(), pc.matched_len.copy(), pc.suffix_len.copy()
    total = int(k.sum())

    def run(pt_, m_, k_, total_=total, n_pages=pc.n_pages, offs=None):
        sr.check_gather_inputs(n_pages, to_dev(pt_), to_dev(m_), to_dev(k_), total_, offs)

    run(pt, m, k)                                   # a valid batch passes
    bad = pt.copy()
    last = (int(m[2]) - 1) // 64
    bad[2, last] = pc.n_pages + 3                   # page id past the pool
    with pytest.raises(ValueError):
        run(bad, m, k)
    k2 = k.copy()
    k2[1] = m[1] + 1                                 # more anchors than the prefix holds
    with pytest.raises(ValueError):
        run(pt, m, k2, int(k2.sum()))
    with pytest.raises(ValueError):
        run(pt, m, k, total + 1)                     # total does not match sum k
    m2 = m.copy()
    m2[3] = -5
    with pytest.raises(ValueError):
        run(pt, m2, k)
    # sparse anchors: a request asks for more anchors than its pages keep
    n_near = [len(oracle.anchor_positions(int(x), NEAR)) for x in m]
    k3 = np.asarray(n_near, np.int32)
    run(pt, m, k3, int(k3.sum()), offs=NEAR)
    k3[0] += 1
    with pytest.raises(ValueError):
        run(pt, m, k3, int(k3.sum()), offs=NEAR)


def test_sr_debug_gather_returns_before_enqueue(monkeypatch):
    """With SR_DEBUG=1 a gather whose page table points outside the pool is
    rejected before any copy is enqueued: the output stays untouched."""
    import torch
    import linear_attention_state_anchor_amd as sr
    print("[gather] SR_DEBUG", flush=True)
    monkeypatch.setenv("SR_DEBUG", "1")
    pc = suffix_pool_case(3, 100, 300, 0.2, 0.5, 32, seed=12)
    pool = to_dev(pc.pool())
    total = int(pc.suffix_len.sum())
    packed = torch.full((total, 32), 7, dtype=torch.int16, device="cuda")
    pt = pc.page_table.copy()
    pt[0, (int(pc.matched_len[0]) - 1) // 64] = pc.n_pages
    with pytest.raises(ValueError):
        sr.gather_suffix(pool, to_dev(pt), to_dev(pc.matched_len), to_dev(pc.suffix_len), total,
                         packed=packed.view(torch.bfloat16))
    torch.cuda.synchronize()
    assert bool((packed == 7).all())
    out, _ = sr.gather_suffix(pool, to_dev(pc.page_table), to_dev(pc.matched_len),
                              to_dev(pc.suffix_len), total)    # valid: runs
    ref, _ = oracle.gather_suffix(pc.pool(), pc.page_table, pc.matched_len, pc.suffix_len)
    np.testing.assert_array_equal(out.view(torch.int16).cpu().numpy().view(np.uint16), ref)
