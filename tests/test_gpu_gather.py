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


def test_gather_full_size_sampled():
    """64 hits, m ~ U{8192..32768}, k = ceil(r m), r ~ U[0.05, 0.10], hidden
    2560, pool of full prefixes with shuffled pages.  The pool is filled on
    the device from a seeded generator; the oracle computes the source row of
    every packed row, checked for a sample of 4096 rows."""
    import torch
    import linear_attention_state_anchor_amd as sr
    print("[gather] full size", flush=True)
    pc = suffix_pool_case(64, 8192, 32768, 0.05, 0.10, 2560, seed=105)
    gen = torch.Generator(device="cuda").manual_seed(105)
    pool = torch.randint(-32768, 32767, (pc.n_pages, PAGE, 2560), dtype=torch.int16,
                         device="cuda", generator=gen).view(torch.bfloat16)
    total = int(pc.suffix_len.sum())
    packed, cu = sr.gather_suffix(pool, to_dev(pc.page_table), to_dev(pc.matched_len),
                                  to_dev(pc.suffix_len), total)
    idx_pool = np.arange(pc.n_pages * PAGE, dtype=np.int64).reshape(pc.n_pages, PAGE, 1)
    src, cu_ref = oracle.gather_suffix(idx_pool, pc.page_table, pc.matched_len,
                                       pc.suffix_len)
    np.testing.assert_array_equal(cu.cpu().numpy(), cu_ref)
    rows = np.random.default_rng(0).choice(total, 4096, replace=False)
    flat = pool.view(-1, 2560)
    want = flat[torch.from_numpy(src[rows, 0]).cuda()].view(torch.int16)
    got = packed[torch.from_numpy(rows).cuda()].view(torch.int16)
    assert torch.equal(want, got)
