"""Shared-prefix (cascade) decode on the GPU, through the C ABI.  Each query
row still attends to its sequence's whole context, so the oracle is the one
of plain decode (fp64 attention over the oracle's quantisation of the same
bf16 inputs): max |err| <= 2e-3 and relative L2 <= 1e-3 over every output.
The plain FP4 decode of the same cache is a second reference: the two
differ only by fp32 summation order and by where each level rounds its
softmax weights to bf16 hi + lo (SPLIT_RTOL / SPLIT_ATOL)."""
import numpy as np
import pytest

import bit_quantized_kv_rotate_amd as kvq
import kvq_synth as syn
from kvq_gpu_util import SPLIT_ATOL as ATOL, SPLIT_RTOL as RTOL, Filled, assert_close, oracle_decode_batch

pytestmark = pytest.mark.gpu


def _mix(name, batch, hkv, group, n_q, ctx, P=16, n_prefixes=2, frac=0.92):
    return syn.Workload(name, batch=batch, num_kv_heads=hkv, num_q_heads=hkv * group, head_dim=128,
                        page_size=P, context=0, n_q=n_q, ctx_range=ctx, n_prefixes=n_prefixes,
                        shared_frac=frac)


def _check_all(f, q, out, what):
    want = oracle_decode_batch(f, syn.bf16_bits(q))
    for b in range(f.wl.batch):
        assert_close(out[b], want[b], "%s seq %d (L=%d)" % (what, b, int(f.plan.context_lens[b])))


@pytest.mark.parametrize("group,n_q,P,ctx", [
    (8, 3, 16, (200, 3000)),     # 24 rows per KV head: one-wave suffix kernel
    (4, 1, 32, (100, 2500)),     # 4 rows, page 32
    (16, 3, 16, (300, 2000)),    # 48 rows: many-row suffix kernel
    (2, 2, 64, (64, 1800)),      # page 64
])
def test_shared_prefix_matches_oracle(gpu, group, n_q, P, ctx):
    wl = _mix("shared_g%d_nq%d_p%d" % (group, n_q, P), batch=8, hkv=2, group=group, n_q=n_q, ctx=ctx, P=P)
    f = Filled(wl, "fp4")
    q = syn.queries(wl).cuda()
    out = f.decode_shared(q).cpu().numpy()
    _check_all(f, q, out, "shared g%d n_q%d P%d" % (group, n_q, P))
    plain = f.decode(q).cpu().numpy()
    np.testing.assert_allclose(out, plain, rtol=RTOL, atol=ATOL)


def test_shared_prefix_edge_cases(gpu):
    """Shared lengths that end inside a page, shared parts that cover verify
    tokens, a sequence with no suffix at all, one in no group, and a
    sequence that shares nothing although its group exists."""
    wl = _mix("shared_edges", batch=6, hkv=2, group=4, n_q=3, ctx=None, P=32)
    lens = [545, 1000, 642, 97, 800, 64]
    pages = [17, 20, 20, 3, 0, 2]            # whole pages taken from prefix b % 2
    plan = syn.page_plan(wl, lens=lens, shared_pages=pages)
    f = Filled(wl, "fp4", plan=plan)
    q = syn.queries(wl).cuda()
    shared = [
        544,        # 1 own token: the shared part holds 2 of the 3 verify tokens
        640 - 16,   # ends inside a page: the suffix starts mid-page (still prefix data)
        640 - 32,   # one whole shared page left to the suffix scan
        96,         # 1 own token
        0,          # shares nothing: in no group
        64,         # the whole context is shared: no suffix
    ]
    groups = f.prefix_groups(shared)
    out = f.decode_shared(q, groups).cpu().numpy()
    _check_all(f, q, out, "shared edges")
    plain = f.decode(q).cpu().numpy()
    np.testing.assert_allclose(out, plain, rtol=RTOL, atol=ATOL)
    for s in (1, 2, 7):
        got = f.decode_shared(q, groups, flags=kvq.splits_flag(s)).cpu().numpy()
        np.testing.assert_allclose(got, out, rtol=RTOL, atol=ATOL)


def test_shared_prefix_with_nothing_shared_equals_plain(gpu):
    wl = _mix("shared_none", batch=4, hkv=2, group=8, n_q=1, ctx=(40, 900), n_prefixes=2, frac=0.5)
    f = Filled(wl, "fp4")
    q = syn.queries(wl).cuda()
    out = f.decode_shared(q, f.prefix_groups([0] * wl.batch)).cpu().numpy()
    plain = f.decode(q).cpu().numpy()
    np.testing.assert_allclose(out, plain, rtol=RTOL, atol=ATOL)
    _check_all(f, q, out, "nothing shared")


def test_shared_prefix_split_invariance(gpu):
    wl = _mix("shared_split", batch=6, hkv=1, group=8, n_q=3, ctx=(1500, 4000))
    f = Filled(wl, "fp4")
    q = syn.queries(wl).cuda()
    ref = f.decode_shared(q, flags=kvq.splits_flag(1)).cpu().numpy()
    _check_all(f, q, ref, "shared one split")
    for s in (2, 5, 32, 40):
        got = f.decode_shared(q, flags=kvq.splits_flag(s)).cpu().numpy()
        np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)


def test_shared_prefix_rotation_flags(gpu):
    """KVQ_Q_PREROTATED / KVQ_OUT_ROTATED act as in plain decode."""
    wl = _mix("shared_flags", batch=4, hkv=2, group=4, n_q=2, ctx=(300, 1200))
    f = Filled(wl, "fp4")
    q = syn.queries(wl).cuda()
    for flags in (kvq.OUT_ROTATED, kvq.Q_PREROTATED, kvq.Q_PREROTATED | kvq.OUT_ROTATED):
        got = f.decode_shared(q, flags=flags).cpu().numpy()
        plain = f.decode(q, flags=flags).cpu().numpy()
        np.testing.assert_allclose(got, plain, rtol=RTOL, atol=ATOL)
