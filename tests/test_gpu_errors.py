"""Argument checks of the C ABI on a device: every rejected call returns
AR_ERR_INVALID_ARGUMENT with a message and leaves the buffers untouched."""
import pytest
import torch

import gpu_util as gu
import ring_all_reduce_ar_amd as ar

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def comm():
    c = ar.Comm(4, 0)
    yield c
    c.close()


def bufs(n=4, count=64, dtype="f32"):
    return [gu.RankBuf(count, dtype, fill=0x11) for _ in range(n)]


def expect_invalid(fn, *args):
    with pytest.raises(ar.ArError) as ei:
        fn(*args)
    assert ei.value.code == ar.AR_ERR_INVALID_ARGUMENT, str(ei.value)
    assert ar.ar_last_error(), "no error detail"


def untouched(bs):
    torch.cuda.synchronize()
    return all(bool((b.raw[b.lo:b.hi] == 0x11).all()) and b.guards_ok() for b in bs)


def test_two_ranks_share_a_buffer(comm):
    s, d = bufs(), bufs()
    send = [b.ptr() for b in s]
    send[1] = send[0]
    expect_invalid(ar.ar_all_reduce, comm, send, [b.ptr() for b in d], 64, "f32", "sum", "fused", None)
    assert untouched(s + d)


def test_partial_overlap_of_send_and_recv(comm):
    s = bufs(count=128)
    d = bufs()
    recv = [b.ptr() for b in d]
    recv[2] = s[2].sub_ptr(8)  # inside rank 2's send buffer, not the in-place layout
    expect_invalid(ar.ar_all_reduce, comm, [b.sub_ptr(0) for b in s], recv, 64, "f32", "sum", "fused", None)
    assert untouched(s + d)


def test_recv_overlaps_other_rank(comm):
    s, d = bufs(), bufs()
    recv = [b.ptr() for b in d]
    recv[3] = s[0].ptr()
    expect_invalid(ar.ar_all_reduce, comm, [b.ptr() for b in s], recv, 64, "f32", "sum", "stepwise", None)
    assert untouched(s + d)


def test_stepwise_half_needs_workspace(comm):
    s = bufs(dtype="f16")
    ar.ar_comm_set_workspace(comm, None)
    expect_invalid(ar.ar_all_reduce, comm, [b.ptr() for b in s], [b.ptr() for b in s], 64, "f16", "sum",
                   "stepwise", None)
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    ar.ar_comm_set_workspace(comm, small)
    expect_invalid(ar.ar_all_reduce, comm, [b.ptr() for b in s], [b.ptr() for b in s], 64, "f16", "sum",
                   "stepwise", None)
    ar.ar_comm_set_workspace(comm, None)
    assert untouched(s)


def test_workspace_overlapping_a_buffer(comm):
    s = bufs(count=256, dtype="bf16")
    ar.ar_comm_set_workspace(comm, s[1].ptr(), 256 * 4)
    expect_invalid(ar.ar_all_reduce, comm, [b.ptr() for b in s], [b.ptr() for b in s], 64, "bf16", "avg",
                   "stepwise", None)
    ar.ar_comm_set_workspace(comm, None)
    assert untouched(s)


def test_reduce_scatter_needs_workspace_in_stepwise(comm):
    s = bufs(count=4 * 16)
    d = bufs(count=16)
    ar.ar_comm_set_workspace(comm, None)
    expect_invalid(ar.ar_reduce_scatter, comm, [b.ptr() for b in s], [b.ptr() for b in d], 16, "f32", "sum",
                   "stepwise", None)
    assert untouched(s + d)


def test_misaligned_element(comm):
    s, d = bufs(count=65), bufs(count=65)
    expect_invalid(ar.ar_all_reduce, comm, [b.ptr() + 1 for b in s], [b.ptr() for b in d], 64, "f32", "sum",
                   "fused", None)
    assert untouched(s + d)


def test_bad_enums_and_nulls(comm):
    s, d = bufs(), bufs()
    sp, dp = [b.ptr() for b in s], [b.ptr() for b in d]
    expect_invalid(ar.ar_all_reduce, comm, sp, dp, 64, 7, "sum", "fused", None)
    expect_invalid(ar.ar_all_reduce, comm, sp, dp, 64, "f32", 9, "fused", None)
    expect_invalid(ar.ar_all_reduce, comm, sp, dp, 64, "f32", "sum", 5, None)
    expect_invalid(ar.ar_all_reduce, comm, sp[:3] + [0], dp, 64, "f32", "sum", "fused", None)
    expect_invalid(ar.ar_all_reduce, None, sp, dp, 64, "f32", "sum", "fused", 0)
    expect_invalid(ar.ar_all_reduce, comm, sp, dp, 2**62, "f32", "sum", "fused", None)
    assert untouched(s + d)


def test_count_zero_is_a_noop(comm):
    s, d = bufs(), bufs()
    ar.ar_all_reduce(comm, [b.ptr() for b in s], [b.ptr() for b in d], 0, "f32", "sum", "fused")
    ar.ar_reduce_scatter(comm, [b.ptr() for b in s], [b.ptr() for b in d], 0, "f32", "sum", "stepwise")
    ar.ar_all_gather(comm, [b.ptr() for b in s], [b.ptr() for b in d], 0, "f32", "stepwise")
    assert untouched(s + d)


def test_comm_create_limits():
    with pytest.raises(ar.ArError):
        ar.Comm(0, 0)
    with pytest.raises(ar.ArError):
        ar.Comm(ar.MAX_RANKS + 1, 0)
    with pytest.raises(ar.ArError):
        ar.Comm(4, 1 << 20)


def test_all_to_all_rejects_in_place(comm):
    s = bufs(count=4 * 16)
    expect_invalid(ar.ar_all_to_all, comm, [b.ptr() for b in s], [b.ptr() for b in s], 16, "f32", "fused", None)
    assert untouched(s)
