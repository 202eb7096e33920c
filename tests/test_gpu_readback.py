"""Device-to-host readback through the library's pinned buffer (mq_read_to_host):
byte-exact round trips, the grow-on-demand buffer (a 5.6 MB read is larger
than the 4 MiB first allocation, '07 · R3', §4), the pageable arm, and the
pageable fallback with its single warning when pinning fails."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

MIB = 1 << 20


@pytest.fixture(scope="module")
def mq():
    import torch
    assert torch.cuda.is_available()
    from block_quantized_gemv_amd import binding
    binding.lib()
    return binding


def _bytes(seed, n):
    import torch
    g = torch.Generator().manual_seed(seed)
    host = torch.randint(0, 256, (n,), dtype=torch.uint8, generator=g)
    return host.numpy(), host.cuda()


def test_pinned_readback_grows_on_demand(mq):
    mq.mq_readback_release()
    s0 = mq.mq_readback_stats()
    assert s0["pinned_bytes"] == 0
    small_h, small_d = _bytes(11, 1000)
    assert np.array_equal(mq.mq_read_to_host(small_d), small_h)
    s1 = mq.mq_readback_stats()
    assert s1["pinned_bytes"] == 4 * MIB and s1["pinned_reads"] == s0["pinned_reads"] + 1
    big_h, big_d = _bytes(12, 5_600_000)
    assert np.array_equal(mq.mq_read_to_host(big_d), big_h)
    s2 = mq.mq_readback_stats()
    assert s2["pinned_bytes"] == 5_600_000 and s2["pinned_reads"] == s1["pinned_reads"] + 1
    # a smaller read reuses the grown buffer
    assert np.array_equal(mq.mq_read_to_host(small_d), small_h)
    assert mq.mq_readback_stats()["pinned_bytes"] == 5_600_000
    # the pageable arm returns the same bytes and does not touch the buffer
    assert np.array_equal(mq.mq_read_to_host(big_d, pageable=True), big_h)
    s3 = mq.mq_readback_stats()
    assert s3["pageable_reads"] == s2["pageable_reads"] + 1 and s3["pinned_bytes"] == 5_600_000


def test_readback_into_caller_array_and_dtype(mq):
    import torch
    g = torch.Generator().manual_seed(13)
    x = torch.randn(3, 1001, generator=g)
    out = np.full((3, 1001), np.nan, np.float32)
    r = mq.mq_read_to_host(x.cuda(), out=out)
    assert r is out and np.array_equal(out.view(np.uint32), x.numpy().view(np.uint32))
    with pytest.raises(ValueError):
        mq.mq_read_to_host(x.cuda(), out=np.empty(10, np.float32))
    # zero bytes: only waits for the stream
    assert mq.lib().mq_read_to_host(None, None, 0, 0, None) == mq.MQ_OK


def test_readback_waits_for_queued_work(mq):
    """The read is blocking: work queued on the stream before it is done when
    it copies (a long fill kernel queued just before the read)."""
    import torch
    t = torch.empty(8 * MIB, dtype=torch.float32, device="cuda")
    for v in (1.0, 2.0, 3.0):
        t.fill_(v)
        out = mq.mq_read_to_host(t)
        assert (out == v).all()


def test_pinning_failure_falls_back_and_warns_once(mq, capfd):
    mq.mq_readback_release()
    h, d = _bytes(14, 300_000)
    before = mq.mq_readback_stats()
    capfd.readouterr()
    mq.mq_test_set_fault(mq.MQ_FAULT_PINNED_ALLOC)
    try:
        for _ in range(3):
            assert np.array_equal(mq.mq_read_to_host(d), h)
    finally:
        mq.mq_test_set_fault(mq.MQ_FAULT_NONE)
    err = capfd.readouterr().err
    st = mq.mq_readback_stats()
    assert st["pageable_reads"] == before["pageable_reads"] + 3
    assert st["pinned_reads"] == before["pinned_reads"] and st["pinned_bytes"] == 0 and st["warned"]
    assert err.count("readback buffer failed") == (0 if before["warned"] else 1), err
    # with pinning possible again the next read allocates the buffer
    assert np.array_equal(mq.mq_read_to_host(d), h)
    assert mq.mq_readback_stats()["pinned_bytes"] == 4 * MIB
