"""The kernel timing hook (lbsa_time_next_kernel): the next launch stamps the
armed events at its own start and end, the hook is used once, and a stamped
launch computes exactly what a plain one does."""
import pytest
import torch

import _gpu_helpers as H
from _gpu_helpers import requires_gpu
from load_balanced_split_assign_amd import lbsa

pytestmark = [pytest.mark.gpu, requires_gpu]


def test_stamped_split_and_combine_match_plain_launches():
    batch = H.batch_on_gpu("tp8_share")
    P = H.workgroups(batch)
    tm = H.plan(batch, P)
    ref = H.decode(batch, tm, P).clone()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in ev:
        e.record(stream)            # creates the events
    torch.cuda.synchronize()

    ev[0].record(stream)
    lbsa.time_next_kernel(ev[1], ev[2])
    ws = H.decode_split(batch, tm, P)
    lbsa.time_next_kernel(ev[3], ev[4])
    out = lbsa.decode_combine(batch["B"], batch["num_heads"], batch["num_kv_heads"], P, tm, ws)
    ev[5].record(stream)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))

    split_ms, comb_ms = ev[1].elapsed_time(ev[2]), ev[3].elapsed_time(ev[4])
    total_ms = ev[0].elapsed_time(ev[5])
    print(f"split {1000 * split_ms:.2f} us, combine {1000 * comb_ms:.2f} us, both with markers "
          f"{1000 * total_ms:.2f} us", flush=True)
    assert 0.0 < split_ms and 0.0 < comb_ms
    assert split_ms + comb_ms <= total_ms
    assert ev[0].elapsed_time(ev[1]) >= 0.0     # stamps in launch order
    assert ev[2].elapsed_time(ev[3]) >= 0.0
    assert ev[4].elapsed_time(ev[5]) >= 0.0

    # the hook was used once: later plain launches leave the stamps alone
    again = H.decode(batch, tm, P)
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), ref.view(torch.int16))
    assert ev[1].elapsed_time(ev[2]) == split_ms
    assert ev[3].elapsed_time(ev[4]) == comb_ms


def test_rejected_call_disarms_the_hook():
    """An entry point that rejects its arguments launches nothing and disarms
    the hook: the next, valid launch does not stamp the events."""
    batch = H.batch_on_gpu("tp8_share")
    P = H.workgroups(batch)
    tm = H.plan(batch, P)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    for e in ev:
        e.record(stream)
    torch.cuda.synchronize()
    before = ev[0].elapsed_time(ev[1])
    lbsa.time_next_kernel(ev[0], ev[1])
    with pytest.raises(lbsa.LbsaError):
        H.decode_split(batch, tm, P, workspace=torch.empty(16, dtype=torch.uint8, device="cuda:0"))
    H.decode_split(batch, tm, P)
    torch.cuda.synchronize()
    assert ev[0].elapsed_time(ev[1]) == before       # the split launch left the events alone


def test_one_call_stamps_split_and_combine():
    """lbsa_decode launches two kernels; two armed pairs stamp one each, in order."""
    batch = H.batch_on_gpu("tp8_share")
    P = H.workgroups(batch)
    tm = H.plan(batch, P)
    ref = H.decode(batch, tm, P).clone()
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in ev:
        e.record(stream)
    torch.cuda.synchronize()
    lbsa.time_next_kernels([(ev[0], ev[1]), (ev[2], ev[3])])
    out = H.decode(batch, tm, P)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    split_ms, comb_ms = ev[0].elapsed_time(ev[1]), ev[2].elapsed_time(ev[3])
    print(f"split {1000 * split_ms:.2f} us, combine {1000 * comb_ms:.2f} us", flush=True)
    assert split_ms > 0.005 and comb_ms > 0.0
    assert ev[1].elapsed_time(ev[2]) >= 0.0          # the combine starts after the split ends
