"""The binding's event marshalling (CPU): torch creates a torch.cuda.Event's
HIP handle only at its first record(), so an event handed to the library
before that would be read as "no event".  The binding records a done-event
on its copy stream first (so the handle exists and the library's own record
after the copies is the one waiters see), and refuses a pending-ready event
that was never recorded.  Stub events stand in for torch's here."""
import pytest

import quantized_expert_ffn_amd as qm


class StubEvent:
    def __init__(self, handle=0):
        self.cuda_event = handle
        self.recorded_on = []

    def record(self, stream=None):
        self.recorded_on.append(stream)
        if not self.cuda_event:
            self.cuda_event = 0xE7E7


def test_done_event_is_created_before_the_call():
    ev = StubEvent()
    stream = object()
    h = qm._event_handle(ev, "done_event", create_on=stream)
    assert h == 0xE7E7 and ev.recorded_on == [stream]


def test_existing_event_is_passed_as_is():
    ev = StubEvent(0x1234)
    assert qm._event_handle(ev, "done_event", create_on=object()) == 0x1234
    assert ev.recorded_on == []
    assert qm._event_handle(ev, "pending_ready") == 0x1234


def test_never_recorded_pending_event_is_refused():
    with pytest.raises(ValueError, match="never been recorded"):
        qm._event_handle(StubEvent(), "pending_ready")


def test_raw_handles_and_none_pass_through():
    assert qm._event_handle(None, "x") is None
    assert qm._event_handle(0xABC, "x") == 0xABC
