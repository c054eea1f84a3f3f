"""GPU checks of bi_set_launch_events (timing events on the library's own kernels).

With events set, the entry points give the same bits, the elapsed time runs
from the first kernel's start to the last kernel's end (no longer than events
recorded around the calls), a call that launches nothing leaves the events
alone, and clearing the setting stops the kernels from recording them.
"""
import pytest
import torch

import synth
from helpers import bitwise_equal

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from invariant_persistent_bf16_amd import bi
DEV = "cuda"


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    torch.cuda.synchronize()
    return evs


def _conv_case():
    x = synth.randn((4, 3, 224, 224), seed=71, dtype=torch.bfloat16).to(DEV)
    w = synth.randn((1152, 3, 14, 14), seed=72, dtype=torch.bfloat16, scale=0.05).to(DEV)
    b = synth.randn((1152,), seed=73, dtype=torch.bfloat16).to(DEV)
    return lambda: bi.bi_conv2d(x, w, b, stride=(14, 14))


def _attention_case():
    G, T, D = 6, 256, 64
    Q = synth.randn((G, T, D), seed=74, dtype=torch.bfloat16).to(DEV)
    K = synth.randn((G, T, D), seed=75, dtype=torch.bfloat16).to(DEV)
    V = synth.randn((G, T, D), seed=76, dtype=torch.bfloat16).to(DEV)

    def run():
        P = bi.bi_attention_probs(Q, K, 0.125)
        return bi.bi_bmm(P, V, out_dtype=bi.BI_F32)
    return run


@pytest.mark.parametrize("case", ["conv2d", "attention", "mm_fp32"])
def test_launch_events_time_the_kernels(case):
    if case == "conv2d":
        op = _conv_case()
    elif case == "attention":
        op = _attention_case()
    else:
        A = synth.randn((200, 4096), seed=77, dtype=torch.float32).to(DEV)
        B = synth.randn((4096, 256), seed=78, dtype=torch.float32).to(DEV)
        op = lambda: bi.bi_mm(A, B)
    ref = op()
    k0, k1, o0, o1 = _events(4)
    o0.record()
    bi.bi_set_launch_events(k0, k1)
    try:
        got = op()
    finally:
        bi.bi_set_launch_events(None, None)
    o1.record()
    torch.cuda.synchronize()
    assert bitwise_equal(got, ref), f"{case}: bits differ with launch events set"
    t_kernels, t_call = k0.elapsed_time(k1), o0.elapsed_time(o1)
    print(f"{case}: kernels {t_kernels * 1e3:.1f} us, around the calls {t_call * 1e3:.1f} us", flush=True)
    assert 0.0 < t_kernels <= t_call

    # cleared: a further call records neither event
    op()
    torch.cuda.synchronize()
    assert k0.elapsed_time(k1) == t_kernels


def test_launch_events_untouched_by_calls_that_launch_nothing():
    A = synth.randn((64, 128), seed=79, dtype=torch.bfloat16).to(DEV)
    B = synth.randn((128, 96), seed=80, dtype=torch.bfloat16).to(DEV)
    k0, k1 = _events(2)
    bi.bi_set_launch_events(k0, k1)
    try:
        bi.bi_mm(A, B)                                   # records both
        torch.cuda.synchronize()
        t = k0.elapsed_time(k1)
        bi.bi_mm(A[:0], B)                               # M = 0: no kernel
        C = torch.empty(64, 96, dtype=torch.bfloat16, device=DEV)
        rc = bi.lib().bi_mm(64, 96, 128, None, 128, 1, B.data_ptr(), 96, 1, C.data_ptr(), 96, 1,
                            bi.BI_BF16, bi.BI_BF16, None)
        assert rc < 0                                    # A is NULL: an error, no kernel
        torch.cuda.synchronize()
        assert k0.elapsed_time(k1) == t
    finally:
        bi.bi_set_launch_events(None, None)
    with pytest.raises(ValueError):
        bi.bi_set_launch_events(torch.cuda.Event(enable_timing=True), k1)
