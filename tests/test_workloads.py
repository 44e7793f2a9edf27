"""Host-side checks of the seeded input generator (no GPU, no attention math)."""
import torch

from exact_io_aware_07_amd import workloads as W


def test_configs_have_the_stated_shapes():
    assert (W.TINY.B, W.TINY.H, W.TINY.N, W.TINY.d, W.TINY.dtype) == (1, 1, 256, 64, "fp32")
    assert (W.BERT.B, W.BERT.H, W.BERT.N, W.BERT.d, W.BERT.dtype) == (32, 16, 512, 64, "fp16")
    assert (W.LONG.B, W.LONG.H, W.LONG.N, W.LONG.d, W.LONG.dtype) == (1, 32, 4096, 128, "bf16")
    assert (W.TRADE.B, W.TRADE.H, W.TRADE.N, W.TRADE.d) == (1, 12, 23400, 64) and W.TRADE.causal
    assert (W.GPT2.B, W.GPT2.H, W.GPT2.N, W.GPT2.d) == (8, 12, 1024, 64)
    assert W.GPT2.causal and W.GPT2.backward
    assert abs(W.LONG.scale - 128 ** -0.5) < 1e-15


def test_generation_is_deterministic_and_cast():
    w = W.TINY.with_(N=64)
    a, b = W.make_inputs(w, 0), W.make_inputs(w, 0)
    for key in ("q", "k", "v"):
        assert torch.equal(a[key], b[key]) and a[key].dtype == torch.float32
    c = W.make_inputs(w, 1)
    assert not torch.equal(a["q"], c["q"])


def test_bert_padding_lengths_are_in_range():
    w = W.BERT.with_(H=1, N=512)
    x = W.make_inputs(w, 0)
    kv = x["kv_len"]
    assert kv.dtype == torch.int32 and kv.shape == (32,)
    assert int(kv.min()) >= 128 and int(kv.max()) <= 512
    assert len(set(kv.tolist())) > 10
    assert x["q"].dtype == torch.float16 and x["do"] is None


def test_long_context_outlier_rows_are_one_percent_times_eight():
    w = W.LONG.with_(H=2)
    x = W.make_inputs(w, 0)
    rows = W.outlier_rows(w, 0)
    assert rows.shape == (1, 2, 41)
    g = torch.Generator().manual_seed(0)
    torch.randn((1, 2, 4096, 128), generator=g)
    k32 = torch.randn((1, 2, 4096, 128), generator=g)
    for h in range(2):
        idx = rows[0, h]
        assert len(set(idx.tolist())) == 41
        expect = (k32[0, h, idx] * 8).to(torch.bfloat16)
        assert torch.equal(x["k"][0, h, idx], expect)
        others = torch.ones(4096, dtype=torch.bool)
        others[idx] = False
        assert torch.equal(x["k"][0, h, others], k32[0, h, others].to(torch.bfloat16))


def test_backward_workloads_draw_grad_after_values():
    w = W.GPT2.with_(B=1, H=1, N=32)
    x = W.make_inputs(w, 0)
    g = torch.Generator().manual_seed(0)
    ref = [torch.randn((1, 1, 32, 64), generator=g) for _ in range(4)]
    assert torch.equal(x["do"], ref[3].to(torch.bfloat16))
    assert torch.equal(x["q"], ref[0].to(torch.bfloat16))
