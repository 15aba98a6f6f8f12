"""CPU checks of the Python binding's host logic: which parameters the
routing helper sends to Muon, and the stream bookkeeping of the functional
wrappers (no GPU and no library call is needed for either)."""

import pytest
import torch

from matrix_aware_optimizer_step_amd import muon as mu


def p2():
    return torch.zeros(4, 4)


@pytest.mark.parametrize("name", [
    # Hugging Face Llama / Mistral / Qwen
    "model.layers.0.self_attn.q_proj.weight", "model.layers.0.self_attn.o_proj.weight",
    "model.layers.31.mlp.down_proj.weight",
    # BERT-style: attention and MLP output projections are hidden matrices
    "bert.encoder.layer.0.attention.output.dense.weight", "bert.encoder.layer.3.output.dense.weight",
    "encoder.layer.0.attention.self.query.weight",
    # GPT-2 and Meta Llama
    "transformer.h.0.attn.c_attn.weight", "transformer.h.0.mlp.c_proj.weight", "layers.0.attention.wo.weight",
    "layers.0.feed_forward.w2.weight",
    # a nested module named "output" or "head" inside a block; "heads" and
    # "header" only contain the substrings
    "decoder.layers.2.mlp.output.weight", "blocks.0.attn.head.weight", "layers.0.attn.heads.weight",
    "model.header_proj.weight", "model.outputs_proj.weight",
])
def test_hidden_matrices_go_to_muon(name):
    assert mu.is_muon_param(name, p2()), name


@pytest.mark.parametrize("name", [
    "model.embed_tokens.weight", "lm_head.weight", "transformer.wte.weight", "transformer.wpe.weight",
    "tok_embeddings.weight", "output.weight", "head.weight", "classifier.weight", "score.weight",
    "bert.embeddings.word_embeddings.weight", "bert.embeddings.position_embeddings.weight",
    "model.decoder.embed_positions.weight", "Model.LM_Head.weight",
])
def test_embeddings_and_heads_go_to_adamw(name):
    assert not mu.is_muon_param(name, p2()), name


def test_non_matrices_go_to_adamw():
    assert not mu.is_muon_param("model.layers.0.input_layernorm.weight", torch.zeros(4))
    assert not mu.is_muon_param("model.layers.0.self_attn.q_proj.bias", torch.zeros(4))
    assert not mu.is_muon_param("conv.weight", torch.zeros(2, 2, 3, 3))


def test_custom_module_sets():
    assert not mu.is_muon_param("blocks.0.router.weight", p2(), embedding_or_head_modules={"router"})
    assert mu.is_muon_param("lm_head.weight", p2(), embedding_or_head_modules=set(), top_level_head_modules=set())


class FakeTensor:
    def __init__(self, is_cuda=True):
        self.is_cuda = is_cuda
        self.recorded = []

    def record_stream(self, s):
        self.recorded.append(s)


def test_record_on_records_the_launch_stream():
    s = object()
    a, b, host = FakeTensor(), FakeTensor(), FakeTensor(is_cuda=False)
    mu._record_on(s, [a, None, b, host])
    assert a.recorded == [s] and b.recorded == [s] and host.recorded == []
    # the current stream (None) needs no bookkeeping
    c = FakeTensor()
    mu._record_on(None, [c])
    assert c.recorded == []


def test_stream_object_passes_stream_objects_through():
    class S:
        cuda_stream = 1234
    s = S()
    assert mu._stream_object(None) is None
    assert mu._stream_object(s) is s


def test_owned_collects_pointer_arrays_only():
    x = [torch.zeros(3, 5), torch.zeros(3, 5)]
    b_list = mu.batch(x)
    b_one = mu.batch(torch.zeros(3, 5))
    assert len(b_list.owned) == 1 and b_list.owned[0] is b_list.keep[0]
    assert b_list.owned[0].dtype == torch.int64 and b_list.owned[0].numel() == 2
    assert b_one.owned == []
    assert mu._owned([b_list, None, b_one]) == b_list.owned


def test_wrappers_record_what_they_allocate(monkeypatch):
    """momentum() with no workspace and a side stream: the workspace it
    allocated and the pointer array of a list input are recorded on that
    stream after the (stubbed) library call."""
    made = []

    def fake_workspace(nbytes, device):
        t = FakeTensor()
        t.data_ptr = lambda: 0
        t.numel = lambda: 256
        made.append(t)
        return t

    calls = []
    monkeypatch.setattr(mu, "workspace", fake_workspace)
    monkeypatch.setattr(mu.L, "muon_momentum_workspace", lambda *a: 256)
    monkeypatch.setattr(mu.L, "muon_momentum", lambda *a: calls.append(a))
    recorded = []
    monkeypatch.setattr(mu, "_record_on", lambda s, ts: recorded.append((s, list(ts))))
    side = object()
    monkeypatch.setattr(mu, "_stream_object", lambda s: side if s is not None else None)
    monkeypatch.setattr(mu, "_stream", lambda s: 0)
    grads = [torch.zeros(3, 5), torch.zeros(3, 5)]
    mom = torch.zeros(2, 3, 5)
    mu.momentum(grads, mom, None, torch.zeros(2), stream=7)
    assert len(calls) == 1
    (s, ts), = recorded
    assert s is side
    assert made[0] in ts
    assert any(isinstance(t, torch.Tensor) and t.dtype == torch.int64 for t in ts)  # the pointer array
    # a caller-provided workspace is the caller's to keep alive
    recorded.clear()
    mine = fake_workspace(256, None)
    mu.momentum(grads, mom, None, torch.zeros(2), ws=mine, stream=7)
    (s, ts), = recorded
    assert mine not in ts
