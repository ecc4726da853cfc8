"""The ctypes binding rejects malformed arguments on the host, before the library is called:
tensors off the GPU, shapes that do not match q (or the state), mixed input dtypes, and wrong
dtypes for states, offsets, gate parameters and acceptance counts.  CPU only: every case here
fails in the binding's checks, so nothing reaches the library or a device."""
import pytest
import torch

from gated_delta_rule_60_amd import kda as K

B, T, H, DK, DV = 1, 8, 2, 64, 64
bf, f32 = torch.bfloat16, torch.float32


def prefill(dtype=bf, **over):
    d = dict(q=torch.zeros(B, T, H, DK, dtype=dtype), k=torch.zeros(B, T, H, DK, dtype=dtype),
             v=torch.zeros(B, T, H, DV, dtype=dtype), beta=torch.zeros(B, T, H, dtype=dtype),
             g=torch.zeros(B, T, H, DK, dtype=f32))
    d.update(over)
    return d


def decode(draft=False, **over):
    lead = (3, 2, H) if draft else (3, H)
    d = dict(q=torch.zeros(*lead, DK, dtype=bf), k=torch.zeros(*lead, DK, dtype=bf),
             v=torch.zeros(*lead, DV, dtype=bf), beta=torch.zeros(*lead, dtype=bf),
             g=torch.zeros(*lead, DK, dtype=bf), state=torch.zeros(3, H, DK, DV, dtype=f32))
    d.update(over)
    return d


def test_host_tensors_are_rejected():
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kda_chunk_fwd(**prefill())
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kda_decode_step(**decode())
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kda_gate(torch.zeros(H, DK), torch.zeros(T, H, DK, dtype=bf))


@pytest.mark.parametrize("over, what", [
    (dict(k=torch.zeros(B, T, H, DK + 1, dtype=bf)), "k"),
    (dict(v=torch.zeros(B, T + 1, H, DV, dtype=bf)), "v"),
    (dict(beta=torch.zeros(B, T, H, 1, dtype=bf)), "beta"),
    (dict(g=torch.zeros(B, T, H + 1, DK)), "g"),
    (dict(initial_state=torch.zeros(2, H, DK, DV)), "initial_state"),
    (dict(final_state=torch.zeros(B, H, DV, DK + 1)), "final_state"),
    (dict(o=torch.zeros(B, T, H, DK + 64, dtype=bf)), "o"),
])
def test_prefill_shapes(over, what):
    with pytest.raises(ValueError, match=f"{what} must have shape"):
        K.kda_chunk_fwd(**prefill(**over))


@pytest.mark.parametrize("over, what", [
    (dict(k=torch.zeros(B, T, H, DK, dtype=f32)), "share one dtype"),
    (dict(beta=torch.zeros(B, T, H, dtype=f32)), "share one dtype"),
    (dict(g=torch.zeros(B, T, H, DK, dtype=torch.float16)), "g must be one of"),
    (dict(initial_state=torch.zeros(B, H, DK, DV, dtype=bf)), "initial_state must be one of"),
    (dict(o=torch.zeros(B, T, H, DV, dtype=torch.float64)), "o must be one of"),
    (dict(cu_seqlens=torch.tensor([0, 8], dtype=torch.int64)), "cu_seqlens must be one of"),
])
def test_prefill_dtypes(over, what):
    with pytest.raises(ValueError, match=what):
        K.kda_chunk_fwd(**prefill(**over))


def test_packed_batch_needs_b1_and_offsets():
    d = prefill(q=torch.zeros(2, T, H, DK, dtype=bf), k=torch.zeros(2, T, H, DK, dtype=bf),
                v=torch.zeros(2, T, H, DV, dtype=bf), beta=torch.zeros(2, T, H, dtype=bf),
                g=torch.zeros(2, T, H, DK))
    with pytest.raises(ValueError, match="B == 1"):
        K.kda_chunk_fwd(**d, cu_seqlens=torch.tensor([0, 4, 8], dtype=torch.int32))
    with pytest.raises(ValueError, match="two offsets"):
        K.kda_chunk_fwd(**prefill(), cu_seqlens=torch.tensor([0], dtype=torch.int32))
    # the state's leading size follows the number of sequences in cu_seqlens
    with pytest.raises(ValueError, match="initial_state must have shape"):
        K.kda_chunk_fwd(**prefill(), cu_seqlens=torch.tensor([0, 3, 8], dtype=torch.int32),
                        initial_state=torch.zeros(1, H, DK, DV))


def test_gated_and_checkpointed_gate_parameters():
    d = prefill()
    z = d.pop("g").to(bf)
    with pytest.raises(ValueError, match="A must have shape"):
        K.kda_chunk_fwd_gated(**d, A=torch.zeros(H, DK + 1), z=z)
    with pytest.raises(ValueError, match="A must be one of"):
        K.kda_chunk_fwd_gated(**d, A=torch.zeros(H, DK, dtype=torch.float64), z=z)
    with pytest.raises(ValueError, match="z must have shape"):
        K.kda_chunk_fwd_gated(**d, A=torch.zeros(H, DK), z=z[:, :4])
    with pytest.raises(ValueError, match="checkpoints must have shape"):
        K.kda_chunk_fwd_checkpointed(**d, every=64, A=torch.zeros(H, DK), z=z,
                                     checkpoints=torch.zeros(1, H, DK, DV + 1))
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kda_chunk_fwd_checkpointed(**d, every=64, A=torch.zeros(H, DK), z=z)


def test_gate_shapes():
    with pytest.raises(ValueError, match="A must be one of"):
        K.kda_gate(torch.zeros(H, DK, dtype=bf), torch.zeros(T, H, DK, dtype=bf))
    with pytest.raises(ValueError, match="z must have shape"):
        K.kda_gate(torch.zeros(H, DK), torch.zeros(T, H + 1, DK, dtype=bf))
    with pytest.raises(ValueError, match="g must have shape"):
        K.kda_gate(torch.zeros(H, DK), torch.zeros(T, H, DK, dtype=bf), g=torch.zeros(T, H, DK + 1))


@pytest.mark.parametrize("over, what", [
    (dict(k=torch.zeros(3, H, DK + 1, dtype=bf)), "k must have shape"),
    (dict(v=torch.zeros(3, H, DV, dtype=f32)), "share one dtype"),
    (dict(beta=torch.zeros(3, H, 1, dtype=bf)), "beta must have shape"),
    (dict(state=torch.zeros(3, H, DK, DV, dtype=bf)), "state must be one of"),
    (dict(state=torch.zeros(2, H, DK, DV)), "state must have shape"),
    (dict(g=torch.zeros(3, H, DK, dtype=torch.float16)), "g must be one of"),
])
def test_decode_checks(over, what):
    with pytest.raises(ValueError, match=what):
        K.kda_decode_step(**decode(**over))


def test_draft_checks():
    with pytest.raises(ValueError, match="q must be a"):
        K.kda_decode_verify(**decode())                      # per-token shapes, not a draft
    with pytest.raises(ValueError, match="o must have shape"):
        K.kda_decode_verify(**decode(draft=True), o=torch.zeros(3, 2, H, DV + 1, dtype=bf))
    with pytest.raises(TypeError, match="accepted must be an int32"):
        K.kda_decode_commit(**decode(draft=True), accepted=torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="accepted must have shape"):
        K.kda_decode_commit(**decode(draft=True), accepted=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU tensor"):
        K.kda_decode_commit(**decode(draft=True), accepted=torch.zeros(3, dtype=torch.int32))


def test_noncontiguous_rejected():
    q = torch.zeros(B, T, H, 2 * DK, dtype=bf)[..., :DK]
    with pytest.raises(ValueError, match="contiguous"):
        K.kda_chunk_fwd(**prefill(q=q))
