"""The product path fails loudly when the HIP library is missing: every entry
point of the binding raises before doing anything, and nothing falls back to
a CPU or PyTorch implementation (CPU only)."""

import pytest
import torch

import exact_tiled_attention_flashattention_amd as eta


@pytest.fixture
def no_library(monkeypatch):
    monkeypatch.setattr(eta, "LIB_PATH", "/nonexistent/libattn.so")
    monkeypatch.setattr(eta, "_lib", None)


def test_every_entry_point_raises_without_the_library(no_library):
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    lse = torch.zeros(1, 2, 4)
    sl = torch.ones(1, dtype=torch.int32)
    qd = torch.zeros(1, 1, 2, 64, dtype=torch.bfloat16)
    cache = torch.zeros(1, 16, 1, 64, dtype=torch.bfloat16)
    calls = [
        lambda: eta.library(),
        lambda: eta.attn_prefill(q, k, k),
        lambda: eta.attn_prefill_backward(q, k, k, q, lse, q),
        lambda: eta.attn_prefill_paged(qd, cache, cache, sl),
        lambda: eta.attn_decode_paged(qd, cache, cache, sl),
        lambda: eta.attn_decode_paged_fp8(qd, cache, cache, lse, lse, sl),
        lambda: eta.kv_append(qd, qd, cache, cache, sl),
        lambda: eta.kv_append_fp8(qd, qd, cache, cache, lse, lse, sl),
        lambda: eta.attn_gather_paged(cache, sl),
        lambda: eta.attn_decode_workspace_bytes(1, 2, 1, 1, 64, 16),
        lambda: eta.attn_decode_paged_noalloc(qd, cache, cache, sl),
        lambda: eta.attn_prefill_workgroup_waves(1, 2, 1, 4, True),
        lambda: eta.BlockPool(4),
    ]
    for call in calls:
        with pytest.raises(RuntimeError, match="missing"):
            call()
