"""CPU: the adapter cache's policy ("Add multi-LoRA support", Features: Disk ->
CPU (LRU) -> GPU (fixed number of slots)).  The stacked slot tensors live in
host memory here and a plain torch stand-in places each matrix; the GPU test
(tests/test_slots_gpu.py) runs the library's lora_copy_padded and the kernels
on the cache."""

import pytest
import torch

from gemm_lora_shrink_amd.slots import HostAdapter, SlotCache

LAYERS = {"q": (16, (8,)), "gate_up": (16, (12, 12))}
V, H = 10, 8


def place(src, dst, transpose):
    m = src.t() if transpose else src
    dst.zero_()
    dst[:m.shape[0], :m.shape[1]] = m


def make_adapter(name, rank):
    g = torch.Generator().manual_seed(hash(name) % 1000)
    layers = {ln: [(torch.randn(rank, D, generator=g), torch.randn(o, rank, generator=g)) for o in outs]
              for ln, (D, outs) in LAYERS.items()}
    return HostAdapter(name=name, rank=rank, scale=2.0 / rank, layers=layers,
                       embedding=(torch.randn(rank, V, generator=g), torch.randn(H, rank, generator=g)))


RANKS = {"a": 4, "b": 8, "c": 2, "d": 6, "e": 8}


def cache(n_slots=2, cpu_capacity=8):
    loads = []

    def loader(name):
        loads.append(name)
        return make_adapter(name, RANKS[name])
    c = SlotCache(LAYERS, n_slots, 8, torch.float32, "cpu", cpu_capacity=cpu_capacity, loader=loader,
                  embedding=(V, H), copy_fn=place)
    return c, loads


def test_lru_eviction_among_slots_the_batch_does_not_use():
    c, _ = cache()
    c.slots_for(["a"])
    c.slots_for(["b"])
    c.slots_for(["a", None])                 # touches a: b is now least recent
    c.slots_for(["c"])                       # evicts b
    assert set(c.resident()) == {"a", "c"}
    c.slots_for(["c", "d"])                  # a is least recent and unused: evicted
    assert set(c.resident()) == {"c", "d"}
    c.slots_for(["c", "a"])                  # d is evicted, never c (the batch uses it)
    assert set(c.resident()) == {"c", "a"}
    assert c.stats.gpu_evictions == 3 and c.stats.gpu_loads == 5


def test_index_vector_and_base_tokens():
    c, _ = cache(n_slots=3)
    idx = c.slots_for(["b", None, "a", "b", None])
    res = c.resident()
    assert idx.dtype == torch.int32
    assert idx.tolist() == [res["b"], -1, res["a"], res["b"], -1]
    assert c.slots_for([None, None]).tolist() == [-1, -1]


def test_too_many_adapters_for_the_slots():
    c, _ = cache(n_slots=2)
    with pytest.raises(ValueError):
        c.slots_for(["a", "b", "c"])


def test_cpu_tier_is_lru_and_backed_by_the_loader():
    c, loads = cache(n_slots=1, cpu_capacity=2)
    for n in ["a", "b", "a", "c", "b", "a"]:
        c.slots_for([n])
    # CPU tier after each step: [a], [a b], [b a] (a a CPU hit), [a c] (b out),
    # [c b] (a out; b from disk again), [b a] (c out; a from disk again)
    assert loads == ["a", "b", "c", "b", "a"]
    assert c.cpu_resident() == ["b", "a"]
    assert c.stats.cpu_hits == 1 and c.stats.cpu_evictions == 3


def test_slot_contents_are_zero_padded_and_never_stale():
    c, _ = cache(n_slots=1)
    c.slots_for(["b"])                       # rank 8 fills the whole slot
    c.slots_for(["c"])                       # rank 2 reuses it
    ad = make_adapter("c", 2)
    s = c.resident()["c"]
    for ln, (D, outs) in LAYERS.items():
        for i in range(len(outs)):
            A, B = ad.layers[ln][i]
            assert torch.equal(c.A[ln][i][s, :2], A) and not torch.any(c.A[ln][i][s, 2:])
            assert torch.equal(c.B[ln][i][s, :, :2], B) and not torch.any(c.B[ln][i][s, :, 2:])
    Ae, Be = ad.embedding
    assert torch.equal(c.A_emb[s, :, :2], Ae.t()) and not torch.any(c.A_emb[s, :, 2:])
    assert torch.equal(c.B_emb[s, :, :2], Be) and not torch.any(c.B_emb[s, :, 2:])
    assert int(c.ranks[s]) == 2 and float(c.scale[s]) == pytest.approx(1.0)


def test_rank_above_the_slots_is_refused():
    def loader(name):
        return make_adapter(name, 16)
    c = SlotCache(LAYERS, 2, 8, torch.float32, "cpu", cpu_capacity=2, loader=loader, copy_fn=place)
    with pytest.raises(ValueError):
        c.slots_for(["x"])
