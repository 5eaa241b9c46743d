"""Adapter slots: the tiered adapter cache of "Add multi-LoRA support".

That page's Features describe adapters kept in a Disk (unlimited) -> CPU (LRU)
-> GPU (fixed number of slots) cache, adapters of different ranks in one
batch, adapters on every linear layer and on the embeddings, and a batch that
mixes adapter and base-only requests; its Limitations note that the slots are
preallocated (not shared with the KV cache) and that all adapters share one
dtype.  This module is that cache on the host side of the library:

* GPU tier: `n_slots` slots of preallocated stacked tensors, one per LoRA
  layer and output slice (A_i [S][r_max][D], B_i [S][out_i][r_max]), an
  optional embedding pair (A_emb [S][V][r_max], B_emb [S][H][r_max]), and the
  per-slot `ranks` (int32) and `scale` (fp32) the kernels read.  Loading an
  adapter into a slot copies each of its matrices into the slot region with
  zeros past its rank (lora_copy_padded), so a slot never shows values of its
  previous adapter.  Eviction is least-recently-used among the slots the
  batch being prepared does not use.
* CPU tier: up to `cpu_capacity` adapters in pinned host memory, least
  recently used first out.
* Disk tier: the `loader` callable (name -> HostAdapter), standing in for
  reading a PEFT checkpoint; it is called only on a CPU-tier miss.

`slots_for(names)` maps a batch's per-token adapter names (None for base-only
tokens) to the int32 slot index vector the kernels take, loading what is not
resident.  All copies are enqueued on the caller's current stream, after the
work already there, so a slot is never rewritten under a kernel of an earlier
batch on that stream.  A batch may use at most `n_slots` distinct adapters
(the caller's scheduler splits larger ones).
"""

from collections import OrderedDict
from dataclasses import dataclass, field
from typing import Callable, Dict, Hashable, List, Optional, Sequence, Tuple

import torch


@dataclass
class HostAdapter:
    """One adapter in PEFT layout: per LoRA layer, per output slice, an A of
    [rank][D] and a B of [out_i][rank]; optionally an embedding pair
    (A of [rank][V], B of [H][rank]); and its scale (alpha / rank)."""

    name: Hashable
    rank: int
    scale: float
    layers: Dict[str, List[Tuple[torch.Tensor, torch.Tensor]]]
    embedding: Optional[Tuple[torch.Tensor, torch.Tensor]] = None


def _library_copy(src, dst, transpose):
    from . import copy_padded
    copy_padded(src, dst, transpose=transpose)


@dataclass
class CacheStats:
    gpu_hits: int = 0
    gpu_loads: int = 0
    gpu_evictions: int = 0
    cpu_hits: int = 0
    disk_loads: int = 0
    cpu_evictions: int = 0


class SlotCache:
    """Fixed GPU slots of stacked adapter tensors with LRU host and GPU tiers.

    layers: {layer name: (D, (out_0, out_1, ...))}; embedding: (V, H) or None.
    copy_fn(src, dst, transpose): places a device matrix into a slot region
    with zero padding; the library's lora_copy_padded by default.
    """

    def __init__(self, layers, n_slots, r_max, dtype, device, *, cpu_capacity, loader,
                 embedding=None, copy_fn: Optional[Callable] = None):
        if n_slots < 1 or cpu_capacity < 1:
            raise ValueError("need at least one GPU slot and one CPU entry")
        self.layers = dict(layers)
        self.n_slots, self.r_max, self.dtype = n_slots, r_max, dtype
        self.device = torch.device(device)
        self.cpu_capacity = cpu_capacity
        self.loader = loader
        self.copy_fn = copy_fn or _library_copy
        z = dict(dtype=dtype, device=self.device)
        self.A = {n: [torch.zeros((n_slots, r_max, D), **z) for _ in outs] for n, (D, outs) in self.layers.items()}
        self.B = {n: [torch.zeros((n_slots, o, r_max), **z) for o in outs] for n, (D, outs) in self.layers.items()}
        self.A_emb = self.B_emb = None
        if embedding is not None:
            V, H = embedding
            self.A_emb = torch.zeros((n_slots, V, r_max), **z)
            self.B_emb = torch.zeros((n_slots, H, r_max), **z)
        self.ranks = torch.zeros(n_slots, dtype=torch.int32, device=self.device)
        self.scale = torch.zeros(n_slots, dtype=torch.float32, device=self.device)
        self._resident: "OrderedDict[Hashable, int]" = OrderedDict()  # least recent first
        self._free: List[int] = list(range(n_slots - 1, -1, -1))
        self._cpu: "OrderedDict[Hashable, HostAdapter]" = OrderedDict()
        self.stats = CacheStats()

    # ---- tiers -----------------------------------------------------------
    def resident(self):
        """{adapter name: slot} of the GPU tier, least recently used first."""
        return OrderedDict(self._resident)

    def cpu_resident(self):
        return list(self._cpu)

    def _host(self, name) -> HostAdapter:
        if name in self._cpu:
            self._cpu.move_to_end(name)
            self.stats.cpu_hits += 1
            return self._cpu[name]
        a = self.loader(name)
        self.stats.disk_loads += 1
        if a.rank < 1 or a.rank > self.r_max:
            raise ValueError(f"adapter {name!r} has rank {a.rank}, the slots hold 1..{self.r_max}")
        pin = self.device.type == "cuda"

        def host(t):
            t = t.detach().to("cpu", dtype=self.dtype).contiguous()
            return t.pin_memory() if pin else t
        layers = {}
        for lname, (D, outs) in self.layers.items():
            mats = a.layers[lname]
            if len(mats) != len(outs):
                raise ValueError(f"adapter {name!r}: layer {lname} needs {len(outs)} slices")
            for (Am, Bm), o in zip(mats, outs):
                if tuple(Am.shape) != (a.rank, D) or tuple(Bm.shape) != (o, a.rank):
                    raise ValueError(f"adapter {name!r}: layer {lname} has wrong shapes")
            layers[lname] = [(host(Am), host(Bm)) for Am, Bm in mats]
        emb = None
        if self.A_emb is not None:
            Ae, Be = a.embedding
            emb = (host(Ae), host(Be))
        h = HostAdapter(name=name, rank=a.rank, scale=float(a.scale), layers=layers, embedding=emb)
        self._cpu[name] = h
        while len(self._cpu) > self.cpu_capacity:
            self._cpu.popitem(last=False)
            self.stats.cpu_evictions += 1
        return h

    def _load(self, name, slot):
        h = self._host(name)
        dev = self.device
        for lname in self.layers:
            for i, (Am, Bm) in enumerate(h.layers[lname]):
                self.copy_fn(Am.to(dev, non_blocking=True), self.A[lname][i][slot], False)
                self.copy_fn(Bm.to(dev, non_blocking=True), self.B[lname][i][slot], False)
        if self.A_emb is not None:
            Ae, Be = h.embedding
            self.copy_fn(Ae.to(dev, non_blocking=True), self.A_emb[slot], True)  # PEFT [r][V] -> [V][r_max]
            self.copy_fn(Be.to(dev, non_blocking=True), self.B_emb[slot], False)
        self.ranks[slot] = h.rank
        self.scale[slot] = h.scale
        self._resident[name] = slot
        self.stats.gpu_loads += 1

    # ---- batches ---------------------------------------------------------
    def slots_for(self, names: Sequence[Optional[Hashable]]) -> torch.Tensor:
        """The int32 slot index of every token (-1 for None), after loading
        every adapter of the batch that is not resident."""
        distinct = list(OrderedDict.fromkeys(n for n in names if n is not None))
        if len(distinct) > self.n_slots:
            raise ValueError(f"the batch uses {len(distinct)} adapters, the cache has {self.n_slots} slots")
        wanted = set(distinct)
        for n in distinct:
            if n in self._resident:
                self._resident.move_to_end(n)
                self.stats.gpu_hits += 1
        for n in distinct:
            if n in self._resident:
                continue
            if self._free:
                slot = self._free.pop()
            else:
                victim = next(k for k in self._resident if k not in wanted)
                slot = self._resident.pop(victim)
                self.stats.gpu_evictions += 1
            self._load(n, slot)
        idx = torch.tensor([self._resident[n] if n is not None else -1 for n in names], dtype=torch.int32)
        return idx.to(self.device, non_blocking=False)
