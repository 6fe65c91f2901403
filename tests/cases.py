"""Test-case assembly shared by the oracle pins and the GPU parity tests.

Builds, from the seeded generators in ``workloads``, the fp32 sources of a
workload and the oracle's own quantised host cache of them.  Nothing here
computes any part of the method: quantisation is the oracle's (host side) or
the library's (GPU side).
"""
from dataclasses import dataclass

import numpy as np

import oracle
import workloads

POISON_INT8 = 127


@dataclass
class Case:
    w: workloads.Workload
    q: np.ndarray             # fp32 [batch][n_q][hd]
    lens: np.ndarray          # int32 [batch]
    table: np.ndarray         # int32 [batch][max_blocks]
    num_blocks: int
    scale: float
    k_src: list               # per sequence fp32 [L][n_kv][hd]
    v_src: list
    slots: list               # per sequence int32 [L]
    cache: oracle.Cache = None


def build(w, lens=None, poison=True, with_cache=True):
    """Draw a workload's inputs; optionally quantise them into a host cache
    with the oracle.  Unreferenced rows/blocks hold int8 127 and NaN scales
    when ``poison`` (a stray read then shows up as NaN)."""
    if lens is None:
        lens = workloads.seq_lens(w)
    lens = np.asarray(lens, np.int32)
    table, nb = workloads.block_table(w, lens)
    q = workloads.query(w)
    k_src, v_src, slots = [], [], []
    for b in range(w.batch):
        L = max(int(lens[b]), 0)
        k, v = workloads.kv_rows(w, b, L)
        k_src.append(k)
        v_src.append(v)
        slots.append(workloads.slot_mapping(w, table, b, L))
    c = Case(w, q, lens, table, nb, workloads.softmax_scale(w.hd), k_src, v_src, slots)
    if with_cache:
        c.cache = host_cache(c, poison)
    return c


def host_cache(c, poison=True):
    w = c.w
    cache = oracle.Cache(c.num_blocks, w.n_kv, w.kv_bs, w.hd,
                         fill_int8=POISON_INT8 if poison else 0,
                         fill_scale=np.nan if poison else 0.0)
    for b in range(w.batch):
        if len(c.slots[b]):
            cache.append(c.k_src[b], c.v_src[b], c.slots[b])
    return cache


def small(name, **kw):
    """A scaled-down copy of a named workload (same recipe, own seed key)."""
    base = workloads.WORKLOADS[name]
    kw.setdefault("key", base.key + 100)
    return base.scaled(**kw)
