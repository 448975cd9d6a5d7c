"""Test-side glue: put a seeded batch on the GPU through the C ABI and run it."""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

import paged_kv_token_amd as pk
from workloads import Batch

TORCH_DTYPES = None


def torch_dtype(dtype: str):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_device(arr: np.ndarray, dtype: str, device="cuda"):
    """Storage array (float32 / float16 / bf16 bits in uint16) -> torch tensor, bit for bit."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(device)


def to_host_storage(t, dtype: str) -> np.ndarray:
    import torch
    t = t.detach().cpu().contiguous()
    if dtype == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def poison_(t, dtype: str):
    """Fill with NaN bit patterns (so stale reads show up)."""
    t.fill_(float("nan"))
    return t


@dataclass
class GpuBatch:
    batch: Batch
    k_pool: object
    v_pool: object
    q: object
    k_new: object
    v_new: object
    new_slots: object
    block_tables: object
    context_lens: object
    cu_q_lens: object
    q_pos: Optional[object]
    desc: object
    kv_fp8: Optional[tuple] = None     # (k_scale, v_scale) when the pools hold E4M3 codes

    def make_desc(self, flags: int = 0):
        b = self.batch
        fp8 = {} if self.kv_fp8 is None else dict(kv_dtype=pk.PENSIEVE_FP8_E4M3, k_scale=self.kv_fp8[0],
                                                   v_scale=self.kv_fp8[1])
        return pk.make_desc(num_heads=b.num_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                            num_blocks=b.num_blocks, block_table_stride=b.block_table_stride,
                            dtype={"f32": 0, "f16": 1, "bf16": 2}[b.dtype], softmax_scale=b.softmax_scale,
                            context_lens_host=b.context_lens, cu_q_lens_host=b.cu_q_lens, flags=flags,
                            q_pos_host=None if self.q_pos is None else b.q_pos, **fp8)


def upload(batch: Batch, *, append_new: bool = True, poison: bool = True, pass_q_pos: Optional[bool] = None,
           chunk_tokens: int = 1 << 16, kv_fp8: Optional[tuple] = None) -> GpuBatch:
    """Pools filled through pensieve_kv_append: cached history first, then (optionally) the new rows.

    kv_fp8 = (k_scale, v_scale): E4M3 pools (uint8) filled through pensieve_kv_append_fp8;
    poison is then the NaN code 0x7F.
    """
    import torch
    b = batch
    td = torch.uint8 if kv_fp8 is not None else torch_dtype(b.dtype)
    k_pool = torch.empty((b.num_blocks, b.num_kv_heads, b.block_size, b.head_dim), dtype=td, device="cuda")
    v_pool = torch.empty((b.num_blocks, b.num_kv_heads, b.block_size, b.head_dim), dtype=td, device="cuda")
    if kv_fp8 is not None:
        k_pool.fill_(0x7F if poison else 0); v_pool.fill_(0x7F if poison else 0)
    elif poison:
        poison_(k_pool, b.dtype); poison_(v_pool, b.dtype)
    else:
        k_pool.zero_(); v_pool.zero_()

    def append(kk, vv, ss):
        if kv_fp8 is None:
            pk.pensieve_kv_append(kk, vv, k_pool, v_pool, ss)
        else:
            pk.pensieve_kv_append_fp8(kk, vv, k_pool, v_pool, ss, kv_fp8[0], kv_fp8[1])

    for r, k, v, slots, pos in b.iter_requests():
        for lo in range(0, len(pos), chunk_tokens):
            sel = pos[lo:lo + chunk_tokens]
            kk = to_device(k[sel], b.dtype); vv = to_device(v[sel], b.dtype)
            ss = torch.from_numpy(slots[lo:lo + chunk_tokens].copy()).cuda()
            append(kk, vv, ss)
    k_new_np, v_new_np = b.new_kv()
    k_new = to_device(k_new_np, b.dtype); v_new = to_device(v_new_np, b.dtype)
    new_slots = torch.from_numpy(b.new_slots.copy()).cuda()
    if append_new:
        append(k_new, v_new, new_slots)
    use_qpos = (not b.has_default_positions) if pass_q_pos is None else pass_q_pos
    gb = GpuBatch(b, k_pool, v_pool, to_device(b.q_all(), b.dtype), k_new, v_new, new_slots,
                  torch.from_numpy(b.block_tables.copy()).cuda(),
                  torch.from_numpy(b.context_lens.copy()).cuda(),
                  torch.from_numpy(b.cu_q_lens.copy()).cuda(),
                  torch.from_numpy(b.q_pos.copy()).cuda() if use_qpos else None, None, kv_fp8)
    gb.desc = gb.make_desc()
    torch.cuda.synchronize()
    return gb


def run_attn(gb: GpuBatch, flags: int = 0):
    import torch
    desc = gb.make_desc(flags)
    ws = torch.empty(max(pk.pensieve_attn_workspace_size(desc), 256), dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)    # every float in it reads as NaN until the library writes it
    o = torch.empty_like(gb.q)
    poison_(o, gb.batch.dtype)
    pk.pensieve_attn_fwd(desc, gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens, gb.cu_q_lens,
                         gb.q_pos, o, ws)
    torch.cuda.synchronize()
    return o


def run_split(gb: GpuBatch, P: int, flags: int = 0):
    import torch
    b = gb.batch
    desc = gb.make_desc(flags)
    ws = torch.empty(max(pk.pensieve_attn_workspace_size(desc, P), 256), dtype=torch.uint8, device="cuda")
    T = b.total_q
    po = torch.full((T, b.num_heads, P, b.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    pm = torch.full((T, b.num_heads, P), float("nan"), dtype=torch.float32, device="cuda")
    pl = torch.full((T, b.num_heads, P), float("nan"), dtype=torch.float32, device="cuda")
    pk.pensieve_attn_split_partial(desc, P, gb.q, gb.k_pool, gb.v_pool, gb.block_tables, gb.context_lens,
                                   gb.cu_q_lens, gb.q_pos, po, pm, pl, ws)
    o = torch.empty_like(gb.q)
    poison_(o, b.dtype)
    pk.pensieve_attn_split_merge(po, pm, pl, o)
    torch.cuda.synchronize()
    return po, pm, pl, o
