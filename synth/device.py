"""Uploads seeded synthetic inputs to a GPU as torch tensors (plumbing only)."""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass
class DeviceInputs:
    c: int
    k: int
    q: torch.Tensor            # int16 [R][4][128] (bf16 bit patterns)
    kcache: torch.Tensor       # int16 [slots][128]
    num_pages: int
    page_table: torch.Tensor   # int32 [B][pt_stride]
    req_row_ptr: torch.Tensor  # int32 [B+1]
    row_pos: torch.Tensor      # int32 [R]
    max_vis: int

    @property
    def num_rows(self) -> int:
        return int(self.row_pos.shape[0])

    @property
    def ld_out(self) -> int:
        return self.k * self.c + self.c - 1


def _t(a: np.ndarray, dtype, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dtype=dtype).to(device)


def upload(inp, device="cuda") -> DeviceInputs:
    return DeviceInputs(
        c=inp.c, k=inp.k,
        q=torch.from_numpy(np.ascontiguousarray(inp.q).view(np.int16)).to(device),
        kcache=torch.from_numpy(np.ascontiguousarray(inp.kcache).view(np.int16)).to(device),
        num_pages=int(inp.num_pages),
        page_table=_t(inp.page_table, torch.int32, device),
        req_row_ptr=_t(inp.req_row_ptr, torch.int32, device),
        row_pos=_t(inp.row_pos, torch.int32, device),
        max_vis=int(inp.max_vis))


@dataclasses.dataclass
class DeviceCompress:
    k_raw: torch.Tensor                  # int16 [T][128] (bf16 bit patterns)
    req_tok_ptr: torch.Tensor            # int32 [B+1]
    tok_start: torch.Tensor              # int32 [B]
    mrope_pos: "torch.Tensor | None"     # int32 [T][3]
    ring: torch.Tensor                   # int16 [B][4][128]
    ring_pos: torch.Tensor               # int32 [B][3]
    page_table: torch.Tensor             # int32 [B][pt_stride]
    kcache: torch.Tensor                 # int16 [num_pages*16][128]
    num_pages: int
    max_tok: int
    rotary_dim: int
    sections: tuple
    theta: float

    def args(self):
        """Positional arguments of block_scoring_top_amd.idx_compress_store."""
        return (self.k_raw, self.req_tok_ptr, self.tok_start, self.mrope_pos, self.max_tok, self.rotary_dim,
                self.sections, self.theta, self.ring, self.ring_pos, self.page_table, self.kcache,
                self.num_pages)


def upload_compress(ci, device="cuda") -> DeviceCompress:
    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return DeviceCompress(
        k_raw=bf(ci.k_raw.reshape(-1, 128)),
        req_tok_ptr=_t(ci.req_tok_ptr, torch.int32, device),
        tok_start=_t(ci.tok_start, torch.int32, device),
        mrope_pos=None if ci.mrope_pos is None else _t(ci.mrope_pos, torch.int32, device),
        ring=bf(ci.ring), ring_pos=_t(ci.ring_pos, torch.int32, device),
        page_table=_t(ci.page_table, torch.int32, device), kcache=bf(ci.kcache),
        num_pages=int(ci.num_pages), max_tok=int(ci.max_tok), rotary_dim=int(ci.rotary_dim),
        sections=tuple(ci.sections), theta=float(ci.theta))

