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
