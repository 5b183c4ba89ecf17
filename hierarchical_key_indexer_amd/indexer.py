"""Device-memory owner around the C ABI: an index blob plus the workspaces of
build / select / flat select, held as torch uint8 tensors on the GPU.  Every
call goes straight to liblsa.so."""
from __future__ import annotations

import torch

from . import _abi


class LatentIndex:
    def __init__(self, desc: _abi.IndexDesc, device: str = "cuda"):
        self.desc = desc
        self.device = device
        self.index = torch.empty(_abi.index_bytes(desc), dtype=torch.uint8, device=device)
        self._ws = {}

    def workspace(self, name: str, nbytes: int) -> torch.Tensor:
        buf = self._ws.get(name)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
            self._ws[name] = buf
        return buf

    def build(self, keys: torch.Tensor, W: torch.Tensor, stream=None) -> None:
        ws = self.workspace("build", _abi.build_workspace_bytes(self.desc))
        _abi.lsa_build_index(self.desc, keys, W, self.index, ws, stream)

    def release_build_workspace(self) -> None:
        self._ws.pop("build", None)

    def select(self, queries, q_pos, params, scores=True, leaves=False, out=None, stream=None):
        t, hq = queries.shape[0], queries.shape[1]
        width = _abi.select_out_width(params)
        ws = self.workspace("select", _abi.select_workspace_bytes(self.desc, params, t, hq))
        if out is None:
            out = self.alloc_select_outputs(t, hq, params, scores, leaves)
        idx, sc, lv = out
        _abi.lsa_select(self.desc, self.index, queries, q_pos, params, idx, sc, lv, ws, stream)
        return out

    def alloc_select_outputs(self, t, hq, params, scores=True, leaves=False, flat=False):
        width = _abi.select_out_width(params)
        idx = torch.empty((t, hq, width), dtype=torch.int32, device=self.device)
        sc = torch.empty((t, hq, params.k), dtype=torch.float32, device=self.device) if scores else None
        lv = None
        if leaves and not flat:
            nl = params.b if params.beam == _abi.LSA_BEAM_GLOBAL else params.b ** self.desc.n_levels
            lv = torch.empty((t, hq, nl), dtype=torch.int32, device=self.device)
        return idx, sc, lv

    def leaf_counts(self):
        """Members of every leaf bucket, [Hkv, P_L] int64 (host), read from the
        blob: the header holds the byte offset of each level's CSR offsets."""
        import numpy as np
        L = self.desc.n_levels
        hdr = self.index[:256].cpu().numpy()
        off = int(hdr[168 + 8 * (L - 1):176 + 8 * (L - 1)].view(np.uint64)[0])
        nodes = int(np.prod([self.desc.fanout[i] for i in range(L)]))
        hk = self.desc.n_kv_heads
        sec = self.index[off:off + hk * (nodes + 1) * 4].view(torch.int32).view(hk, nodes + 1)
        return np.diff(sec.cpu().numpy().astype(np.int64), axis=1)

    def device_status(self, which: str = "select") -> int:
        """Device status of the last select ("select") or flat select
        ("flat") call on this index, read after it finished: LSA_OK, or
        LSA_ERR_BAD_INDEX when the blob did not match the descriptor."""
        return _abi.device_status(self._ws[which])

    def flat_select(self, queries, q_pos, params, scores=True, out=None, stream=None):
        t, hq = queries.shape[0], queries.shape[1]
        ws = self.workspace("flat", _abi.flat_workspace_bytes(self.desc, params, t, hq))
        if out is None:
            out = self.alloc_select_outputs(t, hq, params, scores, flat=True)
        idx, sc, _ = out
        _abi.lsa_flat_select(self.desc, self.index, queries, q_pos, params, idx, sc, ws, stream)
        return out


def keys_to_device(arr, device="cuda") -> torch.Tensor:
    """Host key/query array (float32, or uint16 bf16 bits) -> device tensor."""
    import numpy as np
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
