"""GPU-side helpers of the parity tests: device buffers and calls through the
C ABI (via the ctypes binding)."""
import numpy as np
import torch

from oracle import lsa_oracle as O


def _abi():
    from hierarchical_key_indexer_amd import _abi as A
    return A


def _li(desc_o: O.IndexDesc, blob=None):
    from hierarchical_key_indexer_amd.indexer import LatentIndex
    A = _abi()
    d = A.IndexDesc.make(desc_o.n_keys, desc_o.n_kv_heads, desc_o.d_head, desc_o.d_latent, desc_o.key_dtype,
                         desc_o.latent_dtype, desc_o.fanout, desc_o.kmeans_iters, desc_o.seed)
    li = LatentIndex(d)
    if blob is not None:
        assert li.index.numel() == blob.size
        li.index.copy_(torch.from_numpy(blob))
    return li


def _dev(arr):
    from hierarchical_key_indexer_amd.indexer import keys_to_device
    return keys_to_device(arr)


def _params(prm: O.SelectParams):
    return _abi().SelectParams.make(prm.b, prm.k, prm.sink, prm.window, prm.beam)


def gpu_select(li, queries, pos, prm, flat=False, leaves=True):
    q = _dev(queries)
    p = torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).cuda()
    if flat:
        idx, sc, lv = li.flat_select(q, p, _params(prm))
    else:
        idx, sc, lv = li.select(q, p, _params(prm), leaves=leaves)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), sc.cpu().numpy(), (None if lv is None else lv.cpu().numpy())


def gpu_build(desc_o, keys, W):
    li = _li(desc_o)
    li.build(_dev(keys), torch.from_numpy(W).cuda())
    torch.cuda.synchronize()
    return li


def _blob_of(li):
    return li.index.cpu().numpy()


def one_head_index(li, desc_o: O.IndexDesc, h: int) -> O.OracleIndex:
    """KV head h of a device-resident index as a one-head oracle index: every
    section of head h is copied from the device into a one-head blob of the
    same layout, which the oracle's reader then decodes."""
    import dataclasses
    d1 = dataclasses.replace(desc_o, n_kv_heads=1)
    lay, lay1 = O.blob_layout(desc_o), O.blob_layout(d1)
    ls = 2 if desc_o.latent_dtype == "bf16" else 4
    dl, n = desc_o.d_latent, desc_o.n_keys
    sizes = {"W": desc_o.d_head * dl * 4, "perm": n * 4, "latent": n * dl * ls}
    for lev in range(1, desc_o.n_levels + 1):
        p = desc_o.nodes(lev)
        sizes[f"cent{lev}"] = p * dl * 4
        sizes[f"cscore{lev}"] = p * dl * ls
        sizes[f"off{lev}"] = (p + 1) * 4
    blob1 = np.zeros(lay1["total"], dtype=np.uint8)
    for name, sz in sizes.items():
        src = lay[name] + h * sz
        blob1[lay1[name]:lay1[name] + sz] = li.index[src:src + sz].cpu().numpy()
    return O.index_from_blob(blob1, d1)
