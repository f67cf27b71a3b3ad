"""A multi-layer model's projections packed on the device.

Every projection is quantized and packed by aq_pack_weights from a device
FP32 weight matrix that a caller-supplied function produces one at a time,
so the FP32 weights of a whole model never sit in memory next to the packed
model (AlignQuant Sec. 3.2: the packed model is what stays resident).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .binding import PackedWeights, aq_labels_from_map, aq_pack_weights


@dataclass
class PackedModel:
    """layers[l][name] is the packed projection `name` of layer l."""
    geometry: list            # [(name, N, K)] per layer
    layers: list = field(default_factory=list)

    def nbytes(self) -> int:
        return sum(pw.nbytes() for layer in self.layers for pw in layer.values())

    def __iter__(self):
        for l, layer in enumerate(self.layers):
            for name, _, _ in self.geometry:
                yield l, name, layer[name]


def pack_model(geometry, maps, weight_fn, bN: int = 64, bK: int = 128, progress=None) -> PackedModel:
    """Pack every projection of every layer.

    geometry  : [(name, N, K)], the projections of one layer in call order;
    maps      : maps[l][p] is the [N/bN, K/bK] precision map (4 or 8) of
                projection p of layer l;
    weight_fn : weight_fn(l, name, N, K) -> device FP32 [N, K] weights;
    progress  : optional callable(l) after each layer.
    """
    model = PackedModel(geometry=list(geometry))
    for l, layer_maps in enumerate(maps):
        layer = {}
        for (name, N, K), z in zip(geometry, layer_maps):
            W = weight_fn(l, name, N, K)
            layer[name] = aq_pack_weights(W, aq_labels_from_map(np.asarray(z, dtype=np.uint8)), bN, bK)
            del W
        model.layers.append(layer)
        if progress is not None:
            progress(l)
    return model


@dataclass
class PackedGroup:
    """Projections that share one input, packed as one (App. E.4): the
    members' tile rows are concatenated in member order, so eq. 16's row
    offsets run over the whole group and one quantization of the shared
    input and one linear call serve every member.  members[i] = (name, n0,
    n1): member i owns output features n0 .. n1-1 of the group."""
    packed: PackedWeights
    members: list

    def slices(self, Y) -> dict:
        """The members' outputs: views of the group output Y [M, N]."""
        return {name: Y[:, n0:n1] for name, n0, n1 in self.members}


def pack_group(members, weights, maps, bN: int = 64, bK: int = 128) -> PackedGroup:
    """Pack input-sharing projections as one (App. E.4 grouping).

    members : member names, in the order their rows are concatenated;
    weights : device FP32 [N_i, K] per member (same K, N_i a multiple of bN);
    maps    : [N_i/bN, K/bK] precision maps (4 or 8) per member.
    """
    import torch
    if not members or len(members) != len(weights) or len(weights) != len(maps):
        raise ValueError("one weight matrix and one map per member")
    K = weights[0].shape[1]
    if any(w.shape[1] != K or w.shape[0] % bN for w in weights):
        raise ValueError("members must share K and have whole tile rows")
    spans, n0 = [], 0
    for name, w in zip(members, weights):
        spans.append((name, n0, n0 + w.shape[0]))
        n0 += w.shape[0]
    z = np.concatenate([np.asarray(m, dtype=np.uint8) for m in maps], axis=0)
    W = torch.cat(list(weights), dim=0)
    pw = aq_pack_weights(W, aq_labels_from_map(z), bN, bK)
    del W
    return PackedGroup(packed=pw, members=spans)


def tile_row_slices(pw: PackedWeights, tile_rows) -> dict:
    """Host copies of the packed bytes of the given tile rows, concatenated in
    the given order: the W4 and W8 tiles and their scales occupy one
    contiguous run per tile row in each buffer (App. E.1 eq. 16), from
    row_off_b[r] to row_off_b[r + 1]."""
    import torch
    p = pw.plan
    torch.cuda.synchronize()
    off4 = pw.row_off4[:p.offs_bytes].cpu().numpy().view(np.int32)
    off8 = pw.row_off8[:p.offs_bytes].cpu().numpy().view(np.int32)
    t4, t8 = 64 * p.bK // 2, 64 * p.bK     # bytes of one W4 / W8 tile
    out = {k: [] for k in ("w4", "w8", "s4", "s8")}
    for r in tile_rows:
        a4, b4, a8, b8 = int(off4[r]), int(off4[r + 1]), int(off8[r]), int(off8[r + 1])
        out["w4"].append(pw.w4[a4 * t4:b4 * t4].cpu().numpy())
        out["w8"].append(pw.w8[a8 * t8:b8 * t8].cpu().numpy())
        out["s4"].append(pw.s4[a4 * 256:b4 * 256].cpu().numpy().view(np.float32))
        out["s8"].append(pw.s8[a8 * 256:b8 * 256].cpu().numpy().view(np.float32))
    res = {k: np.concatenate(v) if v else np.zeros(0) for k, v in out.items()}
    res["row_off4"], res["row_off8"] = off4, off8
    res["labels"] = pw.labels[:p.labels_bytes].cpu().numpy()
    return res
