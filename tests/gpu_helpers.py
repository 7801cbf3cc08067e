"""Test plumbing shared by the GPU parity tests: builds engine-layout tensors
on the GPU, runs the HIP path through the C ABI, copies pages to host
layouts for the oracle and compares per segment.  No codec arithmetic here:
expected values come from the oracle only.
"""
from __future__ import annotations

import numpy as np
import torch

import kv_cache_page_kvc_amd as kvc
from kv_cache_page_kvc_amd import inputs
from oracle import kvc_oracle as O

SEG_BYTES_HDR = 32


def u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class Workload:
    """Engine tensors for one call plus the matching kvc.Layout."""

    def __init__(self, layers, heads, dim, tokens, pool, dtype="bf16", layout="separate", seed=0,
                 k_kind="lognormal", device="cuda"):
        self.L, self.H, self.D, self.T, self.pool = layers, heads, dim, tokens, pool
        self.dtype_name, self.kind_name = dtype, layout
        self.dt = O.BF16 if dtype == "bf16" else O.FP16
        td = inputs.torch_dtype(dtype)
        if layout == "separate":
            self.k, self.v = inputs.separate_kv(layers, pool, tokens, heads, dim, td, seed, device, k_kind)
            self.layout = kvc.Layout.separate(self.k, self.v, heads, dim, tokens)
        else:
            self.k = inputs.packed_kv(layers, pool, heads, tokens, dim, td, seed, device, k_kind)
            self.v = None
            self.layout = kvc.Layout.packed(self.k, heads, dim, tokens)

    def empty_like(self, fill_bits=None):
        """A destination pool of the same geometry (optionally filled)."""
        other = object.__new__(Workload)
        other.__dict__.update({k: v for k, v in self.__dict__.items() if k not in ("k", "v", "layout")})
        other.k = [torch.empty_like(t) for t in self.k]
        other.v = [torch.empty_like(t) for t in self.v] if self.v is not None else None
        for t in other.k + (other.v or []):
            if fill_bits is None:
                t.zero_()
            else:
                t.view(torch.int16).fill_(fill_bits - 65536 if fill_bits >= 32768 else fill_bits)
        if self.v is not None:
            other.layout = kvc.Layout.separate(other.k, other.v, self.H, self.D, self.T)
        else:
            other.layout = kvc.Layout.packed(other.k, self.H, self.D, self.T)
        return other

    def host_layout(self, pages=None):
        """Oracle host layout.  With `pages` (list of block ids) only those
        blocks are copied; the returned map sends a block id to its index in
        the copy."""
        sel = list(range(self.pool)) if pages is None else sorted(set(int(p) for p in pages))
        idx = torch.tensor(sel, dtype=torch.long, device=self.k[0].device)
        remap = {b: j for j, b in enumerate(sel)}
        ks = [u16(t.index_select(0, idx)).reshape(-1) for t in self.k]
        if self.v is not None:
            vs = [u16(t.index_select(0, idx)).reshape(-1) for t in self.v]
            T, H, D = self.T, self.H, self.D
            lay = O.HostLayout(self.dt, self.L, H, D, T, len(sel), T * H * D, H * D, D, ks, vs)
        else:
            T, H, D = self.T, self.H, self.D
            lay = O.HostLayout(self.dt, self.L, H, D, T, len(sel), H * T * 2 * D, 2 * D, T * 2 * D, ks)
        return lay, remap


def gpu_encode(ctx, wl: Workload, codec: kvc.Codec, page_ids, spill_bytes=None, stream=0):
    slot, spill_sugg, _ = kvc.kvc_plan(wl.layout, codec, len(page_ids))
    spill = spill_sugg if spill_bytes is None else spill_bytes
    total = slot + spill
    out = torch.zeros(max(total, 256), dtype=torch.uint8, device="cuda")
    nseg = wl.L * len(page_ids) * 2
    desc = torch.zeros(nseg * 32, dtype=torch.uint8, device="cuda")
    kvc.kvc_encode_pages(ctx, wl.layout, codec, page_ids, out.data_ptr(), total, desc.data_ptr(), stream)
    return out, desc, slot, total


def desc_np(desc: torch.Tensor):
    return desc.cpu().numpy().view(kvc.DESC_DTYPE)


def gpu_decode(ctx, dst: Workload, codec: kvc.Codec, buf: torch.Tensor, nbytes, dst_page_ids, stream=0):
    nseg = dst.L * len(dst_page_ids) * 2
    st = torch.full((nseg,), 255, dtype=torch.uint8, device="cuda")
    kvc.kvc_decode_pages(ctx, dst.layout, codec, buf.data_ptr(), nbytes, dst_page_ids, st.data_ptr(), stream)
    return st


def segments_of(L, n_pages):
    return O.segment_list(L, n_pages)


def oracle_encode(wl: Workload, codec_k, codec_v, seed, page_ids, fixed=None, protected=None, segments=None,
                  crc=False):
    """Oracle encode of the given segments (all if None) of a call."""
    pages_needed = None
    if segments is not None:
        seglist = O.segment_list(wl.L, len(page_ids))
        pages_needed = [int(page_ids[seglist[s][1]]) for s in segments]
    lay, remap = wl.host_layout(pages_needed)
    mapped = np.array([remap.get(int(p), 0) for p in page_ids], np.int32)
    prot = None
    if protected is not None:
        prot = [1 if l in protected else 0 for l in range(wl.L)]
    return O.encode_pages(lay, codec_k, codec_v, seed, mapped, fixed_scales=fixed, protected=prot,
                          segments=segments, crc=crc)


def compare_encoded(gpu_buf: np.ndarray, gpu_desc, ora_buf, ora_status, offs, total, segments):
    """Per segment: status equal; slot bytes identical for encoded and
    policy-raw segments; for data-raw segments the header equal except the
    spill offset, the rest of the slot zero, and the spilled bytes equal the
    source (from the oracle's own spill copy).  The descriptor's flags and crc32 equal the header's."""
    bad = []
    for s in segments:
        st = int(ora_status[s])
        d = gpu_desc[s]
        if int(d["status"]) != st:
            bad.append((s, "status", int(d["status"]), st))
            continue
        o = offs[s]
        hdr_g = gpu_buf[o:o + 32]
        hdr_o = ora_buf[o:o + 32]
        if int(d["flags"]) != int(hdr_g[2]) or int(d["crc32"]) != int(hdr_g[24:28].view(np.uint32)[0]):
            bad.append((s, "descriptor flags/crc32"))
        if st == O.SEG_RAW_DATA or (st == O.SEG_ENCODED and hdr_o[2] & O.FLAG_HEAP):
            # bytes in the spill region (raw source, or an entropy-coded payload):
            # headers equal but for the spill offset, stored bytes equal, rest of the slot zero
            if not (np.array_equal(hdr_g[:16], hdr_o[:16]) and np.array_equal(hdr_g[24:], hdr_o[24:])):
                bad.append((s, "spilled segment header"))
                continue
            size = (offs[s + 1] if s + 1 < len(offs) else total) - o
            if gpu_buf[o + 32:o + size].any():
                bad.append((s, "slot body"))         # a header-only slot is zero after the header
            so_g = int(hdr_g[16:24].view(np.uint64)[0])
            so_o = int(hdr_o[16:24].view(np.uint64)[0])
            n = int(hdr_o[12:16].view(np.uint32)[0])
            if int(d["spill_offset"]) != so_g or not np.array_equal(gpu_buf[so_g:so_g + n], ora_buf[so_o:so_o + n]):
                bad.append((s, "spill bytes"))
            continue
        size = (offs[s + 1] if s + 1 < len(offs) else total) - o
        seg_g, seg_o = gpu_buf[o:o + size], ora_buf[o:o + size]
        if not np.array_equal(seg_g, seg_o):
            diff = np.nonzero(seg_g != seg_o)[0]
            bad.append((s, "slot bytes", int(diff[0]), int(len(diff))))
        if int(d["offset"]) != o:
            bad.append((s, "offset", int(d["offset"]), o))
    return bad


def oracle_decode_segments(ora_buf, wl: Workload, codec_k, codec_v, seed, n_pages, protected, segments):
    """Oracle decode of selected segments: {segment: uint16 [n_vec, D]}."""
    offs, sizes, effs, total = O.plan(wl.L, wl.H, wl.D, wl.T, codec_k, codec_v,
                                      None if protected is None else
                                      [1 if l in protected else 0 for l in range(wl.L)], n_pages)
    n_vec = wl.T * wl.H
    return {s: O.decode_segment(ora_buf[offs[s]:offs[s] + sizes[s]], ora_buf, wl.dt, wl.D, n_vec, seed, heads=wl.H)
            for s in segments}


def gpu_segment_vectors(wl: Workload, layer, comp, block):
    """The n_vec x D bits of one segment of the (destination) pool, canonical order."""
    if wl.v is not None:
        t = (wl.k if comp == 0 else wl.v)[layer][block]           # [T, H, D]
        return u16(t).reshape(wl.T * wl.H, wl.D)
    t = wl.k[layer][block]                                         # [H, T, 2D]
    part = t[..., comp * wl.D:(comp + 1) * wl.D].permute(1, 0, 2)  # [T, H, D]
    return u16(part).reshape(wl.T * wl.H, wl.D)


def bits_to_f32(bits: np.ndarray, dt):
    return O.src_to_f32(bits, dt)
