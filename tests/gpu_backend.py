"""The HIP library in the numpy calling convention of the CPU oracle.

Used by the GPU parity tests: numpy arrays go to the device, the C entry
point runs, results come back to the host for comparison.
"""
from __future__ import annotations

import numpy as np
import torch

from sparse_attention_kv_plan_amd import kvc


def to_dev(a, device="cuda"):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device)
    return torch.from_numpy(a).to(device)


def to_host(t, like=None):
    a = t.cpu().numpy()
    if like is not None and like.dtype == np.uint16:
        return a.view(np.uint16)
    return a


class GpuBackend:
    def __init__(self, device="cuda"):
        self.device = device
        kvc.load()

    def plan_prefill(self, cr, s, e, idx, rows, num_q, cap_c, cap_w):
        d = self.device
        pc, pw, counts = kvc.alloc_prefill_plan(cr, len(s), num_q, d, cap_c=cap_c, cap_w=cap_w)
        pc.fill_(0x5A)
        pw.fill_(0x5A)
        counts.fill_(-7)
        kvc.plan_prefill(cr, to_dev(np.asarray(s, np.int32)), to_dev(np.asarray(e, np.int32)),
                         to_dev(np.asarray(idx, np.int32)), int(rows), int(num_q), pc, pw, counts)
        return pc.cpu().numpy(), pw.cpu().numpy(), counts.cpu().numpy()

    def compress(self, cr, hd, state, inp, ape, pc, num_c):
        d = self.device
        out = torch.full((max(pc.shape[0], 1), hd), float("nan"), dtype=torch.float32, device=d)
        counts = torch.tensor([num_c, 0, 0, 0], dtype=torch.int32, device=d)
        kvc.compress(cr, hd, to_dev(state), to_dev(inp), to_dev(ape), to_dev(pc), counts, out)
        return out[: pc.shape[0]].cpu().numpy().astype(np.float64), int(counts[3].item())

    def write(self, cr, hd, state, inp, pw, num_w):
        d = self.device
        st = to_dev(state)
        counts = torch.tensor([0, num_w, 0, 0], dtype=torch.int32, device=d)
        kvc.write(cr, hd, st, to_dev(inp), to_dev(pw), counts)
        assert int(counts[3].item()) == 0
        return to_host(st, state)

    def plan_decode(self, cr, s, idx, rows):
        d = self.device
        pd = torch.full((len(s), kvc.D_BYTES), 0x5A, dtype=torch.uint8, device=d)
        status = torch.full((1,), -7, dtype=torch.int32, device=d)
        kvc.plan_decode(cr, to_dev(np.asarray(s, np.int32)), to_dev(np.asarray(idx, np.int32)), int(rows), pd,
                        status)
        return pd.cpu().numpy(), int(status.item())

    def plan_prefill_swa(self, cr, s, e, rid, r2t, f2s, sps, ring, rows, num_q, cap_c, cap_w):
        d = self.device
        pc, pw, counts = kvc.alloc_prefill_plan(cr, len(s), num_q, d, cap_c=cap_c, cap_w=cap_w)
        pc.fill_(0x5A)
        pw.fill_(0x5A)
        counts.fill_(-7)
        status = torch.zeros(1, dtype=torch.int32, device=d)
        kvc.plan_prefill_swa(cr, to_dev(np.asarray(s, np.int32)), to_dev(np.asarray(e, np.int32)),
                             to_dev(np.asarray(rid, np.int32)), to_dev(np.asarray(r2t, np.int32)),
                             to_dev(np.asarray(f2s, np.int32)), sps, ring, int(rows), int(num_q), pc, pw, counts,
                             status)
        return pc.cpu().numpy(), pw.cpu().numpy(), counts.cpu().numpy(), int(status.item())

    def plan_decode_swa(self, cr, s, rid, r2t, f2s, sps, ring, rows):
        d = self.device
        pd = torch.full((len(s), kvc.D_BYTES), 0x5A, dtype=torch.uint8, device=d)
        status = torch.full((1,), -7, dtype=torch.int32, device=d)
        kvc.plan_decode_swa(cr, to_dev(np.asarray(s, np.int32)), to_dev(np.asarray(rid, np.int32)),
                            to_dev(np.asarray(r2t, np.int32)), to_dev(np.asarray(f2s, np.int32)), sps, ring,
                            int(rows), pd, status)
        return pd.cpu().numpy(), int(status.item())

    def decode(self, cr, hd, state, inp, ape, pd):
        d = self.device
        st = to_dev(state)
        out = torch.full((pd.shape[0], hd), float("nan"), dtype=torch.float32, device=d)
        status = torch.zeros(1, dtype=torch.int32, device=d)
        kvc.decode(cr, hd, st, to_dev(inp), to_dev(ape), to_dev(pd), out, status)
        return out.cpu().numpy().astype(np.float64), to_host(st, state), int(status.item())

    # online ratio-128 state: slots float32 [slots, 3, hd] on the device, numpy on the host
    def compress_online(self, hd, state, inp, ape, pc, num_c):
        d = self.device
        out = torch.full((max(pc.shape[0], 1), hd), float("nan"), dtype=torch.float32, device=d)
        counts = torch.tensor([num_c, 0, 0, 0], dtype=torch.int32, device=d)
        st = to_dev(np.asarray(state, np.float32))
        kvc.compress_c128_online(hd, st, to_dev(inp), to_dev(ape), to_dev(pc), counts, out[: pc.shape[0]])
        return out[: pc.shape[0]].cpu().numpy().astype(np.float64), int(counts[3].item())

    def write_online(self, hd, state, inp, ape, pw, num_w):
        d = self.device
        counts = torch.tensor([0, num_w, 0, 0], dtype=torch.int32, device=d)
        st = to_dev(np.asarray(state, np.float32))
        kvc.write_c128_online(hd, st, to_dev(inp), to_dev(ape), to_dev(pw), counts)
        return st.cpu().numpy(), int(counts[3].item())

    def decode_online(self, hd, state, inp, ape, pd):
        d = self.device
        out = torch.full((pd.shape[0], hd), float("nan"), dtype=torch.float32, device=d)
        status = torch.zeros(1, dtype=torch.int32, device=d)
        st = to_dev(np.asarray(state, np.float32))
        kvc.decode_c128_online(hd, st, to_dev(inp), to_dev(ape), to_dev(pd), out, status)
        return out.cpu().numpy().astype(np.float64), st.cpu().numpy(), int(status.item())

    # ratio 4 over caller-allocated 4-row pages
    def plan_prefill_page4(self, s, e, idx, bundle, rows, num_q, cap_c, cap_w):
        d = self.device
        pc, pw, counts = kvc.alloc_prefill_plan(4, len(s), num_q, d, cap_c=cap_c, cap_w=cap_w)
        pc.fill_(0x5A)
        pw.fill_(0x5A)
        counts.fill_(-7)
        status = torch.zeros(1, dtype=torch.int32, device=d)
        kvc.plan_prefill_page4(to_dev(np.asarray(s, np.int32)), to_dev(np.asarray(e, np.int32)),
                               to_dev(np.asarray(idx, np.int32)),
                               to_dev(np.asarray(bundle, np.int32).reshape(-1, 4)), int(rows), int(num_q), pc, pw,
                               counts, status)
        return pc.cpu().numpy(), pw.cpu().numpy(), counts.cpu().numpy(), int(status.item())

    def plan_decode_page4(self, s, idx, prev, rows):
        d = self.device
        pd = torch.full((len(s), kvc.D_BYTES), 0x5A, dtype=torch.uint8, device=d)
        status = torch.full((1,), -7, dtype=torch.int32, device=d)
        kvc.plan_decode_page4(to_dev(np.asarray(s, np.int32)), to_dev(np.asarray(idx, np.int32)),
                              to_dev(np.asarray(prev, np.int32)), int(rows), pd, status)
        return pd.cpu().numpy(), int(status.item())
