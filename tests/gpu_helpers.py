"""Host <-> device plumbing for the GPU tests (no arithmetic of the method here)."""
import numpy as np
import torch

import bit_routed_expert_amd as moe


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def pack(planes):
    return moe.moe_w2_pack(dev(planes["gu_codes"]), dev(planes["gu_scales"]),
                           dev(planes["dn_codes"]), dev(planes["dn_scales"]))


def forward(handle, x_bits, ids, w, out_dtype=moe.OUT_F32, path=moe.PATH_AUTO, workspace=None):
    y = moe.moe_w2_forward(handle, dev_bf16(x_bits), dev(np.asarray(ids, np.int32)),
                           dev(np.asarray(w, np.float32)), out_dtype=out_dtype, path=path,
                           workspace=workspace)
    torch.cuda.synchronize()
    return y


def rel_max_err(y_gpu, y_ref):
    """max |y_gpu - y_ref| / rms(y_ref) over the compared entries."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    rms = np.sqrt(np.mean(np.square(y_ref)))
    return float(np.max(np.abs(y_gpu - y_ref)) / rms)


def bf16_rne_bits(f32):
    """fp32 array -> bf16 bit patterns, round to nearest even (torch's conversion)."""
    t = torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)
