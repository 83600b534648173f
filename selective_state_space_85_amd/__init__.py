"""MI355X (gfx950) selective scan: a C-ABI HIP library plus a thin torch binding.

    from selective_state_space_85_amd import scan_fwd, step
    y = scan_fwd(u, delta, A, B, C, D=Dskip, z=z)          # (B, L, D)
    y_t = step(h, u_t, delta_t, A, B_t, C_t, D=Dskip, z=z_t)  # h (B, D, N) updated in place
    grads = scan_bwd(u, delta, A, B, C, dy, D=Dskip, z=z)    # du, ddelta, dA, dB, dC, dD, dz, dh0
    ck = torch.empty(scan_ckpt_shape(Bsz, L, D, N), device="cuda")  # training: the forward keeps
    y = scan_fwd(u, delta, A, B, C, D=Dskip, z=z, ckpt=ck)  # every 16th state, the backward
    grads = scan_bwd(u, delta, A, B, C, dy, D=Dskip, z=z, ckpt=ck)  # reuses them
    u = conv1d_silu(xz[..., :D], conv_weight, conv_bias)     # the block's causal conv + SiLU
    y2 = ssd_fwd(x, dt, A_heads, B, C, D=D_heads)            # multi-head (Mamba-2) recurrence

The library itself is ``libssscan.so`` (``include/ss_scan.h``), built by
``selective_state_space_85_amd.build``.
"""
from ._lib import LIB_PATH, SSError, load as load_library  # noqa: F401
from .ops import (conv1d_silu, scan_bwd, scan_bwd_workspace_bytes, scan_ckpt_shape, scan_fwd,  # noqa: F401
                  scan_fwd_noalloc, scan_plan, scan_workspace_bytes, ssd_fwd, ssd_workspace_bytes, step)

__all__ = ["scan_fwd", "scan_fwd_noalloc", "scan_bwd", "step", "conv1d_silu", "ssd_fwd", "scan_plan", "scan_workspace_bytes",
           "scan_bwd_workspace_bytes", "scan_ckpt_shape", "ssd_workspace_bytes", "load_library", "LIB_PATH",
           "SSError"]
