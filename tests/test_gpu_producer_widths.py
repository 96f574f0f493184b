"""Bit-exact parity of the four fused producers (residual add + RMSNorm + ROW_MX or MX block-32
encoding, in the pages' row layouts and staged in the projection's operand layout) against the
oracle at every row width class: the one-wavefront-per-row kernels are instantiated for rows of
up to 1024, 2048, 4096, 5120 and 8192 elements (2, 4, 8, 10 and 16 chunks of 8 per lane), and
wider rows take the block-per-row kernels.  The widths below hit each instantiation at its
upper edge and just past the previous one (lanes with no chunk in the last round), the
narrowest legal row (one MX block) and the first width past the wavefront kernels, with a
ragged token count (37, so the staged images carry 219 padding rows) and one unpadded width
below H ([RMSNORM-MX] "unpadded_hidden_size")."""
import numpy as np
import pytest

import gpu_common as G
import oracle
import synth

pytestmark = pytest.mark.gpu

T = 37
WIDTHS = [(32, 0), (96, 0), (1024, 0), (1056, 1000), (2080, 0), (4096, 0), (5120, 0),
          (5152, 0), (8192, 0), (8224, 8200)]


@pytest.mark.parametrize("H,Hu", WIDTHS, ids=[f"H{h}" + (f"-Hu{u}" if u else "") for h, u in WIDTHS])
def test_fused_producers_every_width(H, Hu):
    import torch
    import rope_mxfp8_qkv_amd as q
    q.lib()
    dev = G.torch_dev()
    hid, res, gam = synth.producer_inputs(90 + H % 97, T, H)
    if Hu:
        hid[:, Hu:] = 0
        res[:, Hu:] = 0
    hd, rd, gd = G.bf16_dev(hid, dev), G.bf16_dev(res, dev), G.bf16_dev(gam, dev)
    print(f"fused producers T={T} H={H} Hu={Hu}", flush=True)

    # ROW_MX: packed rows and the staged image + row scales
    res_ref, packed_ref, _ = oracle.rmsnorm_rowmx(hid, res, gam, 1e-6, Hu)
    codes_ref, s_ref = oracle.rowmx_unpack(packed_ref, H)
    packed = torch.empty((T, H + 4), dtype=torch.uint8, device=dev)
    res_out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    q.rmsnorm_mx_quantize(hd, gd, 1e-6, packed, residual=rd, residual_out=res_out, unpadded_h=Hu)
    img = torch.full((q.qkv_act_image_bytes(T, H),), 0xA5, dtype=torch.uint8, device=dev)
    sc = torch.full((T,), float("nan"), dtype=torch.float32, device=dev)
    res_out2 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    q.rmsnorm_mx_quantize_staged(hd, gd, 1e-6, img, sc, residual=rd, residual_out=res_out2,
                                 unpadded_h=Hu)
    torch.cuda.synchronize()
    G.check_equal(G.bf16_host(res_out), res_ref, "residual_out (ROW_MX)")
    G.check_equal(G.bf16_host(res_out2), res_ref, "residual_out (staged ROW_MX)")
    G.check_equal(packed.cpu().numpy(), packed_ref, "ROW_MX rows")
    G.check_equal(G.unstage(img, np.arange(T), H), codes_ref, "staged ROW_MX codes")
    G.check_equal(sc.cpu().numpy().view(np.uint32), s_ref.astype(np.float32).view(np.uint32),
                  "staged ROW_MX scales")
    G.check_stage_padding(img, T, H)

    # MX block-32: natural codes + exponents + bf16 normed rows, and the staged images
    res_ref, codes_ref, e8_ref, norm_ref, _ = oracle.rmsnorm_mx(hid, res, gam, 1e-6, Hu)
    codes = torch.empty((T, H), dtype=torch.uint8, device=dev)
    e8 = torch.empty((T, H // 32), dtype=torch.uint8, device=dev)
    norm = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    q.rmsnorm_mx_block_quantize(hd, gd, 1e-6, codes, e8, residual=rd, residual_out=res_out,
                                norm_out=norm, unpadded_h=Hu)
    img.fill_(0xA5)
    eimg = torch.full((q.qkv_act_exp_image_bytes(T, H) // 4,), 0x5A5A5A5A, dtype=torch.int32,
                      device=dev)
    q.rmsnorm_mx_block_quantize_staged(hd, gd, 1e-6, img, eimg, residual=rd,
                                       residual_out=res_out2, unpadded_h=Hu)
    torch.cuda.synchronize()
    G.check_equal(G.bf16_host(res_out), res_ref, "residual_out (MX)")
    G.check_equal(G.bf16_host(res_out2), res_ref, "residual_out (staged MX)")
    G.check_equal(G.bf16_host(norm), norm_ref, "bf16 normed rows")
    G.check_equal(codes.cpu().numpy(), codes_ref, "MX codes")
    G.check_equal(e8.cpu().numpy(), e8_ref, "MX exponents")
    G.check_equal(G.unstage(img, np.arange(T), H), codes_ref, "staged MX codes")
    G.check_equal(G.unstage_exp(eimg, np.arange(T), H), e8_ref, "staged MX exponents")
    G.check_stage_padding(img, T, H)
    G.check_exp_padding(eimg, T, H)
