"""CPU checks of the HIP library: it loads, exports every declared symbol, and
its host-side validation rejects bad arguments before touching a GPU."""
import os
import re

import pytest

from w4a16_routed_expert_amd import binding as B
from w4a16_routed_expert_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_every_declared_symbol_is_exported(lib):
    decl = declared_functions()
    assert len(decl) >= 9
    for name in decl:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert sorted(B.EXPORTS) == decl


def test_row_layout_matches_the_generator(lib):
    for H, I in ((256, 512), (2048, 1024), (2048, 1408), (128, 128)):
        rb, off = B.moe_expert_row_bytes(H, I)
        lay = synth.expert_row_layout(H, I)
        assert rb == lay["row_bytes"]
        assert off == {k: v for k, v in lay.items() if k != "row_bytes"}
    assert B.moe_expert_row_bytes(2048, 1000)[0] == 0


def test_route_workspace_holds_the_logits(lib):
    assert B.moe_route_workspace_size(32, 2048, 64) >= 32 * 64 * 4
    assert B.moe_route_workspace_size(32, 2048, 64) % 256 == 0
    assert B.moe_route_workspace_size(4, 2048, 65) == 0          # unsupported shapes report 0


def test_host_validation_rejects_bad_arguments(lib):
    F = 0x1000  # never dereferenced: validation fails first
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(F, F, None, 4, 256, 65, 2, None, F, F, F, F, F, F, F, F, 1 << 20, stream=0)
    assert ei.value.code == B.MOE_ERR_UNSUPPORTED
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(F, F, None, 4, 256, 8, 9, None, F, F, F, F, F, F, F, F, 1 << 20, stream=0)
    assert ei.value.code == B.MOE_ERR_UNSUPPORTED
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(None, F, None, 4, 256, 8, 2, None, F, F, F, F, F, F, F, F, 1 << 20, stream=0)
    assert ei.value.code == B.MOE_ERR_INVALID_ARG
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(F, F, None, 4, 8192, 8, 2, None, F, F, F, F, F, F, F, None, 0, stream=0)
    assert ei.value.code == B.MOE_ERR_UNSUPPORTED
    with pytest.raises(B.MoeError) as ei:
        B.moe_route(F, F, None, 4, 200, 8, 2, None, F, F, F, F, F, F, F, F, 1 << 20, stream=0)
    assert ei.value.code == B.MOE_ERR_UNSUPPORTED
    with pytest.raises(B.MoeError) as ei:     # the workspace is required
        B.moe_route(F, F, None, 4, 256, 8, 2, F, F, F, F, F, F, F, F, None, 0, stream=0)
    assert ei.value.code == B.MOE_ERR_WORKSPACE
    with pytest.raises(B.MoeError) as ei:     # and must be 256-byte aligned
        B.moe_route(F, F, None, 4, 256, 8, 2, F, F, F, F, F, F, F, F, F + 16, 1 << 20, stream=0)
    assert ei.value.code == B.MOE_ERR_WORKSPACE
    with pytest.raises(B.MoeError) as ei:     # row stride not a multiple of 256
        B.moe_w4a16_expert_ffn(F, 4, 256, 512, 8, 2, F, 199_680 + 16, None, F, F, F, F, F, F, stream=0)
    assert ei.value.code == B.MOE_ERR_INVALID_ARG
    with pytest.raises(B.MoeError) as ei:     # I not a multiple of 128
        B.moe_w4a16_expert_ffn(F, 4, 256, 500, 8, 2, F, 1 << 20, None, F, F, F, F, F, F, stream=0)
    assert ei.value.code == B.MOE_ERR_UNSUPPORTED
    for call in (B.moe_w4a16_expert_ffn, B.moe_w4a16_gateup):   # unknown kernel family
        with pytest.raises(B.MoeError) as ei:
            if call is B.moe_w4a16_gateup:
                call(F, 4, 256, 512, 8, 2, F, 1 << 20, None, F, F, F, F, F, mode=3, stream=0)
            else:
                call(F, 4, 256, 512, 8, 2, F, 1 << 20, None, F, F, F, F, F, F, mode=3, stream=0)
        assert ei.value.code == B.MOE_ERR_INVALID_ARG and "mode" in B.moe_last_error()
    with pytest.raises(B.MoeError) as ei:
        B.moe_w4a16_down(4, 256, 512, 8, 2, F, 1 << 20, None, F, F, F, F, F, mode=-1, stream=0)
    assert ei.value.code == B.MOE_ERR_INVALID_ARG
    with pytest.raises(B.MoeError) as ei:     # only one of the shared-expert pointers
        B.moe_combine(F, F, F, F, None, 4, 256, 2, F, stream=0)
    assert ei.value.code == B.MOE_ERR_INVALID_ARG
    assert "shared" in B.moe_last_error()


def test_layer_ksplit_mode_checks_and_workspace(lib):
    F = 0x1000
    buf = B.LayerBuffers(F, F, F, F, F, F, F, F, F, F, F, F, 1 << 30)
    # the K-split expert FFN needs T <= 16, H/128 even and H, I <= 2048: rejected on the host
    for T, H, I in ((17, 256, 512), (4, 384, 512), (4, 256, 4096)):
        with pytest.raises(B.MoeError) as ei:
            B.moe_layer_forward(F, F, None, T, H, I, 8, 2, F, 1 << 20, None, None, None, None, F, buf,
                                mode=B.MOE_FFN_PATH_KSPLIT, stream=0)
        assert ei.value.code == B.MOE_ERR_UNSUPPORTED and "K-split" in B.moe_last_error()
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_forward(F, F, None, 4, 256, 512, 8, 2, F, 1 << 20, None, None, None, None, F, buf, mode=5,
                            stream=0)
    assert ei.value.code == B.MOE_ERR_INVALID_ARG
    # the one-launch layer: decode batches of the shapes it is built for, rejected on the host otherwise
    for T, H, I, E, k in ((65, 2048, 1024, 64, 8), (4, 384, 512, 8, 2), (4, 2048, 1024, 63, 8),
                          (64, 256, 512, 8, 8)):
        with pytest.raises(B.MoeError) as ei:
            B.moe_layer_forward(F, F, None, T, H, I, E, k, F, 1 << 22, None, None, None, None, F, buf,
                                mode=B.MOE_FFN_PATH_ONE_LAUNCH, stream=0)
        assert ei.value.code == B.MOE_ERR_UNSUPPORTED and "one-launch" in B.moe_last_error(), (T, H, I, E, k)
    # a workspace sized for T serves every smaller batch (the planes of the
    # K-split path depend on the batch through the slice width)
    for (H, I, E, k) in ((2048, 1024, 64, 8), (2048, 1408, 60, 4), (256, 512, 8, 2)):
        sizes = [B.moe_layer_workspace_size(T, H, I, E, k) for T in list(range(0, 40)) + list(range(250, 262))]
        assert all(b >= a for a, b in zip(sizes, sizes[1:])), (H, I, E, k)
        # T = 1 on the OLMoE shape: 8 pairs x 32 planes of 2048 FP32 values at least
        if (H, I, E, k) == (2048, 1024, 64, 8):
            assert sizes[1] >= 8 * 32 * 2048 * 4
    assert B.moe_layer_workspace_size(4, 2048, 1024, 64, 9) == 0


def test_layer_with_shared_expert_checks(lib):
    # moe_layer_forward_shared validates the shared expert's arguments, the
    # layer shape and (on its routing + shared gate/up path) the layer buffers
    # before any device call
    F = 0x1000
    buf = B.LayerBuffers(F, F, F, F, F, F, F, F, F, F, F, F, 1 << 30)
    qwen = (2048, 1408, 60, 4)

    def call(T=1, H=2048, I=1408, E=60, k=4, Is=5632, wsg=F, sh_out=F, sh_ws_bytes=1 << 30, bufs=buf):
        B.moe_layer_forward_shared(F, F, None, T, H, I, E, k, F, 1 << 23, None, wsg, F, F, F, Is, sh_out, F, F,
                                   sh_ws_bytes, F, bufs, stream=0)

    for kw, code, word in ((dict(Is=5600), B.MOE_ERR_UNSUPPORTED, "multiples of 128"),
                           (dict(wsg=None), B.MOE_ERR_INVALID_ARG, "null"),
                           (dict(sh_out=F + 8), B.MOE_ERR_INVALID_ARG, "aligned"),
                           (dict(sh_ws_bytes=256), B.MOE_ERR_WORKSPACE, "shared-expert workspace"),
                           (dict(E=65, k=4), B.MOE_ERR_UNSUPPORTED, None),
                           (dict(bufs=B.LayerBuffers(F, F, F, F, F, F, F, F, F, F, F, F, 4096)),
                            B.MOE_ERR_WORKSPACE, "layer workspace")):
        with pytest.raises(B.MoeError) as ei:
            call(**kw)
        assert ei.value.code == code, kw
        if word:
            assert word in B.moe_last_error(), (kw, B.moe_last_error())
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_forward_shared(F, F, None, 1, 2048, 1408, 60, 4, F, 1 << 23, None, F, F, F, F, 5632, F, F, F,
                                   1 << 30, F, buf, mode=9, stream=0)
    assert ei.value.code == B.MOE_ERR_INVALID_ARG and "mode" in B.moe_last_error()
    assert B.moe_layer_workspace_size(1, *qwen) > 4096
    # T = 0: nothing to do
    call(T=0)


def test_table_create_rejects_before_touching_the_gpu(lib):
    # moe_table_create validates the descriptor and the host source's identity
    # and layout before any device call, so these run without a GPU.
    import numpy as np
    cfg = synth.CONFIGS["tiny"]
    rows = synth.make_expert_rows(cfg)
    stride = rows.strides[0]
    # steps of 2 tokens x top-2 with capacity 3 need min(5, 4 + 1) = 5 spare rows
    with pytest.raises(B.MoeError) as ei:
        B.moe_table_create(cfg.E, cfg.H, cfg.I, 3, 4, 2, cfg.k, 2, rows, stride, stream=0)
    assert ei.value.code == B.MOE_ERR_CAPACITY and "spare" in B.moe_last_error()
    with pytest.raises(B.MoeError) as ei:          # no staging
        B.moe_table_create(cfg.E, cfg.H, cfg.I, 3, 5, 0, cfg.k, 2, rows, stride, stream=0)
    assert ei.value.code == B.MOE_ERR_CAPACITY
    dig = np.array([B.moe_row_digest(rows[e]) for e in range(cfg.E)], np.uint64)
    bad = dig.copy()
    bad[6] ^= np.uint64(1)
    with pytest.raises(B.MoeError) as ei:          # identity: the digest of expert 6 does not match
        B.moe_table_create(cfg.E, cfg.H, cfg.I, 3, 5, 2, cfg.k, 2, rows, stride, row_digests=bad, stream=0)
    assert ei.value.code == B.MOE_ERR_SOURCE and "6" in B.moe_last_error()
    broken = rows.copy()
    off = synth.expert_row_layout(cfg.H, cfg.I)["down_s"]
    broken[1, off:off + 2] = np.frombuffer(np.float16(np.inf).tobytes(), np.uint8)
    with pytest.raises(B.MoeError) as ei:          # layout: a non-finite FP16 scale
        B.moe_table_create(cfg.E, cfg.H, cfg.I, 3, 5, 2, cfg.k, 2, broken, stride, stream=0)
    assert ei.value.code == B.MOE_ERR_SOURCE and "scale" in B.moe_last_error()
    # the digest is a plain function of the bytes
    assert B.moe_row_digest(rows[3]) == B.moe_row_digest(rows[3].copy())
    assert B.moe_row_digest(rows[3]) != B.moe_row_digest(rows[4])
