"""C-ABI tests that need no GPU: the library loads, exports every function
include/sdit.h declares, and the host-side validators reject bad arguments
with the documented status (nothing is launched by a validator)."""
import ctypes
import os
import re

import pytest

import streaming_video_dit_amd as sdit

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdit.h")

A16 = 0x10000          # fake, 16-byte aligned device addresses (never dereferenced)
MB = 1 << 20


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sdit_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    names = _declared_functions()
    assert "sdit_attn_fwd" in names and "sdit_kv_quant_int8" in names and "sdit_qknorm_rope3d" in names
    L = sdit.lib()
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings():
    L = sdit.lib()
    assert L.sdit_abi_version() == sdit.ABI_VERSION == 1
    assert L.sdit_status_string(0) == b"SDIT_OK"
    assert L.sdit_status_string(2) == b"SDIT_ERR_UNSUPPORTED"
    assert ctypes.sizeof(sdit.KVSegment) == 40


def _rope_args(**kw):
    a = dict(q_in=A16, k_in=A16 + 16 * MB, q_out=A16 + 32 * MB, k_out=A16 + 48 * MB, gamma_q=A16 + 64 * MB,
             gamma_k=A16 + 65 * MB, T=3, Hl=30, Wl=52, t0=9, n_heads=12, head_dim=128, d_t=44, d_h=42, d_w=42)
    a.update(kw)
    return a


def test_qknorm_validation():
    v = lambda **kw: sdit.validate_qknorm_rope3d_args(**_rope_args(**kw))
    assert v() == sdit.SDIT_OK
    assert v(q_out=A16, k_out=A16 + 16 * MB) == sdit.SDIT_OK              # exact in place
    assert v(head_dim=96, d_t=32, d_h=32, d_w=32) == sdit.SDIT_ERR_UNSUPPORTED
    assert v(d_t=43, d_h=43) == sdit.SDIT_ERR_INVALID                      # odd widths
    assert v(d_t=40) == sdit.SDIT_ERR_INVALID                              # does not sum to d
    assert v(q_in=A16 + 4) == sdit.SDIT_ERR_INVALID                        # misaligned
    assert v(k_in=None) == sdit.SDIT_ERR_INVALID
    assert v(q_out=A16 + 1024) == sdit.SDIT_ERR_INVALID                    # partial overlap
    assert v(n_heads=0) == sdit.SDIT_ERR_INVALID
    assert v(T=0, q_in=None) == sdit.SDIT_OK                               # empty grid: no-op
    assert v(theta=0.0) == sdit.SDIT_ERR_INVALID
    assert "axis split" in (v(d_t=40), sdit.last_error())[1]


def test_qknorm_quant_validation():
    def v(**kw):
        a = _rope_args()
        a.update(v_in=A16 + 80 * MB, k_codes=A16 + 96 * MB, k_scales=A16 + 104 * MB, v_codes=A16 + 112 * MB,
                 v_scales=A16 + 120 * MB)
        a.update(kw)
        return sdit.validate_qknorm_rope3d_kv_quant_int8_args(**a)
    assert v() == sdit.SDIT_OK
    assert v(q_out=A16, k_out=A16 + 16 * MB) == sdit.SDIT_OK              # exact in place
    assert v(d_t=40) == sdit.SDIT_ERR_INVALID                              # the plain call's checks come first
    assert v(v_in=None) == sdit.SDIT_ERR_INVALID
    assert v(k_codes=A16 + 96 * MB + 8) == sdit.SDIT_ERR_INVALID          # misaligned codes
    assert v(v_scales=A16 + 120 * MB + 2) == sdit.SDIT_ERR_INVALID        # misaligned scales
    assert v(k_scales=A16 + 96 * MB + 4096) == sdit.SDIT_ERR_INVALID      # scales inside the k codes
    assert v(v_codes=A16 + 80 * MB) == sdit.SDIT_ERR_INVALID              # codes over v_in
    assert v(k_codes=A16 + 64 * MB) == sdit.SDIT_ERR_INVALID              # codes over gamma
    assert v(v_in=A16 + 32 * MB) == sdit.SDIT_ERR_INVALID                 # q_out over v_in
    assert v(T=0, q_in=None, v_in=None, k_codes=None) == sdit.SDIT_OK     # empty grid: no-op
    assert v(head_dim=96, d_t=32, d_h=32, d_w=32) == sdit.SDIT_ERR_UNSUPPORTED


def test_kv_quant_validation():
    v = sdit.validate_kv_quant_args
    assert v(A16, A16 + 16 * MB, A16 + 32 * MB, 100, 12, 128) == sdit.SDIT_OK
    assert v(A16, A16 + 16 * MB, A16 + 32 * MB, 100, 12, 80) == sdit.SDIT_ERR_UNSUPPORTED
    assert v(A16, A16 + 8, A16 + 32 * MB, 100, 12, 128) == sdit.SDIT_ERR_INVALID
    assert v(A16, A16 + 1024, A16 + 32 * MB, 100, 12, 128) == sdit.SDIT_ERR_INVALID   # overlap
    assert v(None, None, None, 0, 12, 128) == sdit.SDIT_OK
    assert v(A16, A16 + 16 * MB, A16 + 32 * MB + 2, 100, 12, 128) == sdit.SDIT_ERR_INVALID


def _segs(n=3, **kw):
    base = [dict(k=A16 + (1 + 2 * i) * 64 * MB, v=A16 + (2 + 2 * i) * 64 * MB, len=100 + i, dtype=sdit.SDIT_BF16)
            for i in range(n)]
    for i, s in kw.items():
        base[int(i[1:])].update(s)
    return base


def test_attn_validation():
    q, out, mask = A16, A16 + 1000 * MB, A16 + 2000 * MB

    def v(segs=None, **kw):
        a = dict(q=q, n_q=300, segs=_segs() if segs is None else segs, block_mask=mask, block_q=128, block_k=128,
                 n_heads=12, head_dim=128, out=out, lse=None)
        a.update(kw)
        return sdit.validate_attn_args(**a)

    assert v() == sdit.SDIT_OK
    assert v(lse=A16 + 3000 * MB) == sdit.SDIT_OK
    assert v(block_q=48) == sdit.SDIT_ERR_UNSUPPORTED
    assert v(head_dim=256) == sdit.SDIT_ERR_UNSUPPORTED
    assert v(segs=_segs(9)) == sdit.SDIT_ERR_INVALID
    assert v(segs=[]) == sdit.SDIT_ERR_INVALID
    assert v(segs=_segs(s1=dict(dtype=sdit.SDIT_INT8))) == sdit.SDIT_ERR_INVALID           # int8 without scales
    assert v(segs=_segs(s1=dict(dtype=sdit.SDIT_INT8, k_scale=A16 + 4000 * MB,
                                v_scale=A16 + 4001 * MB))) == sdit.SDIT_OK
    assert v(segs=_segs(s0=dict(k_scale=A16 + 4000 * MB))) == sdit.SDIT_ERR_INVALID        # bf16 with scale
    assert v(segs=_segs(s2=dict(dtype=7))) == sdit.SDIT_ERR_INVALID
    assert v(segs=_segs(s2=dict(len=-1))) == sdit.SDIT_ERR_INVALID
    assert v(segs=_segs(s2=dict(len=0, k=None, v=None))) == sdit.SDIT_OK                   # empty segment
    assert v(segs=_segs(s0=dict(k=A16 + 8))) == sdit.SDIT_ERR_INVALID                      # misaligned
    assert v(block_mask=None) == sdit.SDIT_ERR_INVALID
    assert v(out=q + 4096) == sdit.SDIT_ERR_INVALID                                       # out overlaps q
    assert v(out=_segs()[1]["k"] + 256) == sdit.SDIT_ERR_INVALID                          # out overlaps K
    assert v(lse=A16 + 3000 * MB + 2) == sdit.SDIT_ERR_INVALID
    assert v(n_q=0, q=None, out=None, block_mask=None) == sdit.SDIT_OK
    assert v(n_q=-1) == sdit.SDIT_ERR_INVALID
    assert v(n_heads=0) == sdit.SDIT_ERR_INVALID
    assert v(softmax_scale=float("nan")) == sdit.SDIT_ERR_INVALID
    assert v(softmax_scale=2.0 ** -41) == sdit.SDIT_ERR_INVALID    # the -1e30 mask bias would surface
    assert v(softmax_scale=2.0 ** -40) == sdit.SDIT_OK
    assert v(softmax_scale=-1.0) == sdit.SDIT_OK                   # selects 1/sqrt(head_dim)
    assert "segment 1" in (v(segs=_segs(s1=dict(dtype=sdit.SDIT_INT8))), sdit.last_error())[1]


def test_attn_balanced_validation():
    q, out, mask = A16, A16 + 1000 * MB, A16 + 2000 * MB
    ws = A16 + (1 << 40)
    need = sdit.attn_workspace_bytes(128)
    assert need == 8 * 31 * 2 * 256 * 129 * 4          # SDIT_ATTN_WORKSPACE_BYTES(128)
    header = open(HEADER).read()
    assert "#define SDIT_ATTN_WORKSPACE_BYTES(head_dim) ((int64_t)8 * 31 * 2 * 256 * ((head_dim) + 1) * 4)" in header

    def v(segs=None, **kw):
        a = dict(q=q, n_q=300, segs=_segs() if segs is None else segs, block_mask=mask, block_q=128, block_k=128,
                 n_heads=12, head_dim=128, out=out, lse=None, workspace=ws, workspace_bytes=need, split_tile=-1)
        a.update(kw)
        return sdit.validate_attn_balanced_args(**a)

    n_tiles = sum(-(-sg["len"] // 64) for sg in _segs())
    assert v() == sdit.SDIT_OK
    assert v(split_tile=0) == sdit.SDIT_OK
    assert v(split_tile=n_tiles - 1) == sdit.SDIT_OK
    assert v(split_tile=n_tiles) == sdit.SDIT_ERR_INVALID           # no tail piece left
    assert v(split_tile=-2) == sdit.SDIT_ERR_INVALID
    assert v(workspace_bytes=need - 1) == sdit.SDIT_ERR_INVALID
    assert v(workspace=None) == sdit.SDIT_ERR_INVALID
    assert v(workspace=ws + 8) == sdit.SDIT_ERR_INVALID               # misaligned
    assert v(workspace=out - 4096) == sdit.SDIT_ERR_INVALID           # overlaps out
    assert v(workspace=q) == sdit.SDIT_ERR_INVALID                    # overlaps q
    assert v(lse=ws + need - 64) == sdit.SDIT_ERR_INVALID             # lse inside the workspace
    assert v(workspace=_segs()[2]["v"] - 1024) == sdit.SDIT_ERR_INVALID   # overlaps a segment's V
    assert v(workspace=mask - need + 16) == sdit.SDIT_ERR_INVALID     # ends inside the block mask
    assert v(workspace=mask - need) == sdit.SDIT_OK                   # ends where the mask starts
    assert v(head_dim=80) == sdit.SDIT_ERR_UNSUPPORTED                # the attention checks come first
    assert v(n_q=0, q=None, out=None, block_mask=None, workspace=None) == sdit.SDIT_OK
    assert "workspace" in (v(workspace_bytes=16), sdit.last_error())[1]


def test_balanced_plan():
    """The cut rule: on an XCD of C CUs with r units past its last full wave,
    the r tail pieces take ceil(r / (C - r)) rounds on the free CUs, so the
    head piece gets t = ceil(rounds (n + 3) / (rounds + 1)) of the n key
    tiles; no cut when every XCD's units fill whole waves, when some XCD's
    partial wave keeps more than 3/4 of its CUs busy, or when the cut would
    save fewer than 8 tiles or under 5% of the XCD's run. Values for a
    256-CU device (8 XCDs of 32) worked out by hand."""
    plan = sdit.attn_balanced_plan
    # Wan chunk: 19 q-tiles x 12 heads = 228 units -> 29 or 28 per XCD, none full:
    # 29 of 32 CUs busy, more than 3/4, so no cut
    assert plan(4680, 12, 302, 256) == (0, 228)
    # forced, it would take 29 + 29 workgroups on the busiest XCD
    assert plan(4680, 12, 302, 256, split_tile=278) == (278, 8 * (29 + 29))
    # Large-DiT: 13 x 32 = 416 units -> 52 per XCD = one full wave + 20; 12 free CUs: 2 rounds;
    # 78 tiles -> t = ceil(2 * 81 / 3) = 54
    assert plan(3120, 32, 78, 256) == (54, 8 * (52 + 20))
    # SR: 137 x 12 = 1644 units -> 206 or 205 per XCD = 6 waves + 14 or 13; one round; 545 tiles -> 274
    assert plan(34848, 12, 545, 256) == (274, 8 * (206 + 14))
    # exactly whole waves: nothing to cut, one workgroup per unit
    assert plan(256 * 32, 8, 300, 256) == (0, 256)
    # 31 of 32 CUs busy: no cut
    assert plan(256 * 31, 8, 100, 256) == (0, 248)
    # 24 of 32 busy (exactly 3/4): 3 rounds, 200 tiles -> t = ceil(3 * 203 / 4) = 153
    assert plan(256 * 24, 8, 200, 256) == (153, 8 * 48)
    # one unit of 10 tiles: the tail piece would be under 8 tiles
    assert plan(100, 1, 10, 256) == (0, 1)
    # a forced cut is taken as given wherever a partial wave exists
    assert plan(300, 2, 10, 256, split_tile=4) == (4, 8 * 2)
    assert plan(300, 2, 10, 256, split_tile=0) == (0, 4)
    with pytest.raises(RuntimeError):
        plan(300, 2, 10, 256, split_tile=10)


def test_attn_partial_validation():
    q, out, mask, lse = A16, A16 + 1000 * MB, A16 + 2000 * MB, A16 + 3000 * MB

    def v(**kw):
        a = dict(q=q, n_q=300, segs=_segs(), block_mask=mask, block_q=128, block_k=128, n_heads=12, head_dim=128,
                 out=out, lse=lse)
        a.update(kw)
        return sdit.validate_attn_partial_args(**a)

    assert v() == sdit.SDIT_OK
    assert v(lse=None) == sdit.SDIT_ERR_INVALID                                           # lse required
    # fp32 output is twice the bf16 size: placed just below q, a bf16 out would end at q, an fp32 one overlaps it
    q_hi = A16 + 8 * MB
    assert v(q=q_hi, out=q_hi - 300 * 12 * 128 * 2) == sdit.SDIT_ERR_INVALID
    assert v(lse=out + 300 * 12 * 128 * 4 - 64) == sdit.SDIT_ERR_INVALID                  # lse overlaps fp32 out
    assert v(lse=out + 300 * 12 * 128 * 4) == sdit.SDIT_OK
    assert v(head_dim=96) == sdit.SDIT_ERR_UNSUPPORTED
    assert v(n_q=0, q=None, out=None, block_mask=None, lse=None) == sdit.SDIT_OK
    assert "attn_fwd_partial" in (v(lse=None), sdit.last_error())[1]


def test_attn_merge_validation():
    n_q, H, d = 300, 12, 128
    fbytes, lbytes = n_q * H * d * 4, n_q * H * 4
    parts = [A16 + i * 64 * MB for i in range(3)]
    lses = [A16 + 512 * MB + i * MB for i in range(3)]
    out, lse_out = A16 + 1024 * MB, A16 + 1100 * MB

    def v(**kw):
        a = dict(o_parts=parts, lse_parts=lses, n_q=n_q, n_heads=H, head_dim=d, out=out, lse_out=lse_out)
        a.update(kw)
        return sdit.validate_attn_merge_args(**a)

    assert v() == sdit.SDIT_OK
    assert v(lse_out=None) == sdit.SDIT_OK
    assert v(o_parts=[], lse_parts=[]) == sdit.SDIT_ERR_INVALID
    assert v(o_parts=parts * 3, lse_parts=lses * 3) == sdit.SDIT_ERR_INVALID               # 9 > 8 parts
    assert v(o_parts=[parts[0]] * 8, lse_parts=[lses[0]] * 8) == sdit.SDIT_OK
    assert v(o_parts=[parts[0], None, parts[2]]) == sdit.SDIT_ERR_INVALID
    assert v(o_parts=[parts[0] + 8, parts[1], parts[2]]) == sdit.SDIT_ERR_INVALID         # misaligned
    assert v(lse_parts=[lses[0], lses[1] + 2, lses[2]]) == sdit.SDIT_ERR_INVALID
    assert v(out=parts[1] + fbytes - 64) == sdit.SDIT_ERR_INVALID                         # out overlaps a part
    assert v(lse_out=lses[2] + lbytes - 4) == sdit.SDIT_ERR_INVALID                       # lse_out overlaps
    assert v(lse_out=out + n_q * H * d * 2 - 4) == sdit.SDIT_ERR_INVALID                  # lse_out overlaps out
    assert v(head_dim=80) == sdit.SDIT_ERR_UNSUPPORTED
    assert v(n_heads=0) == sdit.SDIT_ERR_INVALID
    assert v(n_q=0, out=None) == sdit.SDIT_OK
    assert "part 1" in (v(o_parts=[parts[0], None, parts[2]]), sdit.last_error())[1]


def test_window_permute_validation():
    x, y = A16, A16 + 256 * MB            # 2 x 96 x 168 tokens x 12 heads x 128 bf16 = 99 MB each

    def v(**kw):
        a = dict(x=x, y=y, T=2, Hl=96, Wl=168, n_heads=12, head_dim=128, window=8, inverse=False)
        a.update(kw)
        return sdit.validate_window_permute_args(**a)

    assert v() == sdit.SDIT_OK
    assert v(inverse=True) == sdit.SDIT_OK
    assert v(Wl=164) == sdit.SDIT_ERR_INVALID            # not whole windows
    assert v(window=6) == sdit.SDIT_ERR_UNSUPPORTED
    assert v(head_dim=96) == sdit.SDIT_ERR_UNSUPPORTED
    assert v(y=x + 1024) == sdit.SDIT_ERR_INVALID         # overlap (no in-place reordering)
    assert v(y=y + 8) == sdit.SDIT_ERR_INVALID            # misaligned
    assert v(x=None) == sdit.SDIT_ERR_INVALID
    assert v(T=0, x=None, y=None) == sdit.SDIT_OK
    assert v(n_heads=0) == sdit.SDIT_ERR_INVALID


def test_norm_validation():
    x, y = A16, A16 + 512 * MB            # 32760 tokens x 5120 bf16 = 335 MB each
    g, sh = A16 + 1024 * MB, A16 + 1025 * MB

    def rms(**kw):
        a = dict(x=x, y=y, gamma=g, n_tok=32760, dim=5120, eps=1e-6)
        a.update(kw)
        return sdit.validate_rmsnorm_args(**a)

    def ln(**kw):
        a = dict(x=x, y=y, scale=g, shift=sh, n_tok=32760, dim=5120, eps=1e-6)
        a.update(kw)
        return sdit.validate_layernorm_modulate_args(**a)

    for v in (rms, ln):
        assert v() == sdit.SDIT_OK
        assert v(y=x) == sdit.SDIT_OK                    # exact in place
        assert v(y=x + 1024) == sdit.SDIT_ERR_INVALID    # partial overlap
        assert v(y=y + 8) == sdit.SDIT_ERR_INVALID       # misaligned
        assert v(x=None) == sdit.SDIT_ERR_INVALID
        assert v(dim=5124) == sdit.SDIT_ERR_UNSUPPORTED  # not a multiple of 8
        assert v(dim=8200) == sdit.SDIT_ERR_UNSUPPORTED  # above SDIT_MAX_NORM_DIM
        assert v(dim=8192) == sdit.SDIT_OK
        assert v(dim=0) == sdit.SDIT_ERR_UNSUPPORTED
        assert v(n_tok=-1) == sdit.SDIT_ERR_INVALID
        assert v(n_tok=1 << 26) == sdit.SDIT_ERR_INVALID
        assert v(n_tok=0, x=None, y=None) == sdit.SDIT_OK
        assert v(eps=-1.0) == sdit.SDIT_ERR_INVALID
        assert v(eps=float("nan")) == sdit.SDIT_ERR_INVALID
    assert rms(gamma=None) == sdit.SDIT_ERR_INVALID
    assert rms(gamma=g + 4) == sdit.SDIT_ERR_INVALID
    assert rms(gamma=y + 4096) == sdit.SDIT_ERR_INVALID  # output overlaps gamma
    assert ln(shift=None) == sdit.SDIT_ERR_INVALID
    assert ln(scale=y) == sdit.SDIT_ERR_INVALID
    assert "layernorm_modulate" in (ln(dim=12), sdit.last_error())[1]


def test_extreme_sizes_are_rejected_not_wrapped():
    """Sizes near the int32 limits: each product of dimensions is formed
    without overflow and compared with its limit, so a huge request is
    rejected instead of wrapping into a small, valid-looking size."""
    I32 = 2**31 - 1
    far = [A16 + (i << 44) for i in range(1, 8)]        # disjoint fake buffers, 16 TB apart
    INV, UNS, OK = sdit.SDIT_ERR_INVALID, sdit.SDIT_ERR_UNSUPPORTED, sdit.SDIT_OK

    def qk(T, Hl, Wl, n_heads):
        return sdit.validate_qknorm_rope3d_args(A16, A16, far[0], far[1], far[2], far[3], T, Hl, Wl, 0,
                                                n_heads, 128, 44, 42, 42)
    assert qk(I32, I32, I32, 1) == INV                   # T * Hl * Wl past 2^63
    assert qk(65536, 65536, 0, 12) == OK                 # T * Hl alone past int32, but no tokens
    assert qk(1 << 15, 1 << 15, 1, 12) == INV            # 2^30 tokens x 12 heads x 128 > 2^40 elements
    assert qk(16, 16, 16, I32) == INV                    # head count that would wrap the byte size
    assert sdit.validate_kv_quant_args(A16, far[0], far[1], I32, I32, 128) == INV
    assert sdit.validate_kv_quant_args(A16, far[0], far[1], 1 << 20, 1 << 13, 128) == OK   # exactly 2^40
    assert sdit.validate_kv_quant_args(A16, far[0], far[1], 1 << 20, (1 << 13) + 1, 128) == INV

    def wp(T, Hl, Wl, n_heads):
        return sdit.validate_window_permute_args(A16, far[0], T, Hl, Wl, n_heads, 128, 8, False)
    assert wp(I32, 1 << 24, 1 << 24, 1) == INV           # T * Hl * Wl past 2^63
    assert wp(1, 64, 64, I32) == UNS                     # row of n_heads * head_dim wider than 2^24
    assert wp(1 << 14, 128, 128, 4096) == INV            # 2^28 tokens x 2^19 per token > 2^40 elements
    assert wp(0, 1 << 20, 1 << 20, 12) == OK
    assert sdit.validate_attn_merge_args([far[0]], [far[1]], I32, I32, 128, far[2], far[3]) == INV
    assert sdit.validate_attn_merge_args([far[0]], [far[1]], 1 << 24, 1 << 9, 128, far[2], far[3]) == OK

    huge = sdit.make_segments([dict(k=A16, v=A16, len=I32)])
    assert sdit.validate_attn_args(far[0], 4096, huge, far[1], 128, 128, 12, 128, far[2], None) == UNS
    assert sdit.validate_attn_args(far[0], I32, huge, far[1], 16, 16, 1 << 16, 128, far[2], None) == INV


def test_error_message_is_per_call():
    sdit.validate_kv_quant_args(A16, A16 + 8, A16 + 32 * MB, 100, 12, 128)
    assert sdit.last_error() != ""
    sdit.validate_kv_quant_args(A16, A16 + 16 * MB, A16 + 32 * MB, 100, 12, 128)
    assert sdit.last_error() == ""


def test_product_path_does_not_touch_the_oracle():
    import sys
    import subprocess
    code = ("import sys, streaming_video_dit_amd as s; s.lib(); "
            "assert not any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules), sorted(sys.modules)")
    subprocess.run([sys.executable, "-c", code], check=True, cwd=ROOT)
    src = open(os.path.join(ROOT, "streaming_video_dit_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("oracle-free", "")
