"""The C-ABI library on the CPU: it loads, exports what the header declares, and rejects
bad arguments before any HIP call (so no GPU is needed and nothing is launched)."""
import ctypes

import pytest

import paged_kv_attention_causal_amd as pk

EINVAL, EUNSUP, EWS = 1, 2, 3
P = ctypes.c_void_p(4096)     # a non-null pointer that is never dereferenced
NULL = None


@pytest.fixture(scope="module")
def L():
    return pk.lib()


def test_library_exports_every_declared_symbol(L):
    names = pk.header_symbols()
    assert {"attn_prefill", "attn_decode_contig", "attn_decode_paged", "mla_decode_latent",
            "attn_decode_workspace_size", "mla_decode_workspace_size", "pkva_status_string",
            "pkva_version"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.pkva_version().decode().startswith("pkvattn")
    assert L.pkva_status_string(0) == b"ok"
    assert L.pkva_status_string(2) == b"unsupported dtype or size"
    assert L.pkva_status_string(99) == b"unknown status"


def _prefill(L, **kw):
    a = dict(dtype=1, q=P, k=P, v=P, o=P, batch=1, n_heads=28, n_kv_heads=4, head_dim=128,
             seq_q=64, seq_kv=64, off=0, scale=0.088, bt=NULL, maxb=0, bs=0, nb=0, cap=64)
    a.update(kw)
    return L.attn_prefill(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["batch"], a["n_heads"],
                          a["n_kv_heads"], a["head_dim"], a["seq_q"], a["seq_kv"], a["off"],
                          a["scale"], a["bt"], a["maxb"], a["bs"], a["nb"], a["cap"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), EUNSUP),               # not fp32/bf16: rejected like a non-f32 input
    (dict(dtype=-1), EUNSUP),
    (dict(q=NULL), EINVAL),
    (dict(o=NULL), EINVAL),
    (dict(n_kv_heads=3), EINVAL),          # does not divide n_heads
    (dict(n_kv_heads=0), EINVAL),
    (dict(n_heads=0), EINVAL),
    (dict(batch=0), EINVAL),
    (dict(seq_q=0), EINVAL),
    (dict(seq_kv=0), EINVAL),
    (dict(off=-1), EINVAL),
    (dict(scale=float("nan")), EINVAL),
    (dict(scale=float("inf")), EINVAL),
    (dict(scale=-0.5), EINVAL),
    (dict(cap=63), EINVAL),                # contiguous cache shorter than seq_kv
    (dict(bt=P, maxb=4, bs=12, nb=10), EINVAL),   # block size not a power of two
    (dict(bt=P, maxb=3, bs=16, nb=10), EINVAL),   # table too short for seq_kv
    (dict(bt=P, maxb=4, bs=16, nb=0), EINVAL),
    (dict(head_dim=64), EUNSUP),           # not built
    # cache and pool rows are indexed in 31 bits
    (dict(batch=2, cap=(1 << 30) + 1, seq_kv=64), EINVAL),
    (dict(bt=P, maxb=4, bs=16, nb=(1 << 27)), EINVAL),
    (dict(dtype=0, head_dim=128), EUNSUP),
    (dict(dtype=1, head_dim=16), EUNSUP),
])
def test_prefill_validation(L, kw, code):
    assert _prefill(L, **kw) == code


def _decode(L, paged, **kw):
    a = dict(dtype=1, q=P, k=P, v=P, o=P, batch=4, n_heads=32, n_kv_heads=8, head_dim=128,
             bt=P, maxb=8, bs=16, nb=100, lens=P, cap=128, maxlen=128, scale=0.088,
             ws=P, wsb=1 << 30)
    a.update(kw)
    if paged:
        return L.attn_decode_paged(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["batch"],
                                   a["n_heads"], a["n_kv_heads"], a["head_dim"], a["bt"], a["maxb"],
                                   a["bs"], a["nb"], a["lens"], a["maxlen"], a["scale"], a["ws"],
                                   a["wsb"], NULL)
    return L.attn_decode_contig(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["batch"],
                                a["n_heads"], a["n_kv_heads"], a["head_dim"], a["lens"], a["cap"],
                                a["maxlen"], a["scale"], a["ws"], a["wsb"], NULL)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("kw,code", [
    (dict(dtype=5), EUNSUP),
    (dict(lens=NULL), EINVAL),
    (dict(k=NULL), EINVAL),
    (dict(maxlen=0), EINVAL),
    (dict(n_kv_heads=5), EINVAL),
    (dict(n_heads=64, n_kv_heads=4), EUNSUP),     # group of 16 is not packed
    (dict(head_dim=96), EUNSUP),
    (dict(ws=NULL), EWS),
    (dict(wsb=16), EWS),
    (dict(ws=ctypes.c_void_p(4100)), EWS),        # workspace not 16-byte aligned
    (dict(scale=float("nan")), EINVAL),
])
def test_decode_validation(L, paged, kw, code):
    assert _decode(L, paged, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(bt=NULL), EINVAL),
    (dict(bs=24), EINVAL),
    (dict(maxb=7), EINVAL),        # 7 * 16 < max_seq_len 128
    (dict(nb=0), EINVAL),
])
def test_paged_decode_table_validation(L, kw, code):
    assert _decode(L, True, **kw) == code


def test_contig_decode_capacity_validation(L):
    assert _decode(L, False, cap=127) == EINVAL


def test_decode_workspace_size_formula(L):
    # slots = ranges + batch, ranges <= min(2048, ceil(batch * max_seq_len / 64));
    # per slot and head: head_dim + 2 floats; then batch + 2 int32 prefix sums
    def expect(B, H, D, maxlen):
        ranges = min(2048, -(-B * maxlen // 64))
        return (ranges + B) * H * (D + 2) * 4 + (B + 2) * 4
    assert L.attn_decode_workspace_size(64, 32, 8, 128, 8192) == expect(64, 32, 128, 8192)
    assert expect(64, 32, 128, 8192) == 2112 * 32 * 130 * 4 + 66 * 4
    assert L.attn_decode_workspace_size(1, 4, 2, 16, 72) == expect(1, 4, 16, 72) == 3 * 4 * 18 * 4 + 12
    assert L.attn_decode_workspace_size(1, 4, 3, 16, 72) == 0     # invalid heads
    assert L.attn_decode_workspace_size(0, 4, 2, 16, 72) == 0


def _mla(L, **kw):
    a = dict(dtype=1, q=P, lat=P, o=P, batch=32, n_heads=128, R=512, Pr=64, lens=P, cap=4096,
             maxlen=4096, scale=0.072, ws=P, wsb=1 << 30)
    a.update(kw)
    return L.mla_decode_latent(a["dtype"], a["q"], a["lat"], a["o"], a["batch"], a["n_heads"],
                               a["R"], a["Pr"], a["lens"], a["cap"], a["maxlen"], a["scale"],
                               a["ws"], a["wsb"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), EUNSUP),
    (dict(dtype=3), EUNSUP),
    (dict(R=256), EUNSUP),
    (dict(Pr=32), EUNSUP),
    (dict(n_heads=200), EUNSUP),          # above 128 and not a multiple of 128
    (dict(q=NULL), EINVAL),
    (dict(cap=100), EINVAL),
    (dict(maxlen=0), EINVAL),
    (dict(scale=-1.0), EINVAL),
    (dict(batch=1, ws=NULL), EWS),         # small batch splits the context: needs a workspace
])
def test_mla_validation(L, kw, code):
    assert _mla(L, **kw) == code


def test_mla_workspace_size(L):
    # One workgroup serves up to 128 heads of a sequence; the context is split
    # until about 256 workgroups run, in pieces that are whole 32-token tiles.
    # Per piece and head: 512 bf16 (O / l) + max and sum in fp32.
    per = 512 * 2 + 8
    # 32 sequences x 1 head group -> 8 pieces of 512 tokens
    assert L.mla_decode_workspace_size(32, 128, 512, 4096) == 32 * 8 * 128 * per
    # one sequence -> 128 pieces of 32 tokens (the tile)
    assert L.mla_decode_workspace_size(1, 128, 512, 4096) == 1 * 128 * 128 * per
    # 256 sequences fill the GPU unsplit: no workspace
    assert L.mla_decode_workspace_size(256, 128, 512, 4096) == 0
    # any head count up to 128 (one workgroup of 128 heads, the rest idle)
    assert L.mla_decode_workspace_size(1, 100, 512, 4096) == 1 * 128 * 100 * per
    assert L.mla_decode_workspace_size(1, 0, 512, 4096) == 0
    assert L.mla_decode_workspace_size(1, 160, 512, 4096) == 0   # above 128, not a multiple


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 16)
    with pytest.raises(ValueError):
        pk.attn_decode_contig(q, torch.zeros(1, 8, 2, 16), torch.zeros(1, 8, 2, 16),
                              torch.ones(1, dtype=torch.int32), max_seq_len=8, attention_scale=0.25)


# ---------------------------------------------------------------- ragged prefill, push, arms

def _varlen(L, **kw):
    a = dict(dtype=1, q=P, k=P, v=P, o=P, batch=4, n_heads=32, n_kv_heads=8, head_dim=128,
             cu=P, skv=P, total_q=100, max_q=64, scale=0.088, bt=P, maxb=8, bs=16, nb=40, cap=0)
    a.update(kw)
    return L.attn_prefill_varlen(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["batch"],
                                 a["n_heads"], a["n_kv_heads"], a["head_dim"], a["cu"], a["skv"],
                                 a["total_q"], a["max_q"], a["scale"], a["bt"], a["maxb"], a["bs"],
                                 a["nb"], a["cap"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), EUNSUP),
    (dict(cu=NULL), EINVAL),
    (dict(skv=NULL), EINVAL),
    (dict(total_q=0), EINVAL),
    (dict(max_q=0), EINVAL),
    (dict(n_kv_heads=5), EINVAL),
    (dict(scale=-1.0), EINVAL),
    (dict(bs=12), EINVAL),
    (dict(nb=(1 << 27)), EINVAL),              # pool rows beyond 31 bits
    (dict(bt=NULL, cap=0), EINVAL),           # contiguous without a capacity
    (dict(bt=NULL, batch=3, cap=(1 << 30)), EINVAL),
    (dict(head_dim=64), EUNSUP),
])
def test_prefill_varlen_validation(L, kw, code):
    assert _varlen(L, **kw) == code


def _append(L, **kw):
    a = dict(dtype=1, kn=P, vn=P, kc=P, vc=P, batch=2, hkv=8, d=128, n_new=1, pos=P, bt=P, maxb=4,
             bs=16, nb=10, cap=0)
    a.update(kw)
    return L.kv_append(a["dtype"], a["kn"], a["vn"], a["kc"], a["vc"], a["batch"], a["hkv"], a["d"],
                       a["n_new"], a["pos"], a["bt"], a["maxb"], a["bs"], a["nb"], a["cap"], NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=4), EUNSUP),
    (dict(kn=NULL), EINVAL),
    (dict(pos=NULL), EINVAL),
    (dict(n_new=0), EINVAL),
    (dict(d=0), EINVAL),
    (dict(bs=6), EINVAL),
    (dict(nb=0), EINVAL),
    (dict(bt=NULL, cap=0), EINVAL),
])
def test_kv_append_validation(L, kw, code):
    assert _append(L, **kw) == code


def _mla_append(L, **kw):
    a = dict(dtype=1, c=P, kr=P, lat=P, batch=2, R=512, Pr=64, pos=P, theta=1e4, bt=NULL, maxb=0,
             bs=0, nb=0, cap=10)
    a.update(kw)
    return L.mla_append_latent(a["dtype"], a["c"], a["kr"], a["lat"], a["batch"], a["R"], a["Pr"],
                               a["pos"], a["theta"], a["bt"], a["maxb"], a["bs"], a["nb"], a["cap"],
                               NULL)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=9), EUNSUP),
    (dict(c=NULL), EINVAL),
    (dict(kr=NULL), EINVAL),
    (dict(Pr=63), EINVAL),                  # the rotary width pairs entries
    (dict(theta=float("nan")), EINVAL),
    (dict(cap=0), EINVAL),
    (dict(bt=P, maxb=2, bs=3, nb=4), EINVAL),
])
def test_mla_append_validation(L, kw, code):
    assert _mla_append(L, **kw) == code


def _ext(L, paged, arms, **kw):
    a = dict(dtype=1, q=P, k=P, v=P, o=P, batch=4, n_heads=32, n_kv_heads=8, head_dim=128,
             bt=P, maxb=8, bs=16, nb=100, lens=P, cap=128, maxlen=128, scale=0.088,
             ws=P, wsb=1 << 30)
    a.update(kw)
    ap = None if arms is None else ctypes.byref(arms)
    if paged:
        return L.attn_decode_paged_ext(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["batch"],
                                       a["n_heads"], a["n_kv_heads"], a["head_dim"], a["bt"],
                                       a["maxb"], a["bs"], a["nb"], a["lens"], a["maxlen"],
                                       a["scale"], ap, a["ws"], a["wsb"], NULL)
    return L.attn_decode_contig_ext(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["batch"],
                                    a["n_heads"], a["n_kv_heads"], a["head_dim"], a["lens"],
                                    a["cap"], a["maxlen"], a["scale"], ap, a["ws"], a["wsb"], NULL)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("arms,kw,code", [
    (None, {}, EINVAL),                                        # the arms are required
    (pk.Arms(-1, 0.0, None, None, 0), {}, EINVAL),             # negative window
    (pk.Arms(0, -2.0, None, None, 0), {}, EINVAL),             # negative softcap
    (pk.Arms(0, float("inf"), None, None, 0), {}, EINVAL),
    (pk.Arms(0, 0.0, None, None, -4), {}, EINVAL),
    (pk.Arms(0, 0.0, None, None, 64), {}, EUNSUP),            # V width not built
    (pk.Arms(0, 0.0, None, None, 128), dict(head_dim=256), EUNSUP),
    (pk.Arms(8, 1.0, None, None, 128), dict(ws=NULL), EWS),
])
def test_decode_ext_validation(L, paged, arms, kw, code):
    assert _ext(L, paged, arms, **kw) == code


def test_noalloc_validation_before_any_hip_call(L):
    # pure argument errors come back before the scratch lookup
    assert L.attn_decode_paged_noalloc(1, P, P, P, P, 4, 32, 5, 128, P, 8, 16, 100, P, 128, 0.1,
                                       NULL) == EINVAL
    assert L.attn_decode_paged_noalloc(1, P, P, P, P, 4, 32, 8, 128, NULL, 8, 16, 100, P, 128, 0.1,
                                       NULL) == EINVAL
    # sizes beyond the 64 MiB scratch: (2048 + 4096) x 32 x 130 x 4 B
    assert L.attn_decode_paged_noalloc(1, P, P, P, P, 4096, 32, 8, 128, P, 512, 16, 1000, P, 8192,
                                       0.1, NULL) == 5


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), EUNSUP),               # bf16 only
    (dict(q=NULL), EINVAL),
    (dict(nope=120), EUNSUP),
    (dict(R=500), EUNSUP),
    (dict(Pr=6), EUNSUP),
    (dict(batch=0), EINVAL),
    (dict(q=ctypes.c_void_p(4104)), EINVAL),   # not 16-byte aligned
])
def test_mla_absorb_validation(L, kw, code):
    a = dict(dtype=1, q=P, kb=P, qa=P, batch=4, H=16, nope=128, Pr=64, R=512)
    a.update(kw)
    assert L.mla_absorb_q(a["dtype"], a["q"], a["kb"], a["qa"], a["batch"], a["H"], a["nope"],
                          a["Pr"], a["R"], NULL) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=0), EUNSUP),
    (dict(vb=NULL), EINVAL),
    (dict(vd=100), EUNSUP),
    (dict(R=520), EUNSUP),
    (dict(H=0), EINVAL),
])
def test_mla_up_proj_validation(L, kw, code):
    a = dict(dtype=1, o=P, vb=P, out=P, batch=4, H=16, R=512, vd=128)
    a.update(kw)
    assert L.mla_up_proj(a["dtype"], a["o"], a["vb"], a["out"], a["batch"], a["H"], a["R"],
                         a["vd"], NULL) == code


@pytest.mark.parametrize("kw,code", [
    (dict(bt=NULL), EINVAL),
    (dict(bs=24), EINVAL),
    (dict(maxb=100), EINVAL),              # 100 x 16 < max_seq_len 4096
    (dict(nb=(1 << 27)), EINVAL),
])
def test_mla_paged_validation(L, kw, code):
    a = dict(dtype=1, q=P, lat=P, o=P, batch=32, H=128, R=512, Pr=64, bt=P, maxb=256, bs=16,
             nb=9000, lens=P, maxlen=4096, scale=0.072, ws=P, wsb=1 << 30)
    a.update(kw)
    assert L.mla_decode_latent_paged(a["dtype"], a["q"], a["lat"], a["o"], a["batch"], a["H"],
                                     a["R"], a["Pr"], a["bt"], a["maxb"], a["bs"], a["nb"],
                                     a["lens"], a["maxlen"], a["scale"], a["ws"], a["wsb"],
                                     NULL) == code
