"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

import stream_decode_attention_amd as sda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "decattn.h")


def _ensure_built():
    if not os.path.exists(sda.LIB_PATH):
        from stream_decode_attention_amd.build import build_library
        build_library()


@pytest.fixture(scope="module")
def lib():
    _ensure_built()
    return sda.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:int|size_t|const char\s*\*)\s*(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_boundary():
    names = set(declared_functions())
    assert {"decode_attn", "decode_attn_noalloc", "chunk_attn", "attn_partial", "attn_merge", "decattn_workspace_bytes",
            "decattn_default_chunk", "decattn_status_str", "decattn_abi_version",
            "decattn_probe_read", "decattn_probe_copy", "rope_kv_write", "prefill_attn",
            "gemv_bf16", "gemv_int8", "quantize_rows_int8", "spec_accept",
            "spec_accept_workspace_bytes"} <= names


def test_every_declared_symbol_is_exported(lib):
    raw = ctypes.CDLL(sda.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name
    # and the binding knows a signature for every one of them
    assert set(declared_functions()) == set(sda._SIGNATURES)


def test_version_and_status_strings(lib):
    assert sda.abi_version() == 1
    assert sda.status_str(0) == "ok"
    for s in (1, 2, 3, 4, 99, -1):
        assert isinstance(sda.status_str(s), str) and sda.status_str(s)


def _ws(B, T, Hq, Hkv, D, S, C):
    NC = -(-S // C)
    rows = B * Hkv * NC * T * (Hq // Hkv)
    up = lambda x: -(-x // 256) * 256
    return up(rows * 2 * 4) + up(rows * D * 4)


@pytest.mark.parametrize("shape", [
    (1, 1, 15, 5, 64, 128, 32), (8, 1, 32, 8, 128, 32768, 256), (1, 6, 24, 8, 128, 16384, 64),
    (2, 3, 4, 4, 64, 100, 16), (1, 1, 8, 1, 128, 50, 1024),
])
def test_workspace_bytes_formula(lib, shape):
    B, T, Hq, Hkv, D, S, C = shape
    assert sda.workspace_bytes(B, T, Hq, Hkv, D, S, C) == _ws(B, T, Hq, Hkv, D, S, C)


def test_default_chunk_is_supported_power_of_two(lib):
    for shape in [(1, 1, 15, 5, 64, 128), (1, 1, 15, 5, 64, 4096), (1, 1, 32, 4, 64, 8192),
                  (8, 1, 32, 8, 128, 32768), (1, 6, 24, 8, 128, 16384)]:
        c = sda.default_chunk(*shape)
        assert c >= 16 and c & (c - 1) == 0
        assert sda.workspace_bytes(*shape, 0) == sda.workspace_bytes(*shape, c)


FAKE = 0x100000  # 16-byte aligned, never dereferenced: every call below fails its host checks


def _decode(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, lens=FAKE, B=1, Hq=8, Hkv=2, D=64, S=64, scale=0.125,
             out=FAKE, od=1, ws=FAKE, wsb=1 << 20, chunk=0, stream=None)
    a.update(kw)
    return lib.decode_attn(a["q"], a["k"], a["v"], a["lens"], a["B"], a["Hq"], a["Hkv"], a["D"], a["S"],
                           a["scale"], a["out"], a["od"], a["ws"], a["wsb"], a["chunk"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=9, Hkv=2), 1),                 # Hq not a multiple of Hkv
    (dict(B=0), 1), (dict(S=-1), 1), (dict(Hkv=0), 1),
    (dict(D=96), 2), (dict(D=256), 2),      # head dim
    (dict(Hq=18, Hkv=2), 2),                # G = 9 > 8
    (dict(B=4097), 2),                      # lengths staged in LDS: B <= 4096
    (dict(chunk=48), 2), (dict(chunk=8), 2), (dict(chunk=-32), 2), (dict(chunk=1 << 21), 2),
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(lens=None), 1),
    (dict(out=None), 1), (dict(ws=None), 1),
    (dict(q=FAKE + 2), 1), (dict(k=FAKE + 8), 1), (dict(out=FAKE + 4), 1), (dict(lens=FAKE + 2), 1),
    (dict(od=7), 1),
    (dict(scale=float("nan")), 1), (dict(scale=float("inf")), 1),
    (dict(wsb=16), 3),
])
def test_decode_rejects_bad_arguments(lib, kw, status):
    assert _decode(lib, **kw) == status


@pytest.mark.parametrize("D,refused", [(128, 1 << 24), (64, 1 << 25)])
def test_one_kv_head_must_fit_a_32bit_byte_range(lib, D, refused):
    """The kernels address one kv head's cache with 32-bit byte offsets, so
    (S_max + 512) * D * 2 must stay below 2^32; past it every entry point that
    plans split-KV tiles refuses instead of reading wrapped offsets."""
    largest = (0xFFFFFFFF // (D * 2)) - 512
    for T, Hq, Hkv in ((1, 8, 8), (6, 24, 8)):
        assert sda.workspace_bytes(1, T, Hq, Hkv, D, refused, 0) == 0
        assert sda.default_chunk(1, T, Hq, Hkv, D, refused) == 0
        assert sda.workspace_bytes(1, T, Hq, Hkv, D, largest + 1, 0) == 0
        assert sda.workspace_bytes(1, T, Hq, Hkv, D, largest, 0) > 0
        assert sda.default_chunk(1, T, Hq, Hkv, D, largest) > 0
    assert _decode(lib, B=1, Hq=8, Hkv=8, D=D, S=refused, wsb=1 << 40) == 2
    assert _decode(lib, B=1, Hq=8, Hkv=8, D=D, S=largest + 1, wsb=1 << 40) == 2
    chunk = lambda S: lib.chunk_attn(FAKE, FAKE, FAKE, FAKE, 1, 6, 24, 8, D, S, 0.088, FAKE, 1, FAKE,
                                     1 << 40, 0, None)
    assert chunk(refused) == 2
    part = lambda S: lib.attn_partial(FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 8, D, S, 0.1, 0, FAKE, 1 << 40, 0, None)
    assert part(refused) == 2
    merge = lambda S: lib.attn_merge(FAKE, 1, 1, 8, 8, D, S, 0, FAKE, 1, FAKE, 1 << 40, 0, None)
    assert merge(refused) == 2
    # the largest accepted S_max gets past the shape checks (it then fails on
    # the deliberately tiny workspace, status 3, before anything is launched)
    assert _decode(lib, B=1, Hq=8, Hkv=8, D=D, S=largest, wsb=16) == 3
    assert lib.attn_merge(FAKE, 1, 1, 8, 8, D, largest, 0, FAKE, 1, FAKE, 16, 0, None) == 3
    assert lib.chunk_attn(FAKE, FAKE, FAKE, FAKE, 1, 6, 24, 8, D, largest, 0.088, FAKE, 1, FAKE,
                          16, 0, None) == 3


def test_noalloc_decode_rejects_before_touching_the_device(lib):
    """decode_attn_noalloc checks everything on the host first: bad shapes and
    pointers, and a partial state larger than its static scratch array, return a
    status before the device array is looked up or anything is launched."""
    def call(B=1, Hq=8, Hkv=2, D=64, S=64, q=FAKE, lens=FAKE, out=FAKE, od=1, chunk=0, scale=0.125):
        return lib.decode_attn_noalloc(q, FAKE, FAKE, lens, B, Hq, Hkv, D, S, scale, out, od, chunk, None)
    assert call(Hq=9) == 1 and call(D=96) == 2 and call(q=None) == 1 and call(lens=FAKE + 2) == 1
    assert call(out=FAKE + 4) == 1 and call(od=5) == 1 and call(scale=float("nan")) == 1
    assert call(chunk=48) == 2 and call(S=1 << 24, D=128) == 2
    # B = 8, Hq = 32, S_max = 32768 at 128-key tiles: ~35 MB of partial state
    need = sda.workspace_bytes(8, 1, 32, 8, 128, 32768, 128)
    assert need > sda.NOALLOC_SCRATCH_BYTES
    assert call(B=8, Hq=32, Hkv=8, D=128, S=32768, chunk=128) == 3
    # the headline shape at its default tiles fits
    assert sda.workspace_bytes(8, 1, 32, 8, 128, 32768, 0) <= sda.NOALLOC_SCRATCH_BYTES


def test_chunk_rejects_bad_arguments(lib):
    args = lambda T, wsb=1 << 24: (FAKE, FAKE, FAKE, FAKE, 1, T, 24, 8, 128, 16384, 0.088, FAKE, 1,
                                   FAKE, wsb, 0, None)
    assert lib.chunk_attn(*args(17)) == 2           # T > 16
    assert lib.chunk_attn(*args(0)) == 1
    assert lib.chunk_attn(*args(6, wsb=1024)) == 3


def test_phase_entry_points_reject_bad_arguments(lib):
    # decode (causal = 0) requires T == 1; causal must be 0 or 1
    assert lib.attn_partial(FAKE, FAKE, FAKE, FAKE, 1, 2, 8, 2, 64, 64, 0.1, 0, FAKE, 1 << 20, 0, None) == 1
    assert lib.attn_partial(FAKE, FAKE, FAKE, FAKE, 1, 1, 8, 2, 64, 64, 0.1, 2, FAKE, 1 << 20, 0, None) == 1
    assert lib.attn_merge(FAKE, 1, 1, 8, 2, 64, 64, 0, FAKE, 1, FAKE, 16, 0, None) == 3
    assert lib.attn_merge(None, 1, 1, 8, 2, 64, 64, 0, FAKE, 1, FAKE, 1 << 20, 0, None) == 1


def test_probes_reject_bad_arguments(lib):
    assert lib.decattn_probe_read(FAKE, 100, FAKE, None) == 1      # not a multiple of 16
    assert lib.decattn_probe_read(None, 1024, FAKE, None) == 1
    assert lib.decattn_probe_copy(FAKE, FAKE + 8, 1024, None) == 1


# rope_kv_write: every case below fails a host check, so nothing is launched.
# Disjoint fake addresses for a B=2, T=3, Hq=8, Hkv=2, D=64, S_max=64 step.
_ROPE_PTRS = dict(q=0x1000000, k=0x2000000, v=0x3000000, pos=0x4000000, qo=0x1000000,
                  kc=0x5000000, vc=0x6000000)


def _rope(lib, rope=None, **kw):
    a = dict(_ROPE_PTRS, B=2, T=3, Hq=8, Hkv=2, D=64, S=64)
    a.update(kw)
    r = rope if rope is not None else sda.rope_params(10000.0)
    rp = ctypes.byref(r) if r is not False else None
    return lib.rope_kv_write(a["q"], a["k"], a["v"], a["pos"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"],
                             a["S"], rp, a["qo"], a["kc"], a["vc"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(pos=None), 1), (dict(qo=None), 1),
    (dict(kc=None), 1), (dict(vc=None), 1),
    (dict(B=0), 1), (dict(T=0), 1), (dict(Hq=0), 1), (dict(S=0), 1), (dict(Hq=9), 1),
    (dict(D=96), 2), (dict(D=256), 2), (dict(S=0x7FFFFFFF), 2),
    (dict(q=0x1000008, qo=0x1000008), 1), (dict(pos=0x4000002), 1), (dict(kc=0x5000004), 1),
    (dict(qo=0x1000010), 1),                    # q_out overlaps q_in without being it
    (dict(vc=0x5000000), 1),                    # the two caches overlap
    (dict(k=0x5000100), 1),                     # new keys inside the key cache
    (dict(qo=0x6000000), 1),                    # q_out inside the value cache
])
def test_rope_kv_write_rejects_bad_arguments(lib, kw, status):
    assert _rope(lib, **kw) == status


def test_rope_kv_write_rejects_bad_frequencies(lib):
    bad = [sda.RopeParams(0.0, 0, 0, 0, 0, 0, 0), sda.RopeParams(float("nan"), 0, 0, 0, 0, 0, 0),
           sda.RopeParams(-1.0, 0, 0, 0, 0, 0, 0), sda.RopeParams(1e4, 2, 0, 0, 0, 0, 0),
           sda.RopeParams(1e4, 0, 2, 0, 0, 0, 0),
           sda.RopeParams(1e4, 0, 1, 0.0, 1.0, 4.0, 8192.0),      # factor 0
           sda.RopeParams(1e4, 0, 1, 8.0, 4.0, 4.0, 8192.0),      # high == low
           sda.RopeParams(1e4, 0, 1, 8.0, 1.0, 4.0, float("inf"))]
    for r in bad:
        assert _rope(lib, rope=r) == 1
    assert _rope(lib, rope=False) == 1          # no description at all
    with pytest.raises(ValueError):
        sda.rope_params(1e4, pairing="interleaved")


def _prefill(lib, **kw):
    a = dict(q=0x1000000, k=0x2000000, v=0x3000000, lens=0x4000000, B=1, T=300, Hq=8, Hkv=2, D=64, S=512,
             scale=0.125, out=0x5000000, od=1)
    a.update(kw)
    return lib.prefill_attn(a["q"], a["k"], a["v"], a["lens"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"], a["S"],
                            a["scale"], a["out"], a["od"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(lens=None), 1), (dict(out=None), 1),
    (dict(B=0), 1), (dict(T=0), 1), (dict(S=0), 1), (dict(Hq=9), 1),
    (dict(D=96), 2), (dict(Hq=18, Hkv=2), 2), (dict(S=1 << 24, D=128), 2),
    (dict(q=0x1000008), 1), (dict(lens=0x4000002), 1), (dict(out=0x5000004), 1), (dict(od=3), 1),
    (dict(scale=float("nan")), 1),
])
def test_prefill_rejects_bad_arguments(lib, kw, status):
    assert _prefill(lib, **kw) == status


def test_gemv_entry_points_reject_bad_arguments(lib):
    W, X, Y, S = 0x1000000, 0x2000000, 0x3000000, 0x4000000
    g = lambda **kw: lib.gemv_bf16(kw.get("W", W), kw.get("x", X), kw.get("B", 2), kw.get("N", 64), kw.get("K", 256),
                                   kw.get("y", Y), kw.get("od", 1), None)
    for kw, st in [(dict(W=None), 1), (dict(x=None), 1), (dict(y=None), 1), (dict(B=0), 1), (dict(N=0), 1),
                   (dict(K=0), 1), (dict(B=9), 2), (dict(K=100), 2), (dict(W=W + 8), 1), (dict(x=X + 2), 1),
                   (dict(y=Y + 4), 1), (dict(od=5), 1), (dict(K=1 << 20), 2), (dict(K=73736), 2)]:
        assert g(**kw) == st, kw
    q = lambda **kw: lib.gemv_int8(kw.get("W", W), kw.get("s", S), X, 1, 64, kw.get("K", 256), Y, 1, None)
    assert q(s=None) == 1 and q(K=264) == 2 and q(s=S + 2) == 1 and q(K=73744) == 2
    z = lambda **kw: lib.quantize_rows_int8(kw.get("W", W), kw.get("N", 64), kw.get("K", 256), kw.get("q", X),
                                            kw.get("s", S), None)
    for kw, st in [(dict(W=None), 1), (dict(q=None), 1), (dict(s=None), 1), (dict(N=0), 1), (dict(K=24), 2),
                   (dict(q=W + 64), 1), (dict(s=W + 16), 1), (dict(q=X + 8), 1)]:
        assert z(**kw) == st, kw


_SPEC = dict(logits=0x10000000, q=0x20000000, drafts=0x30000000, u=0x31000000, r=0x32000000, tau=1.0,
             B=2, T=4, V=1000, S=512, lens=0x40000000, result=0x41000000, ws=0x50000000, wsb=1 << 20)


def _spec(lib, **kw):
    a = dict(_SPEC, **kw)
    return lib.spec_accept(a["logits"], a["q"], a["drafts"], a["u"], a["r"], a["tau"], a["B"], a["T"], a["V"],
                           a["S"], a["lens"], a["result"], a["ws"], a["wsb"], None)


def test_spec_workspace_bytes(lib):
    w = lib.spec_accept_workspace_bytes
    assert w(1, 6, 128256) > 0 and w(0, 6, 100) == 0 and w(1, 0, 100) == 0 and w(1, 6, 0) == 0
    assert w(1, 33, 100) == 0 and w(1, 6, (1 << 24) + 1) == 0
    # the chunk statistics of every position and the residual mass of every
    # chunk (8 bytes per chunk of 1024 to 8192 entries), 16 bytes per row and
    # per draft, each rounded up to 256 bytes
    for B, T, V in [(1, 6, 128256), (64, 6, 128256), (3, 1, 50257), (8, 32, 1 << 24)]:
        nc_max = -(-V // 1024)
        nc_min = -(-V // 8192)
        small = 16 * B + 16 * B * max(T - 1, 1)
        assert (B * T + B) * nc_min * 8 + small <= w(B, T, V) <= (B * T + B) * nc_max * 8 + small + 1024
        assert w(B, T, V) % 256 == 0


@pytest.mark.parametrize("kw,status", [
    (dict(logits=None), 1), (dict(lens=None), 1), (dict(result=None), 1), (dict(ws=None), 1),
    (dict(drafts=None), 1), (dict(r=None), 1), (dict(q=None), 1), (dict(u=None), 1),
    (dict(tau=-1.0), 1), (dict(tau=float("nan")), 1), (dict(tau=float("inf")), 1), (dict(tau=1e-45), 1),
    (dict(B=0), 1), (dict(T=0), 1), (dict(V=0), 1), (dict(S=0), 1), (dict(T=33), 2), (dict(V=(1 << 24) + 1), 2),
    (dict(logits=0x10000002), 1), (dict(lens=0x40000001), 1), (dict(ws=0x50000008), 1), (dict(wsb=64), 3),
    (dict(result=0x10000010), 1),               # result inside logits
    (dict(result=0x40000004), 1),               # result overlaps lens
    (dict(ws=0x20000100), 1),                   # workspace inside q
    (dict(lens=0x32000004), 1),                 # lens overlaps r
])
def test_spec_accept_rejects_bad_arguments(lib, kw, status):
    assert _spec(lib, **kw) == status


def test_binding_rejects_host_tensors_before_calling_the_library():
    """The ctypes layer refuses tensors that are not on a device (it would
    otherwise hand host addresses to the kernels)."""
    import torch
    W = torch.zeros((16, 64), dtype=torch.bfloat16)
    x = torch.zeros((1, 64), dtype=torch.bfloat16)
    y = torch.zeros((1, 16), dtype=torch.float32)
    with pytest.raises(ValueError, match="device tensor"):
        sda.gemv_bf16(W, x, y)
    q = torch.zeros((1, 4, 64), dtype=torch.bfloat16)
    kv = torch.zeros((1, 2, 32, 64), dtype=torch.bfloat16)
    lens = torch.zeros((1,), dtype=torch.int32)
    ws = torch.zeros((4096,), dtype=torch.uint8)
    with pytest.raises(ValueError, match="device tensor"):
        sda.decode_attn(q, kv, kv, lens, 0.125, q.clone(), ws)


def test_query_head_count_limit(lib):
    """Hq up to 2^24 is accepted (the merge divides head indices by G with a
    32-bit multiply-high, exact below 2^28); one group more is refused."""
    assert sda.workspace_bytes(1, 1, 1 << 24, 1 << 21, 64, 16, 16) > 0
    assert sda.workspace_bytes(1, 1, (1 << 24) + 8, ((1 << 24) + 8) // 8, 64, 16, 16) == 0
    assert sda.default_chunk(1, 1, (1 << 24) + 8, ((1 << 24) + 8) // 8, 64, 16) == 0
