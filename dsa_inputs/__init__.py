"""Seeded synthetic inputs for the DSA layer (shared by the oracle side and the GPU side).

This package holds no arithmetic of the attention method.  It provides:

* a counter-based generator (SplitMix64 + Irwin-Hall normal), with a host twin in C
  (``gen_host.c``) and a device twin in HIP (``gen_device.hip``) that produce
  bit-identical tensors, so multi-GB inputs are generated in HBM while the oracle
  regenerates any slice it needs on the host;
* workload descriptions (requests, query rows and their positions, page tables) at
  the shapes of the pages' decode / verify / long-context / chunked-prefill cases.

Tensor ids and flat-index conventions (the same on both sides):

====  ====================  ==============================================
 id    tensor                flat index of element
====  ====================  ==============================================
  1    indexer q  (bf16)     (row * 32 + head) * 128 + d
  2    raw index key (bf16)  (token_base[req] + pos) * 128 + d
  3    head weights (fp32)   row * 32 + head, value U(0,1) / sqrt(32)
  4    MLA q (bf16)          (row * 64 + head) * 576 + d
  5+l  latent of layer l     (token_base[req] + pos) * 576 + d
  9    page permutation      Fisher-Yates draws
 10    context lengths       one draw per request
 11    needle positions      partial Fisher-Yates draws
====  ====================  ==============================================
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_LIB = os.path.join(HERE, "libdsa_gen_host.so")
DEV_LIB = os.path.join(HERE, "libdsa_gen_dev.so")

SEED_BASE = 0x5EED0000
T_IDX_Q, T_RAW_K, T_W, T_MLA_Q, T_LATENT0, T_PERM, T_CTX, T_NEEDLE = 1, 2, 3, 4, 5, 9, 10, 11
# A projection output rows [q_c 2048 | kv_c 512 | k_pe 64] and the kv_a RMSNorm weight
T_KV_A, T_GAMMA = 12, 13
KV_A_WIDTH = 2048 + 576
PAGE = 64


# ----------------------------------------------------------------------------- build / load
def build_host() -> str:
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           os.path.join(HERE, "gen_host.c"), "-o", HOST_LIB]
    subprocess.check_call(cmd)
    return HOST_LIB


def build_device() -> str:
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(HERE, "gen_device.hip"), "-o", DEV_LIB]
    subprocess.check_call(cmd, stderr=subprocess.DEVNULL)
    return DEV_LIB


_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            build_host()
        lib = ctypes.CDLL(HOST_LIB)
        u64, i64, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.gen_normal_bf16.argtypes = [u64, u64, u64, i64, p]
        lib.gen_normal_bf16_at.argtypes = [u64, u64, p, i64, p]
        lib.gen_uniform_f32.argtypes = [u64, u64, u64, i64, ctypes.c_double, p]
        lib.gen_u64.argtypes = [u64, u64, u64, i64, p]
        for f in (lib.gen_normal_bf16, lib.gen_normal_bf16_at, lib.gen_uniform_f32, lib.gen_u64):
            f.restype = None
        _host = lib
    return _host


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"device generator not built: {DEV_LIB} (run __graft_entry__.build())")
        lib = ctypes.CDLL(DEV_LIB)
        u64, i64, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.gen_dev_normal_bf16.argtypes = [u64, u64, u64, i64, p, p]
        lib.gen_dev_uniform_f32.argtypes = [u64, u64, u64, i64, ctypes.c_double, p, p]
        lib.gen_dev_normal_bf16.restype = ctypes.c_int
        lib.gen_dev_uniform_f32.restype = ctypes.c_int
        _dev = lib
    return _dev


# ----------------------------------------------------------------------------- host generator
def normal_bf16(seed: int, tensor_id: int, start: int, n: int) -> np.ndarray:
    """bf16 bit patterns (uint16) of normal(start .. start+n-1)."""
    out = np.empty(n, np.uint16)
    _host_lib().gen_normal_bf16(seed, tensor_id, start, n, out.ctypes.data)
    return out


def normal_bf16_at(seed: int, tensor_id: int, index: np.ndarray) -> np.ndarray:
    index = np.ascontiguousarray(index, dtype=np.int64)
    out = np.empty(index.shape, np.uint16)
    _host_lib().gen_normal_bf16_at(seed, tensor_id, index.ctypes.data, index.size, out.ctypes.data)
    return out


def uniform_f32(seed: int, tensor_id: int, start: int, n: int, mul: float = 1.0) -> np.ndarray:
    out = np.empty(n, np.float32)
    _host_lib().gen_uniform_f32(seed, tensor_id, start, n, mul, out.ctypes.data)
    return out


def draws_u64(seed: int, tensor_id: int, start: int, n: int) -> np.ndarray:
    out = np.empty(n, np.uint64)
    _host_lib().gen_u64(seed, tensor_id, start, n, out.ctypes.data)
    return out


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- device generator
def dev_normal_bf16(seed: int, tensor_id: int, start: int, n: int, out_ptr: int, stream: int = 0) -> None:
    rc = _dev_lib().gen_dev_normal_bf16(seed, tensor_id, start, n, out_ptr, stream)
    if rc:
        raise RuntimeError(f"gen_dev_normal_bf16 failed: hip error {rc}")


def dev_uniform_f32(seed: int, tensor_id: int, start: int, n: int, mul: float, out_ptr: int,
                    stream: int = 0) -> None:
    rc = _dev_lib().gen_dev_uniform_f32(seed, tensor_id, start, n, mul, out_ptr, stream)
    if rc:
        raise RuntimeError(f"gen_dev_uniform_f32 failed: hip error {rc}")


# ----------------------------------------------------------------------------- permutations
def permutation(seed: int, tensor_id: int, n: int) -> np.ndarray:
    """Fisher-Yates permutation of range(n) driven by the counter generator."""
    a = np.arange(n, dtype=np.int64)
    if n > 1:
        d = draws_u64(seed, tensor_id, 0, n)
        for i in range(n - 1, 0, -1):
            j = int(d[i] % np.uint64(i + 1))
            a[i], a[j] = a[j], a[i]
    return a


def choose_distinct(seed: int, tensor_id: int, n: int, k: int) -> np.ndarray:
    """k distinct values of range(n) (partial Fisher-Yates), sorted ascending."""
    a = np.arange(n, dtype=np.int64)
    d = draws_u64(seed, tensor_id, 0, k)
    for i in range(k):
        j = i + int(d[i] % np.uint64(n - i))
        a[i], a[j] = a[j], a[i]
    return np.sort(a[:k])


# ----------------------------------------------------------------------------- workloads
@dataclass
class Workload:
    """One batch of the DSA layer: requests with their contexts, query rows and page table.

    ``ctx[b]`` positions 0..ctx[b]-1 of request b are in the caches after the step's store;
    the query rows of request b sit at the last ``rows_per_req`` of them (decode / verify),
    or at ``row_pos`` given explicitly (prefill).
    """
    name: str
    seed: int
    ctx: np.ndarray                 # [B] context length after the step (tokens)
    row_req: np.ndarray             # [R] request of each query row (grouped, ascending)
    row_pos: np.ndarray             # [R] absolute position of each query row
    rows_per_req: int               # rows sharing one request (contiguous group size)
    page_table: np.ndarray          # [B, max_pages] int32 page ids
    num_pages: int                  # pages in the pool (per cache)
    n_layers: int = 1
    full_layers: tuple = (0,)
    needles: np.ndarray | None = None   # positions planted to win the indexer score (request 0)
    extra: dict = field(default_factory=dict)

    @property
    def B(self) -> int:
        return int(self.ctx.shape[0])

    @property
    def R(self) -> int:
        return int(self.row_pos.shape[0])

    @property
    def token_base(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.ctx)[:-1]]).astype(np.int64)

    @property
    def total_tokens(self) -> int:
        return int(self.ctx.sum())

    @property
    def max_pos(self) -> int:
        return int(self.row_pos.max())

    @property
    def row0(self) -> int:
        """Index of this batch's first query row among all rows of its workload (a chunk of a
        chunked prefill starts past the earlier chunks' rows); seeded query offsets use it."""
        return int(self.extra.get("row0", 0))

    @property
    def rows_total(self) -> int:
        return int(self.extra.get("rows_total", self.R))


def _page_table(seed: int, ctx: np.ndarray, spare_pages: int = 0):
    npg = (ctx + PAGE - 1) // PAGE
    total = int(npg.sum()) + spare_pages
    perm = permutation(seed, T_PERM, total)
    width = int(npg.max())
    pt = np.zeros((len(ctx), width), np.int32)
    off = 0
    for b, n in enumerate(npg):
        pt[b, :n] = perm[off:off + n]
        off += int(n)
    return pt, total


def make_decode(name: str, seed: int, ctx, rows_per_req: int = 1, n_layers: int = 1,
                full_layers=(0,)) -> Workload:
    ctx = np.asarray(ctx, dtype=np.int64)
    B = len(ctx)
    pt, npages = _page_table(seed, ctx)
    row_req = np.repeat(np.arange(B, dtype=np.int32), rows_per_req)
    row_pos = np.concatenate([np.arange(c - rows_per_req, c) for c in ctx]).astype(np.int32)
    return Workload(name, seed, ctx, row_req, row_pos, rows_per_req, pt, npages, n_layers, tuple(full_layers))


def make_prefill(name: str, seed: int, prefix: int, new: int) -> Workload:
    ctx = np.array([prefix + new], np.int64)
    pt, npages = _page_table(seed, ctx)
    row_req = np.zeros(new, np.int32)
    row_pos = np.arange(prefix, prefix + new, dtype=np.int32)
    return Workload(name, seed, ctx, row_req, row_pos, new, pt, npages, 1, (0,),
                    extra={"prefix": prefix})


def prefill_chunk(w: Workload, c: int) -> Workload:
    """Chunk c of a chunked prefill (``w.extra["chunk"]`` rows each): the same request, page
    table and caches, with the chunk's rows as the batch."""
    n = int(w.extra["chunk"])
    a, b = c * n, min(w.R, (c + 1) * n)
    assert 0 <= a < b
    return replace(w, name=f"{w.name}[chunk {c}]", row_req=w.row_req[a:b], row_pos=w.row_pos[a:b],
                   rows_per_req=b - a, extra={**w.extra, "row0": a, "rows_total": w.R, "chunk_index": c})


def config(cid: int, scale: str = "full") -> Workload:
    """The pages' five workload shapes.  scale="small" shrinks them for fast parity runs
    while keeping several tiles, ragged tails and the multi-row / multi-layer structure."""
    seed = SEED_BASE + cid
    small = scale == "small"
    if cid == 0:     # tiny decode: 1 request, L = 4096
        return make_decode("c0_tiny_decode", seed, [4096])
    if cid == 1:     # decode batch: 32 requests, L ~ U[8K, 32K]
        B = 6 if small else 32
        lo, hi = (2100, 5000) if small else (8192, 32768)
        d = draws_u64(seed, T_CTX, 0, B)
        ctx = lo + (d % np.uint64(hi - lo + 1)).astype(np.int64)
        return make_decode("c1_decode_batch", seed, ctx)
    if cid == 2:     # speculative verify: 64 x 6 rows at 128K, 4-layer group (1 full + 3 shared)
        B, L = (3, 5000) if small else (64, 131072)
        return make_decode("c2_verify_128k", seed, [L] * B, rows_per_req=6, n_layers=4, full_layers=(0,))
    if cid == 3:     # long context: 1 request, L = 2^20, 2048 needles
        L = 300_000 if small else 1 << 20
        w = make_decode("c3_long_1m", seed, [L])
        w.needles = choose_distinct(seed, T_NEEDLE, L - 1, 2048)
        return w
    if cid == 4:     # chunked prefill: 8192 new rows on a 65,536-token prefix
        prefix, new = (3000, 70) if small else (65536, 8192)
        return make_prefill("c4_chunked_prefill", seed, prefix, new)
    if cid == 5:     # a whole 1M-token prompt prefilled in 32K-token chunks (prefill_chunk())
        total, chunk = (9000, 3100) if small else (1 << 20, 32768)
        w = make_prefill("c5_chunked_prefill_1m", seed, 0, total)
        w.extra["chunk"] = chunk
        return w
    raise ValueError(cid)


def w_scale() -> float:
    return 1.0 / math.sqrt(32.0)
