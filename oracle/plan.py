"""Oracle shard plan: flatten + align + pad, then cut into 1/N shards.

TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product library. Plain Python
integer arithmetic, written from the definitions:

* FLAT layout -- one flat buffer per wrap unit ("ZeRO vs FSDP: A Rigorous
  Dissection..." section 3.2, The FlatParameter Abstraction: all parameters of
  a group are concatenated into a single 1-D tensor). Tensors keep their listed
  order; each starts at a multiple of ``align`` elements; the total is padded to
  a multiple of ``world * 8`` so the N shards are equal and each is a whole
  number of 16-byte vectors. Padding, flattening and alignment are real bytes
  that the ledger counts ("从 Data Parallel 到 ZeRO/FSDP" section
  "一次 Mixed-precision Adam 为什么接近 16 Bytes/Parameter").
* PER_TENSOR layout -- each tensor sharded on its own (FSDP2's per-parameter
  sharded state, "从 Data Parallel 到 ZeRO/FSDP" section "ZeRO 与 FSDP 的关系"):
  tensor i is flattened row-major, padded to ``T_i = roundup(n_i, world*8)``
  and cut into ``world`` equal contiguous pieces of ``S_i = T_i / world``.
* Rank r owns the r-th of the N equal slices ("ZeRO vs FSDP..." section 2: each
  rank holds a 1/dp slice of whatever is sharded).
* Ledger -- persistent bytes per rank = 16 per owned element: bf16 param 2 +
  bf16 grad 2 + fp32 m 4 + fp32 v 4 + fp32 master 4 ("FSDP2's parameter
  lifecycle..." section "16 bytes per parameter is where planning starts").
"""

from dataclasses import dataclass, field

SHARD_GRANULE = 8  # elements: one 16-byte vector of bf16


def roundup(x, a):
    return -(-x // a) * a


@dataclass
class OraclePiece:
    tensor: int
    own_lo: int  # first owned element, tensor-local (padded) coordinates
    own_hi: int  # one past the last owned element (padded coordinates)
    real_lo: int  # owned real (non-padding) elements, tensor-local
    real_hi: int
    shard_off: int  # where the piece starts in the rank's packed shard
    full_off: int  # where the piece starts in the packed gathered buffer


@dataclass
class OraclePlan:
    layout: str
    world: int
    rank: int
    align: int
    numels: list
    offsets: list = field(default_factory=list)  # FLAT: tensor starts; PER_TENSOR: packed starts
    padded: list = field(default_factory=list)  # PER_TENSOR: T_i
    T: int = 0  # padded flat length (PER_TENSOR: sum of T_i)
    S: int = 0  # owned elements (PER_TENSOR: sum of S_i)
    pieces: list = field(default_factory=list)

    @property
    def persistent_bytes(self):
        return 16 * self.S

    def padding_mask_full(self):
        """bytearray over [0, T): 1 where the element is padding (no tensor covers it)."""
        mask = bytearray([1]) * self.T
        for i, n in enumerate(self.numels):
            o = self.offsets[i]
            mask[o:o + n] = bytes(n)
        return mask


def plan_flat(numels, world, rank, align=1):
    if world < 1 or not (0 <= rank < world) or align < 1:
        raise ValueError("bad world/rank/align")
    offs = []
    end = 0
    for n in numels:
        if n < 0:
            raise ValueError("negative numel")
        o = roundup(end, align)
        offs.append(o)
        end = o + n
    T = roundup(end, world * SHARD_GRANULE)
    S = T // world
    lo_own, hi_own = rank * S, (rank + 1) * S
    pieces = []
    for i, n in enumerate(numels):
        lo = max(offs[i], lo_own)
        hi = min(offs[i] + n, hi_own)
        if lo < hi:
            pieces.append(OraclePiece(i, lo - offs[i], hi - offs[i], lo - offs[i], hi - offs[i],
                                      lo - lo_own, lo))
    return OraclePlan("flat", world, rank, align, list(numels), offs, [], T, S, pieces)


def plan_per_tensor(numels, world, rank, persist_below=0):
    """PER_TENSOR plan. Tensors with fewer than ``persist_below`` elements are
    not sharded: every rank holds and updates the whole tensor, padded to one
    16-byte vector ("ZeRO vs FSDP..." section 7: small parameters such as
    norms stay replicated under a persistence threshold)."""
    if world < 1 or not (0 <= rank < world):
        raise ValueError("bad world/rank")
    padded, offs, pieces = [], [], []
    shard_acc = 0
    full_acc = 0
    for i, n in enumerate(numels):
        if n < 0:
            raise ValueError("negative numel")
        if n < persist_below:
            Ti = roundup(n, SHARD_GRANULE)
            padded.append(Ti)
            offs.append(full_acc)
            pieces.append(OraclePiece(i, 0, Ti, 0, n, shard_acc, full_acc))
            shard_acc += Ti
            full_acc += Ti
            continue
        Ti = roundup(n, world * SHARD_GRANULE)
        Si = Ti // world
        padded.append(Ti)
        offs.append(full_acc)
        lo, hi = rank * Si, (rank + 1) * Si
        pieces.append(OraclePiece(i, lo, hi, min(lo, n), min(hi, n), shard_acc, full_acc + lo))
        shard_acc += Si
        full_acc += Ti
    return OraclePlan("per_tensor", world, rank, 1, list(numels), offs, padded, full_acc, shard_acc,
                      pieces)


@dataclass
class ReshardSlice:
    group_size: int  # k: ranks the parameters stay sharded over after forward
    slice_index: int  # j = r mod k: which of the k equal slices of [0, T) this rank keeps
    slice_off: int  # j * T/k
    slice_len: int  # T/k
    first_source: int  # the kept slice is the N-way shards of ranks first_source ..
    n_sources: int  # .. first_source + n_sources - 1, in order (n_sources = N/k)
    owner_slice: int  # the slice index that holds this rank's own shard: r div (N/k)
    own_off: int  # where this rank's shard starts inside that slice: (r mod (N/k)) * S
    retained_bytes: int  # bf16 parameter bytes this rank keeps after forward: 2 * T/k


def reshard_slice(plan, k):
    """The slice of the gathered flat buffer a rank keeps after forward when
    parameters are resharded to a group of k ranks instead of all N.

    "FSDP2's parameter lifecycle..." section "Reshard policy: pay for the
    memory, or pay for the communication again": reshard_after_forward also
    takes an integer, resharding to a smaller world size than N (intra-node,
    say), so the backward AllGather only runs over that smaller group. The
    plainest reading that makes the group intra-node: k divides N, the groups
    are k consecutive ranks, and the k members of a group split the flat
    buffer [0, T) into k equal contiguous slices, member position j = r mod k
    keeping slice j. A slice of T/k elements is N/k consecutive N-way shards,
    those of ranks j*N/k .. (j+1)*N/k - 1. k = N keeps only the own shard
    (full resharding); k = 1 keeps the whole buffer (no resharding)."""
    if plan.layout != "flat":
        raise ValueError("reshard slices are defined on FLAT plans")
    N, r, S, T = plan.world, plan.rank, plan.S, plan.T
    if k < 1 or k > N or N % k:
        raise ValueError(f"reshard group size {k} must divide the world size {N}")
    per_slice = N // k
    L = T // k
    j = r % k
    return ReshardSlice(k, j, j * L, L, j * per_slice, per_slice, r // per_slice, (r % per_slice) * S, 2 * L)
