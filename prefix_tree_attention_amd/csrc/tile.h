// Internal: 64-row LDS tiles for the gfx950 attention kernels.
//
// A tile holds 64 consecutive tokens x D bf16 of one head as 16-byte chunks
// (D/8 per row).  It is filled straight from HBM by global_load_lds_dwordx4
// (each lane's 16 bytes land at the instruction's LDS base + 16 * lane), so
// staging costs no registers and no LDS store instructions; which chunk a
// lane fetches decides the layout.  The kernels read a tile in two patterns:
//   - row-major operand reads (ds_read_b128): each lane 16 bytes of its row;
//   - transposed operand reads (ds_read_b64_tr_b16): a 16-lane group reads
//     4 consecutive rows x 16 consecutive elements, and lane i of the group
//     receives element i of each of the 4 rows -- i.e. an MFMA operand
//     fragment whose k index runs over rows.
// Two layouts:
//   - Tile (the forward's): natural row order, chunk c of row r at slot
//     position c ^ swz(r) within the row, with the GF(2)-linear swizzle of
//     the row's low 4 bits that measured fastest for both patterns together
//     (every invertible map was timed): for D = 128 (16 chunks per 256-byte
//     row) swz(r) = (4 (r % 4) + 2 ((r / 4) % 2)) ^ 3 ((r / 8) % 2), for
//     D = 64 (8 chunks per 128-byte row) swz(r) = (r % 8) ^ 2 ((r / 8) % 2).
//     Its reads are free of bank conflicts (SQ_LDS_BANK_CONFLICT reads 0);
//     each lane's offsets are loop-invariant registers.
//   - QuadTile (dK/dV and dQ, below): quad-major blocks in which every
//     operand read is one per-lane base plus an immediate, also free of
//     bank conflicts under the LDS's measured pass structure.
// The LDS issues about one wave-wide read per 4.5 clocks whatever its width.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <utility>

#include "mfma.h"

namespace treeattn {

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kTileRows = 64;

__device__ __forceinline__ uint32_t lds_addr(const lds_char* p) { return uint32_t(size_t(p)); }

// Direct HBM -> LDS loads: each lane's 16 (dma16) or 4 (dma4) bytes at
// base + voff land at LDS address lds + 16 * lane (4 * lane); `base` and
// `lds` are wave-uniform.  They are issued as inline asm so that the
// compiler does not count them as pending LDS writes: it cannot tell the
// buffer being filled from the one being read, and would otherwise wait for
// the prefetch to land before the first transposing LDS read of a step.
// Completion is the caller's s_waitcnt vmcnt followed by a workgroup
// barrier.  M0 carries the LDS address (one wait state before its use).
// Both M0 and, for the scalar add, SCC are declared clobbered: with SCC
// undeclared the compiler once kept a compare's result in SCC across a run
// of these loads and selected on the carry of the M0 add instead.
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "m0");
}
// same, LDS address lds + IMM (one scalar add into M0)
template <int IMM>
__device__ __forceinline__ void dma16_at(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
                 "s"(lds), "n"(IMM)
                 : "m0", "scc");
}
__device__ __forceinline__ void dma4(const void* base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "s"(lds)
                 : "m0");
}

template <int D>
struct Tile {
    static constexpr int kChunks = D / 8;              // 16-byte chunks per row
    static constexpr int kBytes = kTileRows * D * 2;   // 16 KB (D=128) / 8 KB (D=64)

    __device__ static __forceinline__ int swz(int r) {
        if constexpr (D == 128)
            return ((r & 3) << 2 | (r & 4) >> 1) ^ (3 * ((r >> 3) & 1));
        else
            return (r & 7) ^ (2 * ((r >> 3) & 1));
    }
    static constexpr int kRowBytes = D * 2;
    // byte offset of (row, chunk) inside the tile; the swizzle depends on
    // r % 16 only, so moving 16 rows down is a plain add of 16 kRowBytes
    __device__ static __forceinline__ int slot(int r, int c) { return (r * kChunks + (c ^ swz(r))) * 16; }

    // Issue this wave's share of the direct loads of one tile, shared by NW
    // waves (1 KB per wave instruction, kLoads<NW> instructions each).
    // `g0` points at element 0 of row 0 (token of row 0, this head);
    // `stride` is the token stride in elements.  Completion: s_waitcnt vmcnt
    // in each wave, then a workgroup barrier.
    template <int NW>
    static constexpr int kLoads = kBytes / 1024 / NW;
    template <int NW = 4>
    __device__ static __forceinline__ void load_async(lds_char* tile, const bf16* __restrict__ g0, int stride,
                                                      int wave, int lane) {
        const uint32_t lds0 = lds_addr(tile) + uint32_t(wave * kLoads<NW> * 1024);
        load_async_j<NW>(lds0, g0, stride, wave, lane, std::make_integer_sequence<int, kLoads<NW>>{});
    }
    template <int NW, int... J>
    __device__ static __forceinline__ void load_async_j(uint32_t lds0, const bf16* __restrict__ g0, int stride,
                                                        int wave, int lane, std::integer_sequence<int, J...>) {
        (dma16_at<1024 * J>(g0, lane_offset<NW>(J, stride, wave, lane), lds0), ...);
    }
    // byte offset (from g0) of the 16 bytes lane `lane` fills in load J
    template <int NW>
    __device__ static __forceinline__ uint32_t lane_offset(int j, int stride, int wave, int lane) {
        const int blk = wave * kLoads<NW> + j;  // 1 KB block = 64 slots
        const int p = blk * 64 + lane;          // slot this lane fills
        const int r = p / kChunks, pos = p % kChunks;
        const int c = pos ^ swz(r);
        return uint32_t(r * stride + 8 * c) * 2u;
    }

    // Row-major operand: 8 bf16 of row r starting at element 8c.
    __device__ static __forceinline__ bf16x8 row_frag(const lds_char* tile, int r, int c) {
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(tile + slot(r, c));
    }

    // Transposed operand: for a 16-lane group whose 4 rows start at r0, lane
    // i (0..15) gets element e0 + i of rows r0..r0+3 (e0 a multiple of 16).
    __device__ static __forceinline__ int tr_offset(int r0, int e0, int i) {
        const int r = r0 + (i >> 2);
        const int e = e0 + 4 * (i & 3);
        return slot(r, e >> 3) + ((e >> 2) & 1) * 8;
    }
    __device__ static __forceinline__ i16x4 tr_at(const lds_char* base, int off) {
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) i16x4*>(const_cast<lds_char*>(base) + off));
    }
    __device__ static __forceinline__ i16x4 tr_frag(const lds_char* tile, int r0, int e0, int i) {
        return tr_at(tile, tr_offset(r0, e0, i));
    }
    // Row-major operand at a precomputed byte offset.
    __device__ static __forceinline__ bf16x8 frag_at(const lds_char* base, int off) {
        return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(base + off);
    }
};

// 64-row tiles in quad-major blocks, for kernels whose per-lane operand
// offsets must not cost address arithmetic at every read.
//
// Rows are grouped by RPB (4 for D = 128, 8 for D = 64): one 1 KB direct
// load fills one block.  Inside a block, the 64 bytes of chunks 4y..4y+3
// (a quad) of row q sit at QS y + 64 q, QS = 64 RPB, so with
// px(x) = QS (x / 2) + 32 (x % 2) for chunk pair x:
//   - a row-major read of chunk 2x + h of row r is at rb(r) + 16 h + px(x),
//   - a transposing read of rows r0..r0+3 (r0 % 4 == 0) and elements
//     16x..16x+15 gives lane i of the 16-lane group 8 bytes at
//     rb(r0) + px(x) + 64 (i / 4) + 8 (i % 4).
// Each lane keeps one base per pattern, and every step of x, every 16-row
// move (+GS) and every 8-row move inside a 16-row group (+R8) is an
// immediate.  Four consecutive lanes of a direct load fetch one aligned 64
// bytes of one row, as in the swizzled tile.
//
// Bank conflicts, as measured on gfx950 with SQ_LDS_BANK_CONFLICT: 64 banks
// of 4 bytes; a ds_read_b128 is served in four passes of 16 lanes, each
// pass the lane quads (4 lanes) of one 32-lane half whose quad index has
// even (0, 3, 5, 6) or odd (1, 2, 4, 7) bit parity; a ds_read_b64_tr_b16
// in two passes, lanes 0-31 and 32-63.  For D = 128 the blocks of a 16-row
// group start at 0, 1056, 2112 and 3168 bytes (16-byte slots 0, 66, 132,
// 198: 0, 2, 0, 2 mod 4) and a group is 4208 bytes (263 slots, odd): under
// that pass structure the row-major reads of the 32x32x16 and 16x16x32
// operand layouts and the transposing reads of both kernels are
// conflict-free.  For D = 64 (blocks at 0 and 1056 of a 2096-byte group)
// only dQ's transposing read keeps a 2-way conflict.
template <int D>
struct QuadTile {
    static_assert(D == 128 || D == 64, "D is 128 or 64");
    static constexpr int kRpb = D == 128 ? 4 : 8;         // rows per 1 KB block
    static constexpr int kQs = 64 * kRpb;                 // quad stride
    static constexpr int kBlocks = 16 / kRpb;             // blocks per 16-row group
    static constexpr int kGs = D == 128 ? 4208 : 2096;    // 16-row group stride
    static constexpr int kR8 = D == 128 ? 2112 : 1056;    // 8-row move inside a group
    static constexpr int kBytes = 4 * kGs;
    __host__ __device__ static constexpr int block_base(int b) {
        return D == 128 ? (b == 0 ? 0 : b == 1 ? 1056 : b == 2 ? 2112 : 3168) : (b == 0 ? 0 : 1056);
    }
    static_assert(D != 128 || (block_base(2) - block_base(0) == kR8 && block_base(3) - block_base(1) == kR8),
                  "8-row moves are one immediate");
    static_assert(D != 64 || block_base(1) == kR8, "8-row moves are one immediate");
    static_assert(block_base(kBlocks - 1) + 1024 <= kGs && kGs % 16 == 0, "blocks fit the group");

    // offset of chunk pair x (chunks 2x, 2x+1) from its row's start
    __host__ __device__ static constexpr int px(int x) { return kQs * (x >> 1) + 32 * (x & 1); }
    // lane i's offset in a transposing read of 4 rows x 16 elements
    __host__ __device__ static constexpr int tr_lane(int i) { return 64 * (i >> 2) + 8 * (i & 3); }
    // offset of row r's start (chunk 0; r in 0..63)
    __host__ __device__ static __forceinline__ int rb(int r) {
        return kGs * (r >> 4) + (D == 128 ? block_base((r >> 2) & 3) + 64 * (r & 3)
                                          : block_base((r >> 3) & 1) + 64 * (r & 7));
    }

    __device__ static __forceinline__ bf16x8 frag_at(const lds_char* base, int off) {
        return Tile<D>::frag_at(base, off);
    }
    __device__ static __forceinline__ i16x4 tr_at(const lds_char* base, int off) { return Tile<D>::tr_at(base, off); }

    // Issue this wave's share (16-row group `wave`) of the direct loads of
    // one tile shared by four waves.  `g0` points at element 0 of row 0;
    // `stride` is the token stride in elements.  Completion: s_waitcnt vmcnt
    // in each wave, then a workgroup barrier.
    __device__ static __forceinline__ void load_async(lds_char* tile, const bf16* __restrict__ g0, int stride,
                                                      int wave, int lane) {
        const uint32_t lds0 = lds_addr(tile) + uint32_t(wave * kGs);
        load_async_j(lds0, g0, stride, wave, lane, std::make_integer_sequence<int, kBlocks>{});
    }
    template <int... J>
    __device__ static __forceinline__ void load_async_j(uint32_t lds0, const bf16* __restrict__ g0, int stride,
                                                        int wave, int lane, std::integer_sequence<int, J...>) {
        (dma16_at<block_base(J)>(g0, lane_offset(J, stride, wave, lane), lds0), ...);
    }
    // byte offset (from g0) of the 16 bytes lane `lane` fills in block J of
    // group `wave`: slot s = lane holds chunk 4 (s / 4RPB) + s % 4 of row
    // (s / 4) % RPB of the block
    __host__ __device__ static __forceinline__ uint32_t lane_offset(int j, int stride, int wave, int lane) {
        const int r = 16 * wave + kRpb * j + ((lane >> 2) & (kRpb - 1));
        const int c = 4 * (lane / (4 * kRpb)) + (lane & 3);
        return uint32_t(r * stride + 8 * c) * 2u;
    }
};

// A compiler-visible use of a loaded value.  The direct loads above are
// invisible to the compiler's wait-count bookkeeping, so a kernel's
// prologue loads are consumed here, before its main loop: otherwise the
// compiler places their waits at the first use inside the loop, where the
// hardware counter also holds the freshly issued prefetch.
__device__ __forceinline__ void consume(const bf16x8& v) { asm volatile("" ::"v"(__builtin_bit_cast(i32x4, v))); }
__device__ __forceinline__ void consume(float v) { asm volatile("" ::"v"(v)); }
__device__ __forceinline__ void consume(int v) { asm volatile("" ::"v"(v)); }

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// wait until at most N of this wave's vector memory operations are pending
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// XCD-aware work order.  Workgroups are dispatched round-robin over the 8
// XCDs (block b runs on XCD b % 8), and each XCD has its own L2.  The
// logical work index returned here gives XCD x the contiguous range
// [x W/8, (x+1) W/8) of a key/value-head-major order, so the workgroups
// sharing K/V tiles (or Q/dO tiles) of one key/value head meet in one L2,
// while each XCD still takes its range heaviest-first.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_logical_block() {
    const int W = int(gridDim.x), b = int(blockIdx.x);
    if (W % kXcds != 0) return b;
    return (b % kXcds) * (W / kXcds) + b / kXcds;
}

// Eight bf16 from two transposed reads (k 0..3 then k 4..7).
__device__ __forceinline__ bf16x8 join_tr(const i16x4& lo, const i16x4& hi) {
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
}

}  // namespace treeattn
