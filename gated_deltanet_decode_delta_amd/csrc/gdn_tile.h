// gdn_tile.h -- the register mapping of one value head's D x D state tile used
// by the decode-shaped kernels (single-token decode, draft verify, and the
// decode with the fused input stage).  Each kernel writes its token loop out in
// full over this mapping: the register allocator keeps the tile in VGPRs only
// when the loads, the update and the stores sit in one straight-line body.
//
// A row of the tile is covered by LPR consecutive lanes (16 at D = 128, one DPP
// row) that each hold NCH 16-byte vectors of it, interleaved so that one load
// instruction of 16 lanes covers 256 contiguous bytes; a lane keeps RPL rows.
// At D = 128 (fp32) a 256-thread workgroup holds the whole 64 KiB tile as 16
// float4 per lane.  The per-row sums S_i.k and S_i.q are in-row DPP
// all-reductions, so every lane of a row ends with u_i, w_i, coef_i and o_i and
// updates its own columns directly.
#pragma once

#include "gdn_device.h"

namespace gdn {

template <typename T, int N>
struct VecT {
    typedef T type __attribute__((ext_vector_type(N)));
};

// VPL: state values per lane the workgroup size aims at (the workgroup has
// D*ROWS/VPL threads, clamped to [64, 1024]); fewer values per lane mean more
// waves per tile and fewer registers per wave.  ROWS: rows of the tile one
// workgroup holds (all D, or a slice of a tile split over workgroups).
template <int D, typename ST, int VPL = 64, int ROWS = D>
struct DecodeTile {
    static constexpr int kMaxVec = 16 / (int)sizeof(ST);
    static constexpr int VEC = kMaxVec < D ? kMaxVec : D;     // state elements per vector access
    static constexpr int LPR = (D / VEC) < 16 ? D / VEC : 16; // lanes per row
    static constexpr int NCH = D / (LPR * VEC);               // vectors per lane per row
    static constexpr int C = NCH * VEC;                       // columns per lane
    static constexpr int NT_RAW = D * ROWS / VPL;
    static constexpr int NT = NT_RAW < 64 ? 64 : (NT_RAW > 1024 ? 1024 : NT_RAW);
    static constexpr int NG = NT / LPR;                       // row groups
    static constexpr int RPL = (ROWS / NG) < 1 ? 1 : ROWS / NG;     // rows per lane
    static constexpr int NGA = ROWS / RPL;                       // row groups holding rows
    static_assert(VEC % 4 == 0, "q/k are read as float4");
    static_assert(RPL <= LPR, "one output row per lane");
    static_assert(NGA <= NG, "rows fit the workgroup");
    static_assert(D % ROWS == 0, "whole slices");
};

// The state tile's 16-byte accesses go through a buffer descriptor over the
// head's slot, which carries an explicit cache policy (the CPol bits of a
// gfx950 buffer instruction: sc0 = 1, nt = 2, sc1 = 16).  The tile is read
// once and written once per call: the loads stream (nt), and the stores
// stream and write through at device scope (sc0 sc1 nt).  Against nt stores
// that took the B=64 fp32 decode from 67.8 to 67.1 us and the B=256 binary16
// decode from 123.8 to 122.1 us; loads with the same bits, or buffer
// instructions with nt alone, changed nothing.
constexpr int kTileLoadPolicy = 2;
constexpr int kTileStorePolicy = 19;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void *slot, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(slot), (short)0, bytes, 0x00020000);
}
template <typename V>
__device__ __forceinline__ V load_tile_vec(__amdgpu_buffer_rsrc_t r, int byte_off) {
    static_assert(sizeof(V) == 16, "16-byte vectors");
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kTileLoadPolicy));
}
template <typename V, int POLICY = kTileStorePolicy>
__device__ __forceinline__ void store_tile_vec(__amdgpu_buffer_rsrc_t r, int byte_off, const V &x) {
    static_assert(sizeof(V) == 16, "16-byte vectors");
    typedef unsigned U __attribute__((ext_vector_type(4)));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(U, x), r, byte_off, 0, POLICY);
}

// Non-temporal store of a state vector (8 or 16 bytes).  The vector goes out as
// 32-bit words: hipcc drops the non-temporal hint of the decode's store of a
// vector of binary16 values (it emits a plain store), but keeps it on words.
template <typename V>
__device__ __forceinline__ void store_state_nt(const V &x, V *p) {
    typedef uint32_t U __attribute__((ext_vector_type(sizeof(V) / 4)));
    static_assert(sizeof(V) % 4 == 0 && sizeof(V) == sizeof(U), "whole 32-bit words");
    __builtin_nontemporal_store(__builtin_bit_cast(U, x), reinterpret_cast<U *>(p));
}

// Sum over a whole wave of per-row-group values, where the LPR lanes of each
// group hold the same value: a butterfly over lane distances LPR, 2 LPR, ..., 32
// (ds_bpermute).  Every lane ends with the same bits (each step adds a pair in
// either order, and IEEE addition commutes), so the result is deterministic.
// Call with the whole wave active.
template <int LPR>
__device__ __forceinline__ float wave_groups_sum(float x) {
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace gdn
