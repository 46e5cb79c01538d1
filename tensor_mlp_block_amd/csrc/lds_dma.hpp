// lds_dma.hpp -- direct global -> LDS loads for gfx950 and the workgroup -> tile mapping shared
// by the MFMA GEMMs.
//
// `buffer_load_dwordx4 ... lds` moves 64 x 16 bytes per wave instruction straight into a
// contiguous 1 KB of LDS: lane l's 16 bytes land at M0 + 16 l, with no register round trip.
// The LDS side of a load is fixed by the lane number, so any layout change (swizzle) is applied
// on the global side, by choosing which 16-byte chunk each lane fetches. A lane whose offset is
// past the buffer resource's range gets zeros from the hardware range check, so ragged tiles
// need no branches.
#pragma once

#include "common.hpp"

namespace mlptp {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
#define MLPTP_LDS __attribute__((address_space(3)))

extern "C" __device__ void llvm_amdgcn_raw_buffer_load_lds(i32x4 rsrc, MLPTP_LDS uint32_t* lds,
                                                           int size, int voffset, int soffset,
                                                           int offset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.lds");

// Buffer resource over [base, base + 2 GiB): offsets >= 0x80000000 are out of range and load
// zeros. Word 3 is the gfx9-family default (32-bit dword format, no swizzle).
__device__ __forceinline__ i32x4 make_buffer_rsrc(const void* base)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a & 0xffffffffu));
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)((a >> 32) & 0xffffu));
    r[2] = (int)0x80000000u;
    r[3] = 0x00020000;
    return r;
}

// Per-lane offset that loads nothing (out of range whether or not the hardware adds the scalar
// offset before its range check).
constexpr int kOutOfRange = (int)0x80000000u;

// Workgroup id -> output tile. Consecutive ids are dealt round-robin over the 8 XCDs (each with
// its own L2), so when the tile count is a multiple of 8 the remap gives each XCD a contiguous
// range of tiles; within the range, GROUP_M row-tiles are walked together so the A rows and B
// columns a group shares stay in that XCD's L2.
template <int GROUP_M>
__device__ __forceinline__ void tile_coords(int64_t bid, int64_t tiles_m, int64_t tiles_n,
                                            int64_t& tm, int64_t& tn)
{
    const int64_t ntiles = tiles_m * tiles_n;
    constexpr int kXcds = 8;
    if (ntiles % kXcds == 0) bid = (bid % kXcds) * (ntiles / kXcds) + bid / kXcds;
    const int64_t per_group = (int64_t)GROUP_M * tiles_n;
    const int64_t group = bid / per_group;
    const int64_t first_m = group * GROUP_M;
    const int64_t gm = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
    const int64_t in_group = bid % per_group;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// s_waitcnt vmcnt(CNT) with the other counters left alone (gfx9 encoding: vmcnt[3:0],
// expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits [15:14]).
template <int CNT>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(CNT >= 0 && CNT < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((CNT & 15) | (7 << 4) | (15 << 8) | ((CNT >> 4) << 14));
}

__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

}  // namespace mlptp
