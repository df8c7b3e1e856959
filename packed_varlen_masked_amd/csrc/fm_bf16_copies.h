// How the bf16 attention kernel spreads the copies (global -> LDS) of its
// K and V tiles over its waves.  Shared by the kernel and by the host-side
// self check (fm_self_check), so that the table every copy address comes
// from can be verified without a GPU.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {
namespace bf16c {

constexpr int BC = 64;                      // key rows per tile
constexpr int GW = 4;                       // waves per group (group 0 copies K, group 1 copies V)
constexpr int KCH = 17, VCH = 20;           // 16-byte chunks per LDS row (K, V; 16 carry data)
constexpr int KBLK = BC * KCH * 16 / 1024;  // 1 KB blocks of data per K tile: 17
constexpr int VBLK = BC * VCH * 16 / 1024;  // per V tile: 20
constexpr int SLOT_BLK = 20;                // 1 KB blocks per ring slot (K slots end in 3 spare blocks)
constexpr int NCOPY = SLOT_BLK / GW;        // block copies per wave per tile: 5

// Copy i (0..4) of wave t (0..3) of its group fills block t + 4i of the slot.
__host__ __device__ constexpr int copy_block(int t, int i) { return t + GW * i; }

// Lane `lane` of the copy of block `blk` of a tile with CH chunks per LDS
// row: row | (byte offset in the source row << 8).  Chunks >= 16 are row
// padding and read chunk 0 of their row; blocks past the tile's data (the
// spare blocks of a K slot) repeat block blk - nblk, so that every lane
// reads a row inside the tile.
__host__ __device__ constexpr uint32_t copy_slot(int CH, int nblk, int blk, int lane) {
    return (uint32_t)((64 * (blk < nblk ? blk : blk - nblk) + lane) / CH) |
           ((uint32_t)((64 * (blk < nblk ? blk : blk - nblk) + lane) % CH < 16
                           ? 16 * ((64 * (blk < nblk ? blk : blk - nblk) + lane) % CH) : 0) << 8);
}

// Source pattern of copy i of wave t of group g.
__host__ __device__ constexpr uint32_t copy_lane(int g, int t, int i, int lane) {
    return g == 0 ? copy_slot(KCH, KBLK, copy_block(t, i), lane) : copy_slot(VCH, VBLK, copy_block(t, i), lane);
}

}  // namespace bf16c
}  // namespace fm
