// pa_layout.h -- LDS tile layouts shared by the attention kernels and the
// passes that pre-build tiles in that layout (host and device).
//
// A KV tile holds 64 consecutive key positions of one (request, KV head).
//
// K tile (bf16, or int8 for the int8-QK arm): row-major [64][D]; the 16-byte
// chunk c of row r is stored at chunk c ^ (r & kswz), kswz = min(chunks, 16) - 1,
// so that 16 consecutive rows read at the same logical chunk hit 16 distinct
// chunk slots (64 LDS banks).
//
// V^T tile (fp16): [D][64]; within each group of 16 keys, keys {0-3, 8-11}
// take slots 0-7 and {4-7, 12-15} take slots 8-15 (the key order in which
// the S accumulator rows reach the PV MFMA), and the 16-byte chunk c of row d
// is stored at c ^ ((d ^ (d >> 3)) & 7).
//
// Tile images in global memory (the workspace) are byte-for-byte copies of
// these LDS tiles, followed by 64 fp32 per-key scales, so a workgroup moves a
// tile with straight 1 KB direct-to-LDS copies.
#pragma once
#include <stdint.h>

namespace pa {

constexpr int TILE_KEYS = 64;

__host__ __device__ constexpr int ktile_swz_mask(int row_bytes) {
    return (row_bytes / 16 < 16 ? row_bytes / 16 : 16) - 1;
}

// bytes of one tile image (tile + 64 fp32 scales)
__host__ __device__ constexpr int64_t image_bytes(int head_dim) {
    return (int64_t)TILE_KEYS * head_dim * 2 + TILE_KEYS * 4;
}

__host__ __device__ inline int64_t tiles_per_request(int32_t max_ctx_len) {
    return ((int64_t)max_ctx_len + TILE_KEYS - 1) / TILE_KEYS;
}

// slot of key k (0..63) in a row of the V^T tile
__host__ __device__ inline int vt_slot(int k) {
    const int k16 = k & 15;
    return (k & ~15) | (k16 & 3) | ((k16 >> 3) << 2) | (((k16 >> 2) & 1) << 3);
}
__host__ __device__ inline int vt_swz(int d) { return (d ^ (d >> 3)) & 7; }
// byte offset of (d, slot) in a [D][64] fp16 V^T tile (8 chunks of 16 B per row)
__host__ __device__ inline int vt_off(int d, int slot) {
    return d * (TILE_KEYS * 2) + ((((slot >> 3) ^ vt_swz(d)) << 4) | ((slot & 7) << 1));
}

}  // namespace pa
