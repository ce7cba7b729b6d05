// pa_layout.h -- LDS tile layouts shared by the attention kernels and the
// passes that pre-build tiles in that layout (host and device).
//
// A KV tile holds 64 consecutive key positions of one (request, KV head).
//
// K tile (bf16 codes/values, or int8 for the int8-QK arm), rows of R bytes.
// It arrives as 64 / rpi direct copies of 1 KB (rpi = 1024 / R consecutive
// keys each, so each copy reads from one cache block); copy q lands at LDS
// byte q * 1040, i.e. 16 bytes of padding per KB: consecutive copies start 4
// banks apart.  The MFMA's 32-row A operand does not take the keys in order:
// row i of key block kb holds key tile_key(32 kb + i), chosen so that the 16
// lanes of one LDS read phase hit 16 different 4-bank groups and every operand
// read of a lane is its own base plus a compile-time offset.
//
// V^T tile (fp16): [D][64] (128-byte rows, no padding).  Its 64 columns
// follow the MFMA positions of the K tile (column of position p holds key
// tile_key(p)), with positions {0-3, 8-11} of each group of 16 in columns 0-7
// and {4-7, 12-15} in columns 8-15: the order in which the S accumulator rows
// reach the PV MFMA, so each PV operand is one 16-byte read.  The eight
// 16-byte chunks of row d are stored permuted, chunk c at c ^ vt_chunk_swz(d):
// a PV operand read takes one chunk from each of 32 consecutive rows (two
// chunks c, c ^ 1 per row over the wave), and rows a multiple of 128 bytes
// apart would otherwise share their banks.  The permutation gives the 16
// rows of a 16-lane read phase 16 different 4-bank groups, and also the 8
// rows x 2 chunks of a phase that pairs lanes l and l + 32.
//
// fp16 tops out at 65504, so a tile holds V * 2^-e: e >= 0 is the smallest
// power of two that brings the tile's largest |V| below 2^15 (0 for any tile
// whose values are all below 2^15 in magnitude, or that holds an infinity;
// NaNs take no part in the maximum).
//
// V^T images in global memory (the workspace) are byte-for-byte copies of the
// LDS tile, followed by 64 fp32 per-key scales in position order (int8 V)
// and a 16-byte word whose first fp32 is the tile's factor 2^e (read by the
// attention kernel from memory, only where some tile of its key range has e >
// 0), so a workgroup moves the tile with straight 1 KB direct-to-LDS copies.
// K images (int8-KV exact arm) hold [64][D] bf16 codes in key order (the 1 KB
// copies re-space them) followed by 64 fp32 per-key scales in key order.
#pragma once
#include <stdint.h>

namespace pa {

constexpr int TILE_KEYS = 64;
constexpr int VT_ROW_BYTES = TILE_KEYS * 2;        // one V^T row (fp16)

constexpr int K_COPY_STRIDE = 1024 + 16;          // LDS bytes per 1 KB K copy
constexpr int VT_RANGE_LOG2 = 15;                 // a tile's |V| * 2^-e stays below 2^15

// e of a V^T tile whose largest magnitude is amax (see above): from amax's
// exponent field, amax < 2^(field - 126); 0 for an infinite amax
__host__ __device__ inline int vt_range_exp(uint32_t amax_bits) {
    const int field = (int)((amax_bits >> 23) & 0xff);
    const int e = field - 126 - VT_RANGE_LOG2;
    return (field == 0xff || e < 0) ? 0 : e;
}

// key (0..63) held at MFMA position p = 32 * kb + i of a K tile whose rows are
// copied rpi at a time (rpi in {2, 4, 8, 16})
__host__ __device__ constexpr int tile_key(int p, int rpi) {
    const int g = 64 / rpi, kb = p >> 5, i = p & 31;
    return rpi * (i % g) + i / g + (32 / g) * kb;
}

// bytes of one V^T tile in LDS and of one V^T image (tile + 64 fp32 scales +
// the factor word); the factor's byte offset in an image
__host__ __device__ constexpr int vt_tile_bytes(int head_dim) { return head_dim * VT_ROW_BYTES; }
__host__ __device__ constexpr int64_t v_image_bytes(int head_dim) {
    return (int64_t)vt_tile_bytes(head_dim) + TILE_KEYS * 4 + 16;
}
__host__ __device__ constexpr int vt_factor_off(int head_dim) { return vt_tile_bytes(head_dim) + TILE_KEYS * 4; }
// stored position of 16-byte chunk c of V^T row d is c ^ vt_chunk_swz(d)
__host__ __device__ constexpr int vt_chunk_swz(int d) { return 2 * ((d >> 1) & 3) + ((d >> 3) & 1); }
// bytes of one K image (int8-KV exact arm): 64 rows of bf16 codes + 64 scales
__host__ __device__ constexpr int64_t k_image_bytes(int head_dim) {
    return (int64_t)TILE_KEYS * head_dim * 2 + TILE_KEYS * 4;
}

__host__ __device__ inline int64_t tiles_per_request(int32_t max_ctx_len) {
    return ((int64_t)max_ctx_len + TILE_KEYS - 1) / TILE_KEYS;
}

// column of MFMA position p (0..63) in a row of the V^T tile, before the row's chunk
// permutation (swaps bits 2 and 3)
__host__ __device__ inline int vt_slot(int p) {
    const int k16 = p & 15;
    return (p & ~15) | (k16 & 3) | ((k16 >> 3) << 2) | (((k16 >> 2) & 1) << 3);
}

}  // namespace pa
