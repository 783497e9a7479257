// Key record layout for head_dim a multiple of 64 and proj_dim a multiple of
// 32 (layout v2; device helpers of the general-shape kernels).
//
// A head_dim d = 128 n + 64 has n full 128-coordinate chunks and one half
// chunk; a proj_dim m = 64 n' + 32 has n' full 64-projection blocks and one
// half block.  Full chunks and blocks are stored as for d % 128 == 0 and
// m % 64 == 0.  The half parts:
//  * codes: coordinate 128 n + 16 t + 4 q + i (t = 0..3, lane group
//    q = 0..3, i = 0..3) is held, in the matrix-core lane order, by lane
//    group q at slot t; lane groups q and q + 2 share the code group
//    (q % 2) at words b (4 n + q % 2) .. + b - 1, q in slots 0..3 and q + 2
//    in slots 4..7.  (The full groups take words 0 .. 4 n b - 1.)
//  * signs: one word after the full blocks' 2 n' words, projection
//    64 n' + j at bit j.
// A lane group's half group is brought to slots 0..3 by lower_half (the
// readers) and placed from slots 0..3 into 4..7 by lift_half (the writers).
#pragma once

#include <stdint.h>

namespace tq {

// Chunks of 128 coordinates, the last one possibly a half chunk.
__host__ __device__ __forceinline__ int key_chunks(int d) { return (d + 127) / 128; }
__host__ __device__ __forceinline__ int key_full_chunks(int d) { return d / 128; }
// 64-projection blocks, the last one possibly a half block.
__host__ __device__ __forceinline__ int sign_blocks(int m) { return (m + 63) / 64; }

// First word of the code group that lane group q reads for chunk c, and the
// slot at which its codes start there (0, or 4 in a half chunk's upper half).
__host__ __device__ __forceinline__ int key_group_word(int q, int c, int n_full, int b) {
  return c < n_full ? b * (q * n_full + c) : b * (4 * n_full + (q & 1));
}
__host__ __device__ __forceinline__ int key_group_slot0(int q, int c, int n_full) {
  return c < n_full ? 0 : 4 * (q >> 1);
}

// Slots 4..7 of a b-bit code group moved to slots 0..3 (what ends up in
// slots 4..7 is not specified).  Slot layout of a group: b = 1 bit s of
// each byte; b = 2 word s/4; b = 4 word s/2; b = 3 slots 0..5 in word s/2
// at bit 3 (s % 2), slot 6 (7) with its two low bits at bits 6..7 of word
// 0 (1) and its high bit at bit 6 (7) of word 2.
template <int B>
__device__ __forceinline__ void lower_half(uint32_t (&w)[B]) {
  if constexpr (B == 1) {
    w[0] >>= 4;
  } else if constexpr (B == 2) {
    w[0] = w[1];
  } else if constexpr (B == 4) {
    w[0] = w[2];
    w[1] = w[3];
  } else if constexpr (B == 3) {
    const uint32_t s67 = ((w[0] >> 6) & 0x03030303u) | ((w[2] >> 4) & 0x04040404u) |
                         ((w[1] >> 3) & 0x18181818u) | ((w[2] >> 2) & 0x20202020u);
    w[0] = w[2] & 0x3F3F3F3Fu;
    w[1] = s67;
  }
}

// The inverse placement: codes in slots 0..3 (and nothing else) moved to
// slots 4..7, slots 0..3 left empty.
template <int B>
__device__ __forceinline__ void lift_half(uint32_t (&w)[B]) {
  if constexpr (B == 1) {
    w[0] <<= 4;
  } else if constexpr (B == 2) {
    w[1] = w[0];
    w[0] = 0u;
  } else if constexpr (B == 4) {
    w[2] = w[0];
    w[3] = w[1];
    w[0] = w[1] = 0u;
  } else if constexpr (B == 3) {
    const uint32_t a = w[0], b = w[1];
    w[0] = (b & 0x03030303u) << 6;
    w[1] = (b & 0x18181818u) << 3;
    w[2] = (a & 0x3F3F3F3Fu) | ((b & 0x04040404u) << 4) | ((b & 0x20202020u) << 2);
  }
}

// Runtime-bit-width forms (small kernels and reconstruction).
// Word offset (from the record start) and slot of coordinate j's code.
__host__ __device__ __forceinline__ void key_code_place(int j, int d, int b, int& word, int& slot) {
  const int n_full = d / 128, g = j >> 7, jj = j & 127, q = (jj >> 2) & 3, t = jj >> 4;
  word = key_group_word(q, g, n_full, b);
  slot = t + key_group_slot0(q, g, n_full);
}

// Sign word (from the first sign word) and bit of projection j.
__host__ __device__ __forceinline__ void sign_place(int j, int m, int& word, int& bit) {
  const int nfull = m / 64;
  if (j >= 64 * nfull) {
    word = 2 * nfull;
    bit = j - 64 * nfull;
    return;
  }
  const int t = j >> 4, q = (j >> 2) & 3, i = j & 3;
  word = 2 * (t / 4) + q / 2;
  bit = 16 * (q % 2) + 4 * (t % 4) + i;
}

}  // namespace tq
