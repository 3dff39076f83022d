// Q4_0 block access shared by the Q4_0 kernels (gfx950).
//
// Minueza-32M -> KMCU v1 page, section 2: an 18-byte block is the fp16 scale
// d (little-endian) followed by 16 bytes of 4-bit codes, byte k holding
// elements 2k (low nibble) and 2k+1 (high nibble); section 3: rows are padded
// to whole blocks, so blocks sit at 2-byte-aligned offsets.
#pragma once
#include "bqm_common.h"

namespace bqm {

constexpr int kQ4Block = 32;
constexpr int kQ4BlockBytes = 18;
constexpr uint32_t kQ4OOB = 0x80000000u;   // buffer offset past every range: reads give 0

__device__ __forceinline__ __amdgpu_buffer_rsrc_t q4_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// One lane's block: the 16 bytes from the 4-byte-aligned address below it and
// the next 4 (2 for a block that ends the buffer); ok == false reads zeros.
struct BlockLoad {
  uint4 v;
  uint32_t v4, sh;
};

__device__ __forceinline__ BlockLoad load_block(__amdgpu_buffer_rsrc_t rw, bool ok, uint32_t off,
                                                uint32_t total) {
  BlockLoad L;
  const uint32_t a4 = off & ~3u;
  L.sh = ok ? (off & 3u) : 0u;                     // 0 or 2: blocks are 2-byte aligned
  L.v = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rw, ok ? a4 : kQ4OOB, 0, 0));
  const bool w4 = ok && a4 + 20 <= total;          // the 4 bytes after exist
  const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b32(rw, w4 ? a4 + 16 : kQ4OOB, 0, 0);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rw, (ok && !w4) ? a4 + 16 : kQ4OOB, 0, 0);
  L.v4 = lo | hi;
  return L;
}

// The scale and the 16 nibble bytes of a loaded block, realigned (blocks
// are 2-byte aligned): byte k of nib[w] holds elements 8w + 2k (low nibble)
// and 8w + 2k + 1 (high nibble).
__device__ __forceinline__ float block_fields(const BlockLoad &L, uint32_t (&nib)[4]) {
  uint32_t w0, w1, w2, w3, w4;
  if (L.sh == 0) {
    w0 = L.v.x; w1 = L.v.y; w2 = L.v.z; w3 = L.v.w; w4 = L.v4;
  } else {
    w0 = __builtin_amdgcn_alignbyte(L.v.y, L.v.x, 2);
    w1 = __builtin_amdgcn_alignbyte(L.v.z, L.v.y, 2);
    w2 = __builtin_amdgcn_alignbyte(L.v.w, L.v.z, 2);
    w3 = __builtin_amdgcn_alignbyte(L.v4, L.v.w, 2);
    w4 = L.v4 >> 16;
  }
  nib[0] = __builtin_amdgcn_alignbyte(w1, w0, 2);
  nib[1] = __builtin_amdgcn_alignbyte(w2, w1, 2);
  nib[2] = __builtin_amdgcn_alignbyte(w3, w2, 2);
  nib[3] = __builtin_amdgcn_alignbyte(w4, w3, 2);
  return half_bits_to_float((uint16_t)(w0 & 0xFFFFu));
}

}  // namespace bqm
