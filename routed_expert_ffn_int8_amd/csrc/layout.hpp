// Device layout of the 4-bit affine weights.
//
// The pages locate an expert inside a stacked tensor at a fixed per-expert
// stride (BigMoeOnEdge, section "from the real routing to the GGUF weight
// slice": slice offset = tensor start + expert id x stride) and repack
// weights into a compute-friendly layout at install/load time (Rockchip-NPU
// plan §2.2 streaming repack; BigMoeOnEdge, section "how it differs from mmap
// and repack").  Here each expert is one contiguous blob at a fixed stride,
// so an HBM cache slot is exactly one blob and a fill is one copy.
//
// A matrix with R rows and C columns (G = C/64 groups) is stored as
//   Q  region: [R/8 row blocks][G groups][2 halves][8 rows][16 bytes]
//              (16 bytes = the 4 packed words of 32 consecutive columns of
//              one row, unchanged nibble order), 256 bytes per (block, group)
//   SB region: [R/8 row blocks][G groups][8 rows] uint32 = fp16 scale | fp16 bias << 16
// so a wavefront that reads 8 rows x 16 bytes touches one 128-byte line, and
// the scale/bias words of 8 rows of one group are 32 contiguous bytes.
#pragma once
#include <cstddef>
#include <cstdint>

namespace moe {

constexpr int kRowBlock = 8;
constexpr int kGroup = 64;

inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

struct MatLayout {
  int rows = 0, cols = 0;
  size_t q_off = 0, sb_off = 0, bytes = 0;  // offsets inside the blob
};

struct BlobLayout {  // one expert: gate, up (rows f, cols d), down (rows d, cols f)
  MatLayout gate, up, down;
  size_t stride = 0;  // bytes per expert blob (256-aligned)
};

inline BlobLayout make_blob_layout(int d, int f) {
  BlobLayout L;
  size_t off = 0;
  auto place = [&](MatLayout& m, int rows, int cols) {
    m.rows = rows;
    m.cols = cols;
    m.q_off = off;
    off = align256(off + (size_t)rows * cols / 2);
    m.sb_off = off;
    off = align256(off + (size_t)rows * (cols / kGroup) * 4);
    m.bytes = (size_t)rows * cols / 2 + (size_t)rows * (cols / kGroup) * 4;
  };
  place(L.gate, f, d);
  place(L.up, f, d);
  place(L.down, d, f);
  L.stride = off;
  return L;
}

// Repack one canonical matrix (q [R][C/8] words, s/b [R][C/64] fp16 bits)
// into `blob` at the offsets of `m`.
void pack_matrix(const MatLayout& m, const uint32_t* q, const uint16_t* s, const uint16_t* b, uint8_t* blob);

}  // namespace moe
